"""CPU oracle for absorbed-latent MLA decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
executes it, and this package imports nothing from the product path: the two
share only the seeded input generators in ``mla_synth``.

Everything here is plain, slow and meant to be checked by eye against the
pages it follows.  Floating point is float64 unless a step is defined in
another precision (the quantisers are defined in IEEE float32, bit for bit).

Sources (cited by key in every module):
  [Audit]    "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界"
             (DeepSeek MLA absorbed cache: real-weight execution and the
             FlashMLA architecture boundary)
  [Report]   "DeepSeek-V2-Lite MLA 吸收式 KV 缓存优化 — 完整实验报告"
             (DeepSeek-V2-Lite absorbed MLA KV-cache optimisation report)
  [Tutorial] "手搓 MLA:从 MHA 到 weight absorption,看懂 DeepSeek 的 KV 压缩"
             (Hand-rolled MLA: from MHA to weight absorption)
  [Budget]   "kv_budget.py" from the TileLang tutorial chapter
             "算子实战 IV：MoE 与 MLA" (parts A, B, C)

Parity status of each function is stated in its module header.
"""
from .mla_ref import (  # noqa: F401
    bf16_to_f64, softmax_scale, absorb_q, unabsorbed_decode, absorbed_decode,
    latent_attention, latent_attention_range, lse_combine, out_proj, wo_proj,
    gather_seq, decode_paged, plan_token_ranges,
)
from .quant import (  # noqa: F401
    quant_int8_sym, quant_int4_asym, dequant_int8, dequant_int4,
    page_bytes, token_bytes, pack_page, unpack_page, pack_pool, dequant_pool_seq,
)
from .accounting import (  # noqa: F401
    naive_cache_bytes, absorbed_cache_bytes, per_token_elements, decode_ai,
    heads_to_cross_ridge, tilelang_register_budget, tilelang_smem_sum,
)
from .layer import rmsnorm, rope_interleaved, layer_front, layer_decode  # noqa: F401

"""Absorbed-latent MLA decode for AMD MI355X (gfx950).

A thin Python face of the C ABI in include/mla.h: every function here only
marshals arguments (torch tensors -> device pointers, the current HIP stream)
and checks the returned status.  All arithmetic runs in the HIP kernels of
libmla_absorbed_latent.so; there is no CPU fallback.

The five steps of one decode, in order:
    cache_append   -> write the new tokens' latent rows (quantising if asked)
    absorb_q       -> fold W_UK into each query head (fp16 q_abs, width 576)
    decode_attn    -> split-KV attention over the shared latent (partials)
    decode_combine -> log-sum-exp merge of the partials (o_lat, lse)
    out_proj       -> expand through W_UV (and optionally W_O)
plus the host-side planner plan_splits, and decode_combine_out_proj, which
runs the last two in one pass.  layer_front produces the inputs of the first
two steps from a layer's hidden states (projections, RMSNorm, RoPE), and
prefill_attn runs a prompt chunk's causal attention in the unabsorbed form.
"""
from .api import (  # noqa: F401
    MlaError, Config, config, cache_bytes_per_token, cache_page_bytes, decode_workspace_bytes,
    plan_splits, cache_append, absorb_q, append_absorb_q, decode_attn, decode_combine, out_proj, decode_combine_out_proj, status_string,
    layer_front, layer_front_workspace_bytes, prefill_attn, prefill_workspace_bytes,
    out_residual,
    CACHE_BF16, CACHE_INT8, CACHE_INT4, CACHE_INT4_SYM, CACHE_INT8_TOK, CACHE_FP8_TOK, CACHE_INT4_SYM_K4,
)

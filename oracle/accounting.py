"""Oracle: cache byte accounting and decode arithmetic intensity.  Test
infrastructure only.

Each formula is the plain definition; the tests pin them to the integers the
pages print (tests/golden/page_figures.json, each entry with its citation).

  naive (expanded) cache  : per token and layer, H heads x (k_nope + k_rope)
                            key elements plus H x v_head value elements
                            ([Audit] §2.1 and §4.1)
  absorbed cache          : per token and layer, latent + RoPE key elements
                            ([Audit] §2.4; [Tutorial] §三 and §五)
  decode AI (MHA / GQA)   : 2 H_q / (H_kv b)             ([Budget] part B)
  decode AI (MLA)         : 2 H_q (2 d_c + d_r) / (b (d_c + d_r))   ([Budget] part B)
  register / shared-memory budget of the TileLang decode tile ([Budget] part C)

Parity: pinned (exact integers and the rationals the pages print).
"""
from __future__ import annotations


def naive_cache_bytes(tokens: int, heads: int = 16, k_nope: int = 128, k_rope: int = 64,
                      v_head: int = 128, elem_bytes: int = 2) -> int:
    """Expanded per-head K [tokens, H, k_nope + k_rope] plus V [tokens, H, v_head]."""
    return tokens * heads * (k_nope + k_rope) * elem_bytes + tokens * heads * v_head * elem_bytes


def absorbed_cache_bytes(tokens: int, d_c: int = 512, d_r: int = 64, elem_bytes: int = 2) -> int:
    """Latent [tokens, d_c] plus shared RoPE key [tokens, d_r]."""
    return tokens * d_c * elem_bytes + tokens * d_r * elem_bytes


def per_token_elements(kind: str, heads: int = 128, head_dim: int = 128, kv_heads: int = 8,
                       d_c: int = 512, d_r: int = 64) -> int:
    """Cached elements per token per layer for the attention families compared in
    [Tutorial] §五 (K and V each head_dim wide for MHA/GQA/MQA)."""
    if kind == "mha":
        return 2 * heads * head_dim
    if kind == "gqa":
        return 2 * kv_heads * head_dim
    if kind == "mqa":
        return 2 * 1 * head_dim
    if kind == "mla":
        return d_c + d_r
    raise ValueError(kind)


def decode_ai(kind: str, heads_q: int, heads_kv: int = 1, d_c: int = 512, d_r: int = 64,
              elem_bytes: int = 2) -> float:
    """FLOP per byte of cache read for one decode token ([Budget] part B)."""
    if kind == "mla":
        return 2.0 * heads_q * (2 * d_c + d_r) / (elem_bytes * (d_c + d_r))
    return 2.0 * heads_q / (heads_kv * elem_bytes)


def heads_to_cross_ridge(balance_flop_per_byte: float, d_c: int = 512, d_r: int = 64,
                         elem_bytes: int = 2) -> float:
    """Query heads at which MLA decode AI equals a machine balance point."""
    return balance_flop_per_byte * elem_bytes * (d_c + d_r) / (2.0 * (2 * d_c + d_r))


def tilelang_register_budget(block_h: int = 64, block_n: int = 64, d_c: int = 512,
                             threads: int = 256):
    """fp32 accumulators acc_o [block_h, d_c] and acc_s [block_h, block_n], spread
    over the thread block: (acc_o regs, acc_s regs, total) per thread."""
    acc_o = block_h * d_c / threads
    acc_s = block_h * block_n / threads
    return acc_o, acc_s, acc_o + acc_s


def tilelang_smem_sum(block_h: int = 64, block_n: int = 64, d_c: int = 512, d_r: int = 64,
                      stages: int = 2, elem_bytes: int = 2) -> int:
    """Sum of the decode tile's shared buffers (Q, Q_pe, S, KV x stages,
    K_pe x stages, O): an upper bound on shared memory, in bytes."""
    q = block_h * d_c * elem_bytes
    q_pe = block_h * d_r * elem_bytes
    s = block_h * block_n * elem_bytes
    kv = block_n * d_c * elem_bytes * stages
    k_pe = block_n * d_r * elem_bytes * stages
    o = block_h * d_c * elem_bytes
    return q + q_pe + s + kv + k_pe + o

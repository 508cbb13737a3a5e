"""Oracle: the two forms of MLA decode attention, split-KV partials and the
log-sum-exp merge.  Test infrastructure only (see the package header).

Notation (one decode query per sequence):
  c_t   in R^512   cached latent of token t          ("c_kv")
  r_t   in R^64    cached decoupled RoPE key           ("k_pe")
  qN_h  in R^128   query, no-RoPE part, head h         ("q_nope")
  qR_h  in R^64    query, RoPE part, head h            ("q_pe")
  W_UK[h], W_UV[h] in R^{128 x 512}, index order "hdc" ([Tutorial] §四 einsums)
  sigma = 1 / sqrt(128 + 64)

Parity pins (tests/test_oracle_pins.py):
  * unabsorbed_decode  -- pinned to torch's scaled_dot_product_attention on
    explicitly expanded K/V (a library routine), and to pure-Python loops on
    tiny inputs.
  * absorbed_decode    -- pinned to unabsorbed_decode by the associativity
    identity of [Audit] §2.2/§2.3 (fp64 agreement at round-off scale, as
    [Tutorial] §四 reports), plus closed forms (one token, zero query,
    identical rows, permutation invariance).
  * latent_attention_range / lse_combine -- pinned by "k random splits merge to
    the unsplit result" and by the closed form of a single split.
  * decode_paged / gather_seq -- pinned by "any page permutation gives the
    contiguous result".
  * out_proj / absorb_q -- pinned through absorbed == unabsorbed (they are the
    two matrix products the identity moves).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

BLOCK = 64
D_C = 512
D_R = 64
D_N = 128
D_V = 128


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is float32 with 16 low zero bits)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def softmax_scale(qk_nope: int = D_N, qk_rope: int = D_R) -> float:
    """Score scale 1/sqrt(d_nope + d_rope): the query/key width before absorption."""
    return 1.0 / np.sqrt(qk_nope + qk_rope)


def _softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def _logsumexp(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=axis, keepdims=True))).squeeze(axis)


# --------------------------------------------------------------------------
# Unabsorbed ("naive") path: expand every cached latent into per-head K and V
# [Audit] §2.1 (k_t = W^K c_t, v_t = W^V c_t per head, then ordinary attention);
# [Tutorial] §三 (mla_unabsorbed: concat the no-RoPE key with the shared RoPE key).
# --------------------------------------------------------------------------
def expand_kv(c: np.ndarray, r: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray):
    """c [L,512], r [L,64], W [H,128,512] -> K [H,L,192], V [H,L,128]."""
    H = w_uk.shape[0]
    L = c.shape[0]
    k_nope = np.einsum("hdc,tc->htd", w_uk, c)          # W_UK[h] c_t
    k = np.concatenate([k_nope, np.broadcast_to(r[None], (H, L, r.shape[1]))], axis=-1)
    v = np.einsum("hdc,tc->htd", w_uv, c)               # W_UV[h] c_t
    return k, v


def unabsorbed_decode(q_nope, q_pe, c, r, w_uk, w_uv, scale=None):
    """One query token per head over L cached tokens, unabsorbed.

    q_nope [H,128], q_pe [H,64], c [L,512], r [L,64] (float64)
    returns out [H,128] and lse [H] (natural log of the softmax denominator).
    """
    scale = softmax_scale() if scale is None else scale
    k, v = expand_kv(c, r, w_uk, w_uv)
    q = np.concatenate([q_nope, q_pe], axis=-1)          # [H,192]
    s = scale * np.einsum("hk,htk->ht", q, k)           # [H,L]
    p = _softmax(s)
    out = np.einsum("ht,htd->hd", p, v)
    return out, _logsumexp(s)


# --------------------------------------------------------------------------
# Absorbed path
# [Audit] §2.2: q^T (W^K c) = (W^K^T q)^T c  -> fold W_UK into the query.
# [Audit] §2.3: sum_t p_t W^V c_t = W^V (sum_t p_t c_t) -> aggregate latents first.
# [Audit] §2.4: the RoPE key is position dependent and stays in the cache.
# [Tutorial] §四 (mla_absorbed einsums "thd,hdc->thc" and "thc,hdc->thd").
# --------------------------------------------------------------------------
def absorb_q(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q~[..., h, c] = sum_d q_nope[..., h, d] * W_UK[h, d, c]."""
    return np.einsum("...hd,hdc->...hc", q_nope, w_uk)


def latent_attention(q_lat, q_pe, c, r, scale=None):
    """MQA over the shared latent: head dim 576 for scores, 512 for values.

    q_lat [H,512], q_pe [H,64], c [L,512], r [L,64]
    returns o_lat [H,512] = softmax(s) @ c and lse [H].
    """
    scale = softmax_scale() if scale is None else scale
    s = scale * (q_lat @ c.T + q_pe @ r.T)              # [H,L]
    p = _softmax(s)
    return p @ c, _logsumexp(s)


def out_proj(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """out[..., h, d] = sum_c W_UV[h, d, c] * o_lat[..., h, c]."""
    return np.einsum("...hc,hdc->...hd", o_lat, w_uv)


def wo_proj(out: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """y = W_O . concat_h(out_h): out [..., H, 128], W_O [hidden, H*128]."""
    flat = out.reshape(out.shape[:-2] + (-1,))
    return flat @ w_o.T


def absorbed_decode(q_nope, q_pe, c, r, w_uk, w_uv, scale=None):
    """Absorbed decode of one query token: returns out [H,128], lse [H], o_lat [H,512]."""
    q_lat = absorb_q(q_nope, w_uk)
    o_lat, lse = latent_attention(q_lat, q_pe, c, r, scale)
    return out_proj(o_lat, w_uv), lse, o_lat


def absorbed_decode_f32(q_nope, q_pe, c, r, w_uk, w_uv, scale=None):
    """absorbed_decode with every array in float32 (numpy's BLAS), the form the
    CPU baseline times; the float64 absorbed_decode above is the parity
    reference.  Returns out [H,128] float32."""
    f = np.float32
    scale = f(softmax_scale() if scale is None else scale)
    q_lat = np.einsum("hd,hdc->hc", q_nope.astype(f), w_uk.astype(f))
    s = scale * (q_lat @ c.astype(f, copy=False).T + q_pe.astype(f) @ r.astype(f, copy=False).T)
    p = _softmax(s)
    o_lat = p @ c.astype(f, copy=False)
    return np.einsum("hc,hdc->hd", o_lat, w_uv.astype(f))


# --------------------------------------------------------------------------
# Split-KV partials and their exact merge.  The pages stream history through a
# running max / running sum (the TileLang accumulators of [Budget] part C); the
# split form below applies the same algebra across independent token ranges:
#   m_j = max s, l_j = sum exp(s - m_j), o_j = sum exp(s - m_j) c_t / l_j,
#   lse_j = m_j + ln l_j;  lse = ln sum_j exp(lse_j), o = sum_j exp(lse_j - lse) o_j.
# An empty range has lse_j = -inf and o_j = 0.
# --------------------------------------------------------------------------
def latent_attention_range(q_lat, q_pe, c, r, t0: int, t1: int, scale=None):
    H = q_lat.shape[0]
    if t1 <= t0:
        return np.zeros((H, c.shape[1])), np.full(H, -np.inf)
    return latent_attention(q_lat, q_pe, c[t0:t1], r[t0:t1], scale)


def lse_combine(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Merge (o_j [H,512], lse_j [H]) partials into (o [H,512], lse [H])."""
    lses = np.stack([p[1] for p in parts])              # [J,H]
    os_ = np.stack([p[0] for p in parts])               # [J,H,512]
    m = np.max(lses, axis=0)                            # [H]
    H = lses.shape[1]
    out = np.zeros((H, os_.shape[-1]))
    lse = np.full(H, -np.inf)
    live = np.isfinite(m)
    if live.any():
        w = np.exp(lses[:, live] - m[live])             # [J,h]
        tot = w.sum(axis=0)
        lse[live] = m[live] + np.log(tot)
        out[live] = np.einsum("jh,jhc->hc", w / tot, os_[:, live])
    return out, lse


def plan_token_ranges(L: int, n_splits: int) -> List[Tuple[int, int]]:
    """Cut [0, L) into n_splits contiguous ranges (some may be empty)."""
    edges = np.linspace(0, L, n_splits + 1).round().astype(int)
    return [(int(edges[i]), int(edges[i + 1])) for i in range(n_splits)]


# --------------------------------------------------------------------------
# Paged cache (block table: logical page -> physical page, 64 tokens a page)
# --------------------------------------------------------------------------
def gather_seq(pool_rows: np.ndarray, block_table_row: np.ndarray, L: int) -> np.ndarray:
    """Gather L token rows of one sequence from a pool indexed [page, slot, ...]."""
    rows = []
    for t in range(0, L, BLOCK):
        page = int(block_table_row[t // BLOCK])
        n = min(BLOCK, L - t)
        rows.append(pool_rows[page, :n])
    return np.concatenate(rows, axis=0)


def decode_paged(q_nope, q_pe, w_uk, w_uv, c_pool, r_pool, block_table, seq_lens, scale=None):
    """Absorbed decode of a batch over a paged cache held as float64 pools.

    c_pool [N,64,512], r_pool [N,64,64]; q_nope [B,H,128], q_pe [B,H,64].
    returns out [B,H,128], o_lat [B,H,512], lse [B,H].
    """
    B = q_nope.shape[0]
    H = q_nope.shape[1]
    out = np.zeros((B, H, w_uv.shape[1]))
    o_lat = np.zeros((B, H, w_uv.shape[2]))
    lse = np.zeros((B, H))
    for b in range(B):
        L = int(seq_lens[b])
        c = gather_seq(c_pool, block_table[b], L)
        r = gather_seq(r_pool, block_table[b], L)
        out[b], lse[b], o_lat[b] = absorbed_decode(q_nope[b], q_pe[b], c, r, w_uk, w_uv, scale)
    return out, o_lat, lse

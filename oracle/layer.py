"""Oracle: one V2-Lite MLA layer around the decode hot path.  Test infrastructure
only.

The layer front produces the four tensors the hot path consumes
([Report] §1.1: the joint down projection yields a 512-wide latent and a 64-wide
RoPE key; [Tutorial] §三: the latent is RMS-normalised before caching, the RoPE
key and the query's RoPE part are rotated by position; [Audit] §3.3: V2-Lite has
a single query projection and a joint down projection whose output puts the
latent first).  Readings taken where the pages are silent:
  * RMSNorm: eps 1e-6, unit gain, computed in float64;
  * RoPE: interleaved pairs (x[2i], x[2i+1]) rotated by pos * base^(-2i/64),
    base 10000, positions 0-based, no YaRN rescaling;
  * the four boundary tensors are rounded once to bf16 (the cache is bf16),
    and both decode forms start from those rounded values.

layer_decode then decodes the last position over all positions (the decoded
token attends to itself: the cache holds prefill + 1 token, as in [Audit] §4.1)
and applies the output projection.

Pins (tests/test_layer_oracle.py): RoPE is the identity at position 0,
preserves pair norms, gives scores that depend only on relative position, and
turns pairs 0, 8, 16 and 24 by exactly 1, 0.1, 0.01 and 0.001 rad per position
(the four decades of a 64-wide key with base 10000); RMSNorm of a constant row
is c / sqrt(c^2 + eps); a one-hot hidden state reads back one column of every
projection, which fixes their orientation and the head-major query split.  The
decode part is pinned through mla_ref.
"""
from __future__ import annotations

import numpy as np

from .mla_ref import bf16_to_f64, absorbed_decode, unabsorbed_decode, wo_proj

D_C = 512
D_R = 64
D_N = 128


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 bits (RNE)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def rmsnorm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_interleaved(x: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate pairs (x[..., 2i], x[..., 2i+1]) by angle pos * base^(-2i/d).

    x [T, ..., d] with positions pos [T]."""
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / d)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]          # [T, d/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    cos = np.cos(ang).reshape(shape)
    sin = np.sin(ang).reshape(shape)
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


def layer_front(case):
    """x, W_q, W_DKV -> bf16 bits of q_nope [T,H,128], q_pe [T,H,64], c_kv [T,512], k_pe [T,64]."""
    T, H = case.T, case.H
    x = bf16_to_f64(case.x)
    pos = np.arange(T)
    q = (x @ bf16_to_f64(case.w_q).T).reshape(T, H, D_N + D_R)
    kv = x @ bf16_to_f64(case.w_dkv).T                                  # [T, 576]
    c = rmsnorm(kv[:, :D_C], case.rms_eps)
    k_pe = rope_interleaved(kv[:, D_C:], pos, case.rope_base)
    q_nope = q[..., :D_N]
    q_pe = rope_interleaved(q[..., D_N:], pos, case.rope_base)
    return (_to_bf16_bits(q_nope), _to_bf16_bits(q_pe), _to_bf16_bits(c), _to_bf16_bits(k_pe))


def layer_decode(case, front=None):
    """Decode the last position of the layer both ways.

    returns dict with y_absorbed [hidden], y_unabsorbed [hidden],
    out_absorbed [H,128], out_unabsorbed [H,128], o_lat [H,512], lse [H].
    """
    qn_b, qp_b, c_b, r_b = layer_front(case) if front is None else front
    t = case.T - 1
    qn = bf16_to_f64(qn_b[t])
    qp = bf16_to_f64(qp_b[t])
    c = bf16_to_f64(c_b)
    r = bf16_to_f64(r_b)
    w_uk = bf16_to_f64(case.w_uk)
    w_uv = bf16_to_f64(case.w_uv)
    w_o = bf16_to_f64(case.w_o)
    out_a, lse, o_lat = absorbed_decode(qn, qp, c, r, w_uk, w_uv, case.softmax_scale)
    out_u, _ = unabsorbed_decode(qn, qp, c, r, w_uk, w_uv, case.softmax_scale)
    return {"y_absorbed": wo_proj(out_a, w_o), "y_unabsorbed": wo_proj(out_u, w_o),
            "out_absorbed": out_a, "out_unabsorbed": out_u, "o_lat": o_lat, "lse": lse}

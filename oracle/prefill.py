"""Oracle: chunked prefill attention in the unabsorbed form.  Test
infrastructure only.

[Tutorial] §四: engines run prefill through the unabsorbed path (each head's key
and value are rebuilt from the cached latent: K_h = W_UK[h] c, V_h = W_UV[h] c,
with the shared RoPE key appended to K_h) and decode through the absorbed one;
the two are the same function of the inputs.  [Tutorial] §三 gives the
unabsorbed computation itself (its mla_naive: expand the latent per head, then
ordinary multi-head attention with query/key width 128 + 64 and value width 128).

Reading taken where the pages are silent: a chunk holds the last T of L
positions of one sequence (the first L - T are an already cached prefix), and
query i, at position p = L - T + i, attends to the keys at positions 0..p
(causal; the token attends to itself, as the decoded token does).

Pins (tests/test_oracle_prefill.py): each row equals the decode oracle's
unabsorbed and absorbed results over its causal prefix (mla_ref, pinned on its
own); the first position of a sequence returns its own value vector exactly;
keys after a query's position do not change its row.
"""
from __future__ import annotations

import numpy as np

from .mla_ref import expand_kv, softmax_scale


def prefill_unabsorbed(q_nope, q_pe, c, r, w_uk, w_uv, scale=None):
    """Causal attention of T queries over L >= T cached positions.

    q_nope [T,H,128], q_pe [T,H,64] (queries at positions L-T .. L-1),
    c [L,512], r [L,64], W_UK / W_UV [H,128,512]  (float64)
    returns out [T,H,128] and lse [T,H] (natural log of each softmax denominator).
    """
    scale = softmax_scale() if scale is None else scale
    T, L = q_nope.shape[0], c.shape[0]
    assert 0 < T <= L
    k, v = expand_kv(c, r, w_uk, w_uv)                             # [H,L,192], [H,L,128]
    q = np.concatenate([q_nope, q_pe], axis=-1)                     # [T,H,192]
    s = scale * np.einsum("thk,hlk->htl", q, k)                    # [H,T,L]
    pos = L - T + np.arange(T)
    masked = np.arange(L)[None, :] > pos[:, None]                   # [T,L]: key after the query
    s = np.where(masked[None], -np.inf, s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=-1, keepdims=True)
    out = np.einsum("htl,hld->thd", e / den, v)
    lse = (m + np.log(den))[..., 0].T                               # [T,H]
    return out, lse

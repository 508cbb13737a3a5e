"""Pins of the prefill oracle (oracle/prefill.py), CPU only.

Each row of a chunk is one decode over its causal prefix, so it must equal the
decode oracle's unabsorbed and absorbed results on that prefix (the absorbed
form shares no code with the expansion: [Tutorial] "手搓 MLA:从 MHA 到 weight
absorption,看懂 DeepSeek 的 KV 压缩" §四 states the two forms are the same
function).  Closed form: the first position of a sequence sees only itself, so
its output is its own value vector W_UV[h] c_0 and its lse is its own score.
Causality: keys after a query's position leave its row bit-for-bit unchanged.
"""
import numpy as np
import pytest

from oracle import mla_ref, prefill


def _inputs(T, L, H, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, H, 128)), rng.standard_normal((T, H, 64)),
            rng.standard_normal((L, 512)) * 0.5, rng.standard_normal((L, 64)),
            rng.standard_normal((H, 128, 512)) * 0.05, rng.standard_normal((H, 128, 512)) * 0.05)


@pytest.mark.parametrize("T,L,H", [(7, 7, 4), (5, 19, 2), (1, 9, 3)])
def test_rows_equal_decode_over_the_causal_prefix(T, L, H):
    qn, qp, c, r, wk, wv = _inputs(T, L, H, seed=T * 100 + L)
    scale = 0.07
    out, lse = prefill.prefill_unabsorbed(qn, qp, c, r, wk, wv, scale)
    assert out.shape == (T, H, 128) and lse.shape == (T, H)
    for i in range(T):
        p = L - T + i
        o_u, l_u = mla_ref.unabsorbed_decode(qn[i], qp[i], c[:p + 1], r[:p + 1], wk, wv, scale)
        o_a, l_a, _ = mla_ref.absorbed_decode(qn[i], qp[i], c[:p + 1], r[:p + 1], wk, wv, scale)
        assert np.allclose(out[i], o_u, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[i], l_u, rtol=1e-12, atol=1e-12)
        assert np.allclose(out[i], o_a, rtol=1e-10, atol=1e-12)
        assert np.allclose(lse[i], l_a, rtol=1e-10, atol=1e-12)


def test_first_position_returns_its_own_value():
    qn, qp, c, r, wk, wv = _inputs(3, 3, 2, seed=5)
    scale = 0.1
    out, lse = prefill.prefill_unabsorbed(qn, qp, c, r, wk, wv, scale)
    for h in range(2):
        assert np.allclose(out[0, h], wv[h] @ c[0], rtol=1e-13, atol=1e-14)
        own = scale * (qn[0, h] @ (wk[h] @ c[0]) + qp[0, h] @ r[0])
        assert lse[0, h] == pytest.approx(own, rel=1e-12)


def test_later_keys_do_not_reach_earlier_rows():
    T, L, H = 6, 10, 2
    qn, qp, c, r, wk, wv = _inputs(T, L, H, seed=9)
    out, lse = prefill.prefill_unabsorbed(qn, qp, c, r, wk, wv)
    c2, r2 = c.copy(), r.copy()
    c2[7:] += 3.0                                   # positions 7..9: rows i >= 3 see them
    r2[7:] -= 2.0
    out2, lse2 = prefill.prefill_unabsorbed(qn, qp, c2, r2, wk, wv)
    assert np.array_equal(out2[:3], out[:3]) and np.array_equal(lse2[:3], lse[:3])
    assert not np.allclose(out2[3:], out[3:])


# ---------------------------------------------------------------- planted mistakes
def _broken_prefill(mistake):
    """prefill_unabsorbed with one planted mistake."""
    def f(q_nope, q_pe, c, r, w_uk, w_uv, scale):
        T, L = q_nope.shape[0], c.shape[0]
        wk, wv = (w_uv, w_uk) if mistake == "swapped_up_projections" else (w_uk, w_uv)
        k, v = mla_ref.expand_kv(c, 0 * r if mistake == "dropped_rope_key" else r, wk, wv)
        q = np.concatenate([q_nope, q_pe], axis=-1)
        s = scale * np.einsum("thk,hlk->htl", q, k)
        pos = (np.arange(T) if mistake == "positions_without_prefix" else L - T + np.arange(T))
        masked = (np.arange(L)[None, :] >= pos[:, None]) if mistake == "diagonal_masked" else \
            (np.arange(L)[None, :] > pos[:, None])
        s = np.where(masked[None], -np.inf, s)
        e = np.exp(s - s.max(-1, keepdims=True))
        e = np.nan_to_num(e)
        den = np.maximum(e.sum(-1, keepdims=True), 1e-300)
        return np.einsum("htl,hld->thd", e / den, v), None
    return f


def _row_pin_holds(fn):
    qn, qp, c, r, wk, wv = _inputs(5, 12, 2, seed=77)
    out, _ = fn(qn, qp, c, r, wk, wv, 0.07)
    for i in range(5):
        p = 12 - 5 + i
        o_a, _, _ = mla_ref.absorbed_decode(qn[i], qp[i], c[:p + 1], r[:p + 1], wk, wv, 0.07)
        if not np.allclose(out[i], o_a, rtol=1e-9, atol=1e-12):
            return False
    return True


@pytest.mark.parametrize("mistake", ["swapped_up_projections", "dropped_rope_key", "positions_without_prefix",
                                     "diagonal_masked"])
def test_planted_mistakes_fail_the_row_pin(mistake):
    assert _row_pin_holds(prefill.prefill_unabsorbed)
    assert not _row_pin_holds(_broken_prefill(mistake))

"""Pins of the attention oracle against what the pages and the mathematics fix.

Sources: [Audit] "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界";
[Tutorial] "手搓 MLA:从 MHA 到 weight absorption,看懂 DeepSeek 的 KV 压缩".

None of these re-types the oracle's own formula: each compares it with an
independent route (a library routine, pure-Python loops, a closed form, an
invariance), chosen so that a dropped term, a wrong sign or index, or a
transposed operand fails at least one of them (see the planted-mistake tests
at the end).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_ref
import mla_synth


def _rand_case(rng, H=2, dn=4, dc=8, dr=4, dv=4, L=5):
    return dict(
        q_nope=rng.standard_normal((H, dn)),
        q_pe=rng.standard_normal((H, dr)),
        c=rng.standard_normal((L, dc)),
        r=rng.standard_normal((L, dr)),
        w_uk=rng.standard_normal((H, dn, dc)),
        w_uv=rng.standard_normal((H, dv, dc)),
        scale=1.0 / math.sqrt(dn + dr),
    )


def _brute_force(q_nope, q_pe, c, r, w_uk, w_uv, scale):
    """Pure-Python loops: expand keys/values per head, then softmax attention."""
    H, dn = len(q_nope), len(q_nope[0])
    L, dc = len(c), len(c[0])
    dr = len(r[0])
    dv = len(w_uv[0])
    out = [[0.0] * dv for _ in range(H)]
    for h in range(H):
        scores = []
        vals = []
        for t in range(L):
            k = [sum(w_uk[h][d][j] * c[t][j] for j in range(dc)) for d in range(dn)]
            v = [sum(w_uv[h][d][j] * c[t][j] for j in range(dc)) for d in range(dv)]
            s = sum(q_nope[h][d] * k[d] for d in range(dn)) + sum(q_pe[h][d] * r[t][d] for d in range(dr))
            scores.append(s * scale)
            vals.append(v)
        m = max(scores)
        e = [math.exp(s - m) for s in scores]
        z = sum(e)
        for d in range(dv):
            out[h][d] = sum(e[t] * vals[t][d] for t in range(L)) / z
    return np.array(out)


# ---------------------------------------------------------------- pin (a)
@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 6, 7])
def test_absorbed_equals_unabsorbed_tiny_fp64(L):
    """[Audit] §2.2/§2.3: moving W_UK to the query and W_UV after the weighted
    sum changes nothing in exact arithmetic; in fp64 the two agree to round-off
    ([Tutorial] §四 reports ~3e-17)."""
    rng = np.random.default_rng(100 + L)
    k = _rand_case(rng, L=L)
    ua, ul = mla_ref.unabsorbed_decode(k["q_nope"], k["q_pe"], k["c"], k["r"], k["w_uk"], k["w_uv"], k["scale"])
    aa, al, _ = mla_ref.absorbed_decode(k["q_nope"], k["q_pe"], k["c"], k["r"], k["w_uk"], k["w_uv"], k["scale"])
    assert np.max(np.abs(ua - aa)) <= 1e-12 * np.max(np.abs(ua))
    assert np.max(np.abs(ul - al)) <= 1e-12 * np.max(np.abs(ul))


@pytest.mark.parametrize("L", [1, 3, 6])
def test_both_paths_match_pure_python_loops(L):
    rng = np.random.default_rng(200 + L)
    k = _rand_case(rng, L=L)
    ref = _brute_force(**{kk: (v.tolist() if isinstance(v, np.ndarray) else v) for kk, v in k.items()})
    ua, _ = mla_ref.unabsorbed_decode(k["q_nope"], k["q_pe"], k["c"], k["r"], k["w_uk"], k["w_uv"], k["scale"])
    aa, _, _ = mla_ref.absorbed_decode(k["q_nope"], k["q_pe"], k["c"], k["r"], k["w_uk"], k["w_uv"], k["scale"])
    assert np.allclose(ua, ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(aa, ref, rtol=1e-12, atol=1e-13)


def test_absorbed_equals_unabsorbed_v2lite_shapes():
    """Same identity at V2-Lite shapes (H=16, 128/64/512), 300 tokens."""
    rng = np.random.default_rng(7)
    H, L = 16, 300
    qn = rng.standard_normal((H, 128))
    qp = rng.standard_normal((H, 64))
    c = rng.standard_normal((L, 512))
    r = rng.standard_normal((L, 64))
    wk = 0.02 * rng.standard_normal((H, 128, 512))
    wv = 0.02 * rng.standard_normal((H, 128, 512))
    ua, ul = mla_ref.unabsorbed_decode(qn, qp, c, r, wk, wv)
    aa, al, _ = mla_ref.absorbed_decode(qn, qp, c, r, wk, wv)
    assert np.max(np.abs(ua - aa)) <= 1e-12 * np.max(np.abs(ua))
    assert np.max(np.abs(ul - al)) <= 1e-12


def test_unabsorbed_matches_torch_sdpa_fp64():
    """The unabsorbed path is ordinary multi-head attention over expanded K/V:
    torch's scaled_dot_product_attention (CPU, float64) must agree."""
    rng = np.random.default_rng(11)
    H, L = 16, 77
    qn = rng.standard_normal((H, 128))
    qp = rng.standard_normal((H, 64))
    c = rng.standard_normal((L, 512))
    r = rng.standard_normal((L, 64))
    wk = 0.02 * rng.standard_normal((H, 128, 512))
    wv = 0.02 * rng.standard_normal((H, 128, 512))
    sc = 1.0 / math.sqrt(192)
    # Build K and V with torch's own matmul, independent of the oracle's einsums.
    ct = torch.from_numpy(c)
    kn = torch.stack([ct @ torch.from_numpy(wk[h]).T for h in range(H)])          # [H,L,128]
    kk = torch.cat([kn, torch.from_numpy(r).expand(H, L, 64)], dim=-1)          # [H,L,192]
    vv = torch.stack([ct @ torch.from_numpy(wv[h]).T for h in range(H)])          # [H,L,128]
    q = torch.cat([torch.from_numpy(qn), torch.from_numpy(qp)], dim=-1)[:, None]  # [H,1,192]
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], kk[None], vv[None], scale=sc)[0, :, 0]
    ua, _ = mla_ref.unabsorbed_decode(qn, qp, c, r, wk, wv, sc)
    aa, _, _ = mla_ref.absorbed_decode(qn, qp, c, r, wk, wv, sc)
    assert np.max(np.abs(ua - ref.numpy())) <= 1e-12 * np.max(np.abs(ref.numpy()))
    assert np.max(np.abs(aa - ref.numpy())) <= 1e-12 * np.max(np.abs(ref.numpy()))


# ---------------------------------------------------------------- closed forms
def test_single_token_returns_its_latent():
    rng = np.random.default_rng(3)
    q_lat = rng.standard_normal((4, 512))
    q_pe = rng.standard_normal((4, 64))
    c = rng.standard_normal((1, 512))
    r = rng.standard_normal((1, 64))
    o, lse = mla_ref.latent_attention(q_lat, q_pe, c, r, 0.1)
    assert np.array_equal(o, np.broadcast_to(c, o.shape))
    s = 0.1 * (q_lat @ c[0] + q_pe @ r[0])
    assert np.allclose(lse, s, rtol=0, atol=1e-14)


def test_zero_query_is_uniform_mean():
    rng = np.random.default_rng(4)
    c = rng.standard_normal((37, 512))
    r = rng.standard_normal((37, 64))
    o, lse = mla_ref.latent_attention(np.zeros((3, 512)), np.zeros((3, 64)), c, r, 0.3)
    assert np.allclose(o, c.mean(axis=0)[None], rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(37), rtol=0, atol=1e-14)


def test_identical_rows_return_that_row():
    rng = np.random.default_rng(5)
    row = rng.standard_normal(512)
    c = np.tile(row, (20, 1))
    r = rng.standard_normal((20, 64))
    o, _ = mla_ref.latent_attention(rng.standard_normal((2, 512)), rng.standard_normal((2, 64)), c, r, 0.07)
    assert np.allclose(o, row[None], rtol=0, atol=1e-13)


def test_token_permutation_invariance():
    rng = np.random.default_rng(6)
    q_lat = rng.standard_normal((5, 512))
    q_pe = rng.standard_normal((5, 64))
    c = rng.standard_normal((50, 512))
    r = rng.standard_normal((50, 64))
    p = rng.permutation(50)
    o1, l1 = mla_ref.latent_attention(q_lat, q_pe, c, r, 0.05)
    o2, l2 = mla_ref.latent_attention(q_lat, q_pe, c[p], r[p], 0.05)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14)
    assert np.allclose(l1, l2, rtol=1e-14, atol=0)


def test_rope_key_term_is_not_dropped():
    """With q_lat = 0 only the RoPE key decides the weights: a one-hot key on one
    token with a large query picks that token out."""
    c = np.eye(8, 512)
    r = np.zeros((8, 64))
    r[5, 0] = 1.0
    q_pe = np.zeros((1, 64))
    q_pe[0, 0] = 1e3
    o, _ = mla_ref.latent_attention(np.zeros((1, 512)), q_pe, c, r, 1.0)
    assert np.allclose(o[0], c[5], atol=1e-12)


# ---------------------------------------------------------------- split + merge
@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 64])
def test_split_merge_equals_unsplit(n_splits):
    rng = np.random.default_rng(50 + n_splits)
    L = 100
    q_lat = 2 * rng.standard_normal((6, 512))
    q_pe = rng.standard_normal((6, 64))
    c = rng.standard_normal((L, 512))
    r = rng.standard_normal((L, 64))
    o, lse = mla_ref.latent_attention(q_lat, q_pe, c, r, 0.07)
    parts = [mla_ref.latent_attention_range(q_lat, q_pe, c, r, a, b, 0.07)
             for a, b in mla_ref.plan_token_ranges(L, n_splits)]
    om, lm = mla_ref.lse_combine(parts)
    assert np.max(np.abs(om - o)) <= 1e-13 * np.max(np.abs(o))
    assert np.max(np.abs(lm - lse)) <= 1e-13 * np.max(np.abs(lse))


def test_merge_ignores_empty_splits_and_all_empty_is_neutral():
    rng = np.random.default_rng(9)
    c = rng.standard_normal((10, 512))
    r = rng.standard_normal((10, 64))
    ql = rng.standard_normal((2, 512))
    qp = rng.standard_normal((2, 64))
    full = mla_ref.latent_attention(ql, qp, c, r, 0.1)
    empty = mla_ref.latent_attention_range(ql, qp, c, r, 4, 4, 0.1)
    assert np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)
    om, lm = mla_ref.lse_combine([empty, full, empty])
    assert np.allclose(om, full[0], rtol=1e-14, atol=1e-15)
    assert np.allclose(lm, full[1], rtol=1e-14, atol=1e-15)
    oe, le = mla_ref.lse_combine([empty, empty])
    assert np.all(oe == 0) and np.all(np.isneginf(le))


# ---------------------------------------------------------------- paging
def test_paged_gather_equals_contiguous():
    rng = np.random.default_rng(12)
    L = 200
    c = rng.standard_normal((L, 512))
    r = rng.standard_normal((L, 64))
    n_pages = (L + 63) // 64
    pool_c = np.zeros((10, 64, 512))
    pool_r = np.zeros((10, 64, 64))
    phys = rng.permutation(10)[:n_pages]
    for i, p in enumerate(phys):
        n = min(64, L - 64 * i)
        pool_c[p, :n] = c[64 * i: 64 * i + n]
        pool_r[p, :n] = r[64 * i: 64 * i + n]
    assert np.array_equal(mla_ref.gather_seq(pool_c, phys, L), c)
    assert np.array_equal(mla_ref.gather_seq(pool_r, phys, L), r)


# ---------------------------------------------------------------- planted mistakes
def _pins_hold(mod):
    """Run the identity + library + closed-form pins against a (possibly broken) module."""
    rng = np.random.default_rng(1)
    k = _rand_case(rng, H=3, dn=4, dc=6, dr=3, dv=5, L=6)
    ref = _brute_force(**{kk: (v.tolist() if isinstance(v, np.ndarray) else v) for kk, v in k.items()})
    aa, _, _ = mod.absorbed_decode(k["q_nope"], k["q_pe"], k["c"], k["r"], k["w_uk"], k["w_uv"], k["scale"])
    ua, _ = mod.unabsorbed_decode(k["q_nope"], k["q_pe"], k["c"], k["r"], k["w_uk"], k["w_uv"], k["scale"])
    return np.allclose(aa, ref, rtol=1e-10, atol=1e-12) and np.allclose(ua, ref, rtol=1e-10, atol=1e-12)


class _Broken:
    """A copy of the oracle's public functions with one planted mistake."""

    def __init__(self, mistake):
        self.mistake = mistake

    def absorbed_decode(self, q_nope, q_pe, c, r, w_uk, w_uv, scale):
        m = self.mistake
        ql = np.einsum("hd,hdc->hc", q_nope, w_uk)
        if m == "transposed_wuk":
            # W_UK read with its two inner axes swapped (same memory, wrong index order)
            ql = np.einsum("hd,hdc->hc", q_nope, w_uk.transpose(0, 2, 1).reshape(w_uk.shape))
        pe = q_pe @ r.T
        if m == "dropped_rope":
            pe = 0 * pe
        if m == "wrong_sign":
            pe = -pe
        s = scale * (ql @ c.T + pe)
        if m == "no_scale":
            s = s / scale
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        o = p @ c
        if m == "wrong_head_index":
            o = o[::-1]
        return np.einsum("hc,hdc->hd", o, w_uv), None, o

    def unabsorbed_decode(self, *a):
        return mla_ref.unabsorbed_decode(*a)


@pytest.mark.parametrize("mistake", ["transposed_wuk", "dropped_rope", "wrong_sign", "no_scale",
                                     "wrong_head_index"])
def test_planted_mistakes_fail_the_pins(mistake):
    assert _pins_hold(mla_ref)
    assert not _pins_hold(_Broken(mistake))


def test_float32_twin_matches_the_float64_oracle():
    """The CPU baseline's float32 form of the absorbed decode agrees with the
    float64 oracle to float32 round-off (it is timed, never used as a reference)."""
    case = mla_synth.small_decode(case_id=31, H=16, seq_lens=[700])
    c_bits, r_bits = case.seq_cache(0)
    f = mla_ref.bf16_to_f64
    args = (f(case.q_nope[0]), f(case.q_pe[0]), f(c_bits), f(r_bits), f(case.w_uk), f(case.w_uv), case.softmax_scale)
    ref, _, _ = mla_ref.absorbed_decode(*args)
    got = mla_ref.absorbed_decode_f32(*args)
    assert got.dtype == np.float32
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))

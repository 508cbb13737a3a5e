"""Why the matrix-core operands are fp16 (CPU only, no GPU code involved).

The decode's rounding steps are emulated in numpy on one sequence with the
V3-shaped workload's sizes and value distributions (H=128, L=8192), and the
result is compared with the fp64 oracle under the output tolerance
(max|d| <= 1e-2 max|ref|, sum|d| / sum|ref| <= 2e-3).  Emulated: the absorbed
query rounded once; scores accumulated exactly, scaled in fp32; a fixed
reference maximum per split (its first 32-token tile); P rounded for the value
product while the fp32 sum takes the unrounded weights; split partials rounded
to fp16; the merged latent rounded to fp16 before the W_UV expansion; the
output rounded to bf16.

With q_abs and P in fp16 the output meets the tolerance; with both in bf16 (the
other 16-bit matrix-core type) it exceeds the mean-relative bound.

FP8 (e4m3) operands, for an FP8 latent cache on the FP8 matrix instructions:
rounded once to e4m3 with an fp32 scale (per head and 32-column block for q_abs,
per head for P), either operand misses the mean-relative bound by about ten
times; split into two e4m3 terms (the value and the e4m3 rounding of its
remainder, both products accumulated in fp32) both operands meet it.  Two FP8
products take the matrix cores as long as one fp16 product of the same shape
(twice the rate, twice the work), so FP8 matrix instructions can only save
operand conversion and LDS traffic, not matrix time.
"""
import numpy as np
import pytest
import torch

import mla_synth
from oracle import mla_ref

MAX_REL, MEAN_REL = 1e-2, 2e-3


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _emulate(case, rq, rp, n_splits=4):
    c_bits, r_bits = case.seq_cache(0)
    c = mla_ref.bf16_to_f64(c_bits)
    r = mla_ref.bf16_to_f64(r_bits)
    qn = mla_ref.bf16_to_f64(case.q_nope[0])
    qp = mla_ref.bf16_to_f64(case.q_pe[0])
    w_uk = mla_ref.bf16_to_f64(case.w_uk)
    w_uv = mla_ref.bf16_to_f64(case.w_uv)
    ref, _, _ = mla_ref.absorbed_decode(qn, qp, c, r, w_uk, w_uv, case.softmax_scale)

    q = rq(np.concatenate([mla_ref.absorb_q(qn[None], w_uk)[0], qp], axis=1)).astype(np.float64)
    keys = np.concatenate([c, r], axis=1)
    s = (q @ keys.T).astype(np.float32) * np.float32(case.softmax_scale * np.log2(np.e))
    L = s.shape[1]
    parts = []
    for j in range(n_splits):
        t0, t1 = j * L // n_splits, (j + 1) * L // n_splits
        ss = s[:, t0:t1]
        m = ss[:, :32].max(axis=1, keepdims=True)
        e = np.exp2(ss - m).astype(np.float32)
        l_sum = e.sum(axis=1, dtype=np.float32)
        o = (rp(e).astype(np.float64) @ c[t0:t1]).astype(np.float32) / l_sum[:, None]
        parts.append((_f16(o).astype(np.float64), (m[:, 0] + np.log2(l_sum)) * np.log(2.0)))
    lse = np.stack([p[1] for p in parts])
    w = np.exp(lse - lse.max(axis=0))
    o_lat = sum(w[j][:, None] * parts[j][0] for j in range(n_splits)) / w.sum(axis=0)[:, None]
    out = np.einsum("hc,hdc->hd", _f16(o_lat).astype(np.float64), w_uv)
    out = _bf16(out).astype(np.float64)
    d = np.abs(out - ref)
    return d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).sum()


@pytest.fixture(scope="module")
def v3_sequence():
    return mla_synth.small_decode(case_id=3, H=128, seq_lens=[8192])


def test_fp16_operands_meet_the_tolerance(v3_sequence):
    mx, mean = _emulate(v3_sequence, _f16, _f16)
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)


def test_bf16_operands_exceed_the_mean_relative_bound(v3_sequence):
    mx, mean = _emulate(v3_sequence, _bf16, _bf16)
    assert mean > MEAN_REL, (mx, mean)


def _e4m3(x):
    """float32 -> nearest e4m3 value (torch's float8_e4m3fn conversion)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float32).numpy()


def _fp8(group=None):
    """Round to e4m3 with an fp32 scale (max|x| -> 448) per `group` consecutive
    values of the last axis (the whole row when None)."""
    def r(x):
        x = np.asarray(x, np.float32)
        shp = x.shape
        g = shp[-1] if group is None else group
        xg = x.reshape(shp[:-1] + (shp[-1] // g, g))
        s = (np.abs(xg).max(axis=-1, keepdims=True) / np.float32(448.0)).astype(np.float32)
        s = np.where(s == 0, np.float32(1.0), s)
        return (_e4m3(xg / s) * s).reshape(shp)
    return r


def _two_term(r1):
    def r(x):
        hi = r1(x)
        return hi + r1(np.asarray(x, np.float32) - hi)
    return r


def test_e4m3_operands_exceed_the_mean_relative_bound(v3_sequence):
    _, mean_q = _emulate(v3_sequence, _fp8(32), _f16)
    _, mean_p = _emulate(v3_sequence, _f16, _fp8())
    assert mean_q > 5 * MEAN_REL and mean_p > 5 * MEAN_REL, (mean_q, mean_p)


def test_two_term_e4m3_operands_meet_the_tolerance(v3_sequence):
    mx, mean = _emulate(v3_sequence, _two_term(_fp8(32)), _two_term(_fp8()))
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)

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
"""
import numpy as np
import pytest

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

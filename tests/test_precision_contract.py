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
operand conversion and LDS traffic, not matrix time.  The last test emulates
the 16-head FP8 decode's own form of that split (power-of-two scales per head
for q~ and per 32 tokens and head for P, the token scale folded into P, the
cache's e4m3 codes as the other operand) on the quantised V2-Lite workload.
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


def _pow2_split(x, axis):
    """The FP8 decode's operand split: a power-of-two scale per slice along
    `axis` (the slice maximum mapped into [128, 256)), two e4m3 terms with the
    second scaled by 2^4; returns the value the matrix core multiplies."""
    x = np.asarray(x, np.float32)
    m = np.abs(x).max(axis=axis, keepdims=True)
    e = np.where(m > 0, np.floor(np.log2(np.where(m > 0, m, 1.0))) - 7, 0).clip(-120, 120)
    s = np.float32(2.0) ** e.astype(np.float32)
    y = (x / s).astype(np.float32)
    hi = _e4m3(y)
    lo = _e4m3((y - hi) * np.float32(16.0))
    return ((hi.astype(np.float64) + lo.astype(np.float64) / 16.0) * s).astype(np.float64)


def test_fp8_matrix_instruction_scheme_meets_the_tolerance():
    """The 16-head FP8 decode's arithmetic on the per-token FP8 cache of the
    quantised V2-Lite workload (one 16,384-token sequence): latent scores from
    the e4m3 codes times q~ split in two e4m3 terms (power-of-two scale per head),
    times the token's scale; RoPE key widened to fp16; softmax with the running
    maximum moved when a 128-token tile exceeds it by more than 8; P times the
    token scale split in two e4m3 terms (power-of-two scale per 32 tokens and
    head) against the raw codes; fp16 partial, fp16 latent into W_UV, bf16
    output.  Reference: the fp64 oracle over the same dequantised cache."""
    from oracle import quant
    case = mla_synth.small_decode(case_id=5, H=16, seq_lens=[16384], normalise=False, outliers=True)
    c_bits, r_bits = case.seq_cache(0)
    f = quant.encode_tokens(quant.CACHE_FP8_TOK, c_bits, r_bits)
    c32, r32 = quant.dequant_fields(quant.CACHE_FP8_TOK, f)
    qn = mla_ref.bf16_to_f64(case.q_nope[0])
    qp = mla_ref.bf16_to_f64(case.q_pe[0])
    w_uk = mla_ref.bf16_to_f64(case.w_uk)
    w_uv = mla_ref.bf16_to_f64(case.w_uv)
    ref, _, _ = mla_ref.absorbed_decode(qn, qp, c32.astype(np.float64), r32.astype(np.float64), w_uk, w_uv,
                                        case.softmax_scale)

    codes = f["codes"]
    v_lat = quant.fp8_e4m3_decode(codes[:, :512]).astype(np.float64)          # raw e4m3 values
    lat_s = f["c_scale"].reshape(-1).astype(np.float64)
    r_val = _f16(_f16(quant.fp8_e4m3_decode(codes[:, 512:]) / 256.0)
                 * _f16(np.repeat(f["r_scale"], 8, axis=1) * 256.0)).astype(np.float64)
    q_abs = _f16(mla_ref.absorb_q(qn[None], w_uk)[0])                          # fp16 q~, as stored
    q_eff = _pow2_split(q_abs, axis=1)
    s = ((v_lat @ q_eff.T) * lat_s[:, None] + r_val @ _f16(qp).astype(np.float64).T).T   # [H, L]
    s = (s * case.softmax_scale / np.log(2.0)).astype(np.float32)
    H, L = s.shape
    m = np.full(H, -np.inf, np.float32)
    l_sum = np.zeros(H, np.float64)
    o = np.zeros((H, 512))
    for t0 in range(0, L, 128):
        st = s[:, t0:t0 + 128]
        mt = st.max(axis=1)
        need = mt > m + 8.0
        if np.any(need):
            alpha = np.where(need, np.exp2(np.where(np.isfinite(m), m - np.where(need, mt, m), -np.inf)), 1.0)
            o *= alpha[:, None]
            l_sum *= alpha
            m = np.where(need, mt, m)
        p = np.exp2(st - m[:, None]).astype(np.float32)
        l_sum += p.sum(axis=1, dtype=np.float32)
        pp = (p * lat_s[None, t0:t0 + 128]).astype(np.float32)
        blocks = pp.reshape(H, -1, 32)
        p_eff = _pow2_split(blocks, axis=2).reshape(H, -1)
        o += p_eff @ v_lat[t0:t0 + 128]
    o_lat = _f16(o / l_sum[:, None]).astype(np.float64)
    out = _bf16(np.einsum("hc,hdc->hd", o_lat, w_uv)).astype(np.float64)
    d = np.abs(out - ref)
    mx, mean = d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).sum()
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)

"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Tolerance for the bf16 outputs (floating point): max|out - ref| <= 1e-2 max|ref|
and sum|out - ref| / sum|ref| <= 2e-3, ref = the oracle's fp64 result from the
same bf16 inputs.  Quantised codes and scales: bit-exact.  Paging invariance and
determinism: bitwise (GPU against GPU).
"""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import (DEV, MAX_REL, MEAN_REL, errors, lse_bound, oracle_seq, run_step, to_dev_bits, upload)
from mla_absorbed_latent_amd import api
from oracle import mla_ref, quant

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ a-1 append
@pytest.mark.parametrize("cache_dtype", [0, 1, 2, 3, 4, 5, 6])
def test_append_bitexact(cache_dtype):
    case = mla_synth.small_decode(case_id=11, H=16, seq_lens=[1, 63, 64, 65, 130], paging="shuffled",
                                  normalise=cache_dtype == 0, outliers=cache_dtype != 0, extra_pages=3)
    _note("append dtype=%d pages=%d" % (cache_dtype, case.num_pages))
    run, dev = upload(case, cache_dtype)
    torch.cuda.synchronize()
    pool = run.pool.cpu().numpy().reshape(case.num_pages, -1)
    ref = quant.pack_pool(cache_dtype, case.num_pages,
                          [(*case.seq_cache(b), case.block_table[b]) for b in range(case.B)])
    for b in range(case.B):
        L = int(case.seq_lens[b])
        for p0 in range(0, L, 64):
            page = int(case.block_table[b, p0 // 64])
            n = min(64, L - p0)
            g = quant.unpack_page(cache_dtype, pool[page])
            r = quant.unpack_page(cache_dtype, ref[page])
            for k in r:
                assert np.array_equal(g[k][:n], r[k][:n]), (b, p0, k)


# ------------------------------------------------------------------ a-2 absorb
@pytest.mark.parametrize("H,B", [(16, 5), (128, 40), (16, 64)])
def test_absorb_q(H, B):
    case = mla_synth.small_decode(case_id=12, H=H, seq_lens=[1] * B)
    cfg = api.config(H)
    q_abs = torch.empty(B, H, 576, dtype=torch.float16, device=DEV)
    api.absorb_q(cfg, to_dev_bits(case.q_nope), to_dev_bits(case.q_pe), to_dev_bits(case.w_uk), q_abs)
    got = q_abs.float().cpu().numpy().astype(np.float64)
    ref = mla_ref.absorb_q(mla_ref.bf16_to_f64(case.q_nope), mla_ref.bf16_to_f64(case.w_uk))
    mx, mean = errors(got[..., :512], ref)
    assert mx <= 2e-3 and mean <= 5e-4, (mx, mean)            # fp16 rounding of fp32 sums
    # q_pe passes through bf16 -> fp16: exact for |x| >= 2^-17 (bf16 has 8 significant
    # bits); below that fp16's subnormal grid (2^-24) limits it.
    qpe = mla_ref.bf16_to_f64(case.q_pe)
    big = np.abs(qpe) >= 2.0 ** -17
    assert np.array_equal(got[..., 512:][big], qpe[big])
    assert np.all(np.abs(got[..., 512:][~big] - qpe[~big]) <= 2.0 ** -24)


# ------------------------------------------------------------------ a-3..a-5 end to end, small
SMALL = [
    (16, [1, 2, 63, 64, 65, 300, 1000]),
    (128, [1, 31, 32, 33, 64, 100, 777]),
    (16, [4096, 17, 5000]),
    (128, [2048, 129, 3000]),
]


@pytest.mark.parametrize("H,lens", SMALL)
@pytest.mark.parametrize("chunk", [0, 1, 3])
@pytest.mark.parametrize("paging", ["shuffled", "identity"])
def test_decode_small(H, lens, chunk, paging):
    case = mla_synth.small_decode(case_id=13, H=H, seq_lens=lens, paging=paging, extra_pages=2)
    _note("decode H=%d lens=%s chunk=%d paging=%s" % (H, lens, chunk, paging))
    run, dev = upload(case)
    out = run_step(run, dev, case.seq_lens, chunk_pages=chunk).float().cpu().numpy()
    o_lat = run.o_lat.cpu().numpy()
    lse = run.lse.cpu().numpy()
    for b in range(case.B):
        ref_out, ref_lse, ref_olat = oracle_seq(case, b)
        mx, mean = errors(out[b], ref_out)
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, mx, mean)
        mx, mean = errors(o_lat[b], ref_olat)
        assert mx <= MAX_REL and mean <= MEAN_REL, ("o_lat", b, mx, mean)
        if not np.isfinite(ref_lse).all():     # an empty sequence: -inf for every head
            assert np.all(np.isneginf(lse[b])) and np.all(np.isneginf(ref_lse))
            continue
        tol = lse_bound(case, b) + 1e-5 * np.maximum(1.0, np.abs(ref_lse))
        assert np.all(np.abs(lse[b] - ref_lse) <= tol), ("lse", b, np.max(np.abs(lse[b] - ref_lse) / tol))


QUANT_DECODE_READY = True
needs_quant = pytest.mark.skipif(not QUANT_DECODE_READY, reason="quantised decode kernels not built yet")


@needs_quant
@pytest.mark.parametrize("cache_dtype", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("H", [16, 128])
def test_decode_quantised_small(cache_dtype, H):
    case = mla_synth.small_decode(case_id=14, H=H, seq_lens=[1, 70, 640, 2000], normalise=False, outliers=True)
    _note("decode quant dtype=%d H=%d" % (cache_dtype, H))
    run, dev = upload(case, cache_dtype)
    out = run_step(run, dev, case.seq_lens, chunk_pages=4).float().cpu().numpy()
    for b in range(case.B):
        ref_out, _, _ = oracle_seq(case, b, cache_dtype)
        mx, mean = errors(out[b], ref_out)
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, mx, mean)


@pytest.mark.parametrize("H", [16, 128])
def test_paging_invariance_bitwise(H):
    lens = [700, 64, 1500]
    a = mla_synth.small_decode(case_id=15, H=H, seq_lens=lens, paging="identity")
    b = mla_synth.small_decode(case_id=15, H=H, seq_lens=lens, paging="shuffled")
    ra, da = upload(a)
    rb, db = upload(b)
    oa = run_step(ra, da, lens, chunk_pages=3).clone()
    ob = run_step(rb, db, lens, chunk_pages=3).clone()
    assert torch.equal(oa, ob)
    assert torch.equal(ra.lse, rb.lse)


@pytest.mark.parametrize("H", [16, 128])
def test_determinism_bitwise(H):
    lens = [900, 33, 4096]
    case = mla_synth.small_decode(case_id=16, H=H, seq_lens=lens)
    run, dev = upload(case)
    o1 = run_step(run, dev, lens).clone()
    l1 = run.lse.clone()
    o2 = run_step(run, dev, lens).clone()
    assert torch.equal(o1, o2) and torch.equal(l1, run.lse)


@pytest.mark.parametrize("H", [16, 128])
def test_split_plans_agree(H):
    lens = [3000, 5000]
    case = mla_synth.small_decode(case_id=17, H=H, seq_lens=lens)
    run, dev = upload(case)
    outs = [run_step(run, dev, lens, chunk_pages=c).float().cpu().numpy() for c in (1, 5, 1000)]
    for o in outs[1:]:
        mx, mean = errors(o, outs[0].astype(np.float64))
        assert mx <= MAX_REL and mean <= MEAN_REL


@pytest.mark.parametrize("H", [16, 128])
def test_empty_sequence_and_invalid_pages(H):
    lens = [0, 200, 130]
    case = mla_synth.small_decode(case_id=18, H=H, seq_lens=[1, 200, 130])
    case.seq_lens[0] = 0                       # empty sequence
    run, dev = upload(case)
    # an out-of-range page id for sequence 2's second page: its tokens count for nothing
    bt = case.block_table.copy()
    bt[2, 1] = case.num_pages + 5
    dev["block_table"] = torch.from_numpy(bt).to(DEV)
    dev["seq_lens"] = torch.from_numpy(np.array(lens, np.int32)).to(DEV)
    out = run_step(run, dev, lens, chunk_pages=1).float().cpu().numpy()
    assert np.all(out[0] == 0) and np.all(np.isneginf(run.lse[0].cpu().numpy()))
    ref1, _, _ = oracle_seq(case, 1)
    mx, mean = errors(out[1], ref1)
    assert mx <= MAX_REL and mean <= MEAN_REL
    # sequence 2 with only tokens 0..63 and 128..129 visible
    c_bits, r_bits = case.seq_cache(2)
    keep = np.r_[0:64, 128:130]
    o2, _, _ = mla_ref.absorbed_decode(mla_ref.bf16_to_f64(case.q_nope[2]), mla_ref.bf16_to_f64(case.q_pe[2]),
                                       mla_ref.bf16_to_f64(c_bits[keep]), mla_ref.bf16_to_f64(r_bits[keep]),
                                       mla_ref.bf16_to_f64(case.w_uk), mla_ref.bf16_to_f64(case.w_uv),
                                       case.softmax_scale)
    mx, mean = errors(out[2], o2)
    assert mx <= MAX_REL and mean <= MEAN_REL


@pytest.mark.parametrize("H", [16, 128])
def test_fused_merge_expand_matches_separate(H):
    """mla_decode_combine_out_proj against mla_decode_combine + mla_out_proj on the
    same partials: o_lat and lse bitwise (same sums in the same order), out within
    the output tolerance (the expansion sums its 512 terms in another order)."""
    lens = [1, 700, 64, 2500, 0, 33] + [130] * 30      # more than one 32-sequence block
    case = mla_synth.small_decode(case_id=20, H=H, seq_lens=[max(1, L) for L in lens])
    case.seq_lens[4] = 0
    run, dev = upload(case)
    dev["seq_lens"] = torch.from_numpy(case.seq_lens.astype(np.int32)).to(DEV)
    run.plan(case.seq_lens, chunk_pages=2)
    run.step(dev["q_nope"], dev["q_pe"], dev["w_uk"], dev["w_uv"], dev["block_table"], dev["seq_lens"], fused=False)
    torch.cuda.synchronize()
    out_sep, olat_sep, lse_sep = run.out.clone(), run.o_lat.clone(), run.lse.clone()
    run.combine_project(dev["w_uv"])
    torch.cuda.synchronize()
    assert torch.equal(run.o_lat, olat_sep) and torch.equal(run.lse, lse_sep)
    mx, mean = errors(run.out.float().cpu().numpy(), out_sep.float().cpu().numpy().astype(np.float64))
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    # without the latent outputs the expansion is unchanged, bit for bit
    out_keep = run.out.clone()
    run.out.zero_()
    run.combine_project(dev["w_uv"], keep_latent=False)
    torch.cuda.synchronize()
    assert torch.equal(run.out, out_keep)
    for b in (0, 1, 3, 4, 35):
        ref_out, _, _ = oracle_seq(case, b)
        if case.seq_lens[b] == 0:
            assert np.all(run.out[b].float().cpu().numpy() == 0)
            continue
        mx, mean = errors(run.out[b].float().cpu().numpy(), ref_out)
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, mx, mean)


@pytest.mark.parametrize("H", [16, 128])
def test_merge_with_no_split_rows(H):
    """Split offsets that give no sequence any row (a caller's plan with no work
    items): both merges write zeros and lse = -inf and read none of the partial
    rows, which here hold NaNs and huge lse values."""
    B = 40
    cfg = api.config(H, 0, 0.07)
    o_part = torch.full((1, H, 512), float("nan"), dtype=torch.float16, device=DEV)
    lse_part = torch.full((1, H), 1e30, dtype=torch.float32, device=DEV)
    offsets = torch.zeros(B + 1, dtype=torch.int32, device=DEV)
    w_uv = torch.randn(H, 128, 512, device=DEV).to(torch.bfloat16)
    out = torch.full((B, H, 128), 1.0, dtype=torch.bfloat16, device=DEV)
    o_lat = torch.full((B, H, 512), 1.0, dtype=torch.float32, device=DEV)
    lse = torch.zeros(B, H, dtype=torch.float32, device=DEV)
    api.decode_combine_out_proj(cfg, o_part, lse_part, offsets, w_uv, out, o_lat, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(o_lat == 0) and torch.all(torch.isneginf(lse))
    o_lat.fill_(1.0)
    lse.zero_()
    api.decode_combine(cfg, o_part, lse_part, offsets, o_lat, lse)
    torch.cuda.synchronize()
    assert torch.all(o_lat == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("hidden", [2048, 520])
@pytest.mark.parametrize("fused", [True, False])
def test_output_projection_with_wo(fused, hidden):
    """V2-Lite layer shapes: one sequence of 26 tokens, H=16, W_O to hidden 2048,
    and a non-square W_O (hidden 520 != 16 * 128) that a transposed operand on
    either side would not survive."""
    layer = mla_synth.v2lite_layer()
    if hidden != 2048:
        w = np.random.default_rng(71).standard_normal((hidden, 16 * 128)).astype(np.float32) * np.float32(0.02)
        layer.w_o = mla_synth.f32_to_bf16_bits(w)
    case = mla_synth.small_decode(case_id=19, H=16, seq_lens=[26])
    run, dev = upload(case)
    run.plan([26], chunk_pages=0)
    y = torch.empty(1, hidden, dtype=torch.bfloat16, device=DEV)
    of = torch.empty(1, 16, 128, dtype=torch.float32, device=DEV)
    run.step(dev["q_nope"], dev["q_pe"], dev["w_uk"], dev["w_uv"], dev["block_table"], dev["seq_lens"],
             w_o=to_dev_bits(layer.w_o), y=y, out_f32=of, fused=fused)
    torch.cuda.synchronize()
    ref_out, _, _ = oracle_seq(case, 0)
    ref_y = mla_ref.wo_proj(ref_out[None], mla_ref.bf16_to_f64(layer.w_o))[0]
    mx, mean = errors(y.float().cpu().numpy()[0], ref_y)
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    mx, mean = errors(of.cpu().numpy()[0], ref_out)
    assert mx <= MAX_REL and mean <= MEAN_REL


@pytest.mark.parametrize("H", [16, 128])
def test_item_longer_than_a_page_table_segment(H):
    """One work item of 1,032 pages: the kernels copy the block table to LDS in
    segments of 1,024 pages, so this item crosses a segment boundary (and ends in
    a ragged tile).  A short second sequence rides along."""
    lens = [66_000, 300]
    case = mla_synth.small_decode(case_id=21, H=H, seq_lens=lens)
    run, dev = upload(case)
    run.plan(lens, chunk_pages=2000)
    assert run.n_items == 2
    out = run.step(dev["q_nope"], dev["q_pe"], dev["w_uk"], dev["w_uv"], dev["block_table"], dev["seq_lens"])
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    for b in (0, 1):
        ref_out, _, _ = oracle_seq(case, b)
        mx, mean = errors(out[b], ref_out)
        _note("  seq %d L=%d max_rel %.2e mean_rel %.2e" % (b, lens[b], mx, mean))
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, mx, mean)


# ------------------------------------------------------------------ full-size workloads, sampled
FULL = [
    ("v2lite_decode", lambda: mla_synth.v2lite_decode(), 0),
    ("v3_decode", lambda: mla_synth.v3_decode(), 0),
    ("v3_ragged", lambda: mla_synth.v3_ragged(), 0),
    pytest.param("v2lite_quant_int8", lambda: mla_synth.v2lite_quant(), 1, marks=needs_quant),
    pytest.param("v2lite_quant_int4", lambda: mla_synth.v2lite_quant(), 2, marks=needs_quant),
    pytest.param("v2lite_quant_int4s", lambda: mla_synth.v2lite_quant(), 3, marks=needs_quant),
    pytest.param("v2lite_quant_int8t", lambda: mla_synth.v2lite_quant(), 4, marks=needs_quant),
    pytest.param("v2lite_quant_fp8t", lambda: mla_synth.v2lite_quant(), 5, marks=needs_quant),
    pytest.param("v2lite_quant_int4k4", lambda: mla_synth.v2lite_quant(), 6, marks=needs_quant),
]


@pytest.mark.parametrize("name,make,cache_dtype", FULL,
                         ids=["v2lite_decode", "v3_decode", "v3_ragged", "v2lite_quant_int8", "v2lite_quant_int4",
                              "v2lite_quant_int4s", "v2lite_quant_int8t", "v2lite_quant_fp8t",
                              "v2lite_quant_int4k4"])
def test_full_size_sampled(name, make, cache_dtype):
    case = make()
    _note("full %s B=%d H=%d tokens=%d" % (name, case.B, case.H, case.total_tokens))
    run, dev = upload(case, cache_dtype)
    out = run_step(run, dev, case.seq_lens).float().cpu().numpy()
    lens = case.seq_lens
    picks = sorted({0, case.B // 2, case.B - 1, int(np.argmax(lens)), int(np.argmin(lens))})
    for b in picks:
        ref_out, _, _ = oracle_seq(case, b, cache_dtype)
        mx, mean = errors(out[b], ref_out)
        _note("  seq %d L=%d max_rel %.2e mean_rel %.2e" % (b, lens[b], mx, mean))
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, mx, mean)
    assert np.isfinite(out).all()


@pytest.mark.parametrize("cache_dtype", [0, 1])
@pytest.mark.parametrize("H,B", [(128, 64), (16, 5)])
def test_append_absorb_fused_matches_the_two_calls(cache_dtype, H, B):
    """mla_append_absorb_q (one launch for a bf16 cache) writes the same pool
    bytes and q_abs, bit for bit, as mla_cache_append then mla_absorb_q; one
    slot is out of range and skipped by both."""
    case = mla_synth.small_decode(case_id=23, H=H, seq_lens=[1] * B)
    cfg = api.config(H, cache_dtype)
    pages = 4
    page = api.cache_page_bytes(cfg)
    c = to_dev_bits(mla_synth.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((B, 512)).astype(np.float32)))
    r = to_dev_bits(mla_synth.f32_to_bf16_bits(np.random.default_rng(4).standard_normal((B, 64)).astype(np.float32)))
    slots = np.random.default_rng(5).permutation(pages * 64)[:B].astype(np.int64)
    slots[B // 2] = pages * 64 + 7                          # out of range: skipped
    slots = torch.from_numpy(slots).to(DEV)
    qn, qp, wk = to_dev_bits(case.q_nope), to_dev_bits(case.q_pe), to_dev_bits(case.w_uk)
    pool_a = torch.zeros(pages * page, dtype=torch.uint8, device=DEV)
    pool_b = torch.zeros_like(pool_a)
    qa = torch.empty(B, H, 576, dtype=torch.float16, device=DEV)
    qb = torch.empty_like(qa)
    api.cache_append(cfg, pool_a, c, r, slots)
    api.absorb_q(cfg, qn, qp, wk, qa)
    api.append_absorb_q(cfg, pool_b, c, r, slots, qn, qp, wk, qb)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b)
    assert torch.equal(qa.view(torch.int16), qb.view(torch.int16))
    assert pool_a.any()

"""GPU parity on inputs that drive the decode's rarely taken branches and the
edges of its documented input range, through the C ABI, against the fp64 oracle.

* Softmax: the 128-head kernel fixes each head's reference maximum at the first
  tile of a work item and redoes the item against exact maxima when a later
  tile exceeds it by more than 2^15; the 16-head kernel rescales its running
  sums only when a wave's maximum grows by more than 2^8.  Queries scaled by 6
  spread the scores over about 50 log2 units (35 nats), so the maximum arrives
  late and both branches run; a sequence whose first tile holds rows scaled by
  4 puts the maximum first and lets later scores fall by more than 24 log2
  units for some heads (their fp16 probabilities underflow to zero), the shape
  of an attention sink.  Each case checks, on the CPU from the oracle's own
  scores, that it really exercises the branch.
* Dequantisation range: caches shrunk by 2^-8, latent groups shrunk to
  max|x| < 2^-7 inside normal tokens, and INT4 groups whose zero point is about
  150 times their scale.
* Work items whose page range lies past the block table (first_page = 2^25,
  where 32-bit token arithmetic would wrap) give o = 0 and lse = -inf.

Tolerance as everywhere: max|out - ref| <= 1e-2 max|ref|, sum|out - ref| /
sum|ref| <= 2e-3.
"""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import DEV, MAX_REL, MEAN_REL, errors, oracle_seq, run_step, upload
from mla_absorbed_latent_amd import api
from oracle import mla_ref, quant

pytestmark = pytest.mark.gpu

FORMATS = [0, 1, 2, 3, 4, 5, 6]


def _note(msg):
    print(msg, flush=True)


def _scaled_bits(bits, factor):
    return mla_synth.f32_to_bf16_bits(mla_synth.bf16_bits_to_f32(bits) * np.float32(factor))


def _with_cache_transform(case, fn):
    """Replace case.seq_cache by fn(b, c_bits, r_bits) -> (c_bits, r_bits)."""
    base = case.seq_cache

    def seq_cache(b):
        c, r = base(b)
        return fn(b, c, r)

    case.seq_cache = seq_cache
    return case


def _log2_scores(case, b, cache_dtype):
    """Oracle scores of sequence b in log2 units, [H, L] (from its dequantised cache)."""
    c_bits, r_bits = case.seq_cache(b)
    if cache_dtype == 0:
        c, r = mla_ref.bf16_to_f64(c_bits), mla_ref.bf16_to_f64(r_bits)
    else:
        c32, r32 = quant.dequant_fields(cache_dtype, quant.encode_tokens(cache_dtype, c_bits, r_bits))
        c, r = c32.astype(np.float64), r32.astype(np.float64)
    q_lat = mla_ref.absorb_q(mla_ref.bf16_to_f64(case.q_nope[b]), mla_ref.bf16_to_f64(case.w_uk))
    s = case.softmax_scale * (q_lat @ c.T + mla_ref.bf16_to_f64(case.q_pe[b]) @ r.T)
    return s / np.log(2.0)


def _h128_redo_taken(s):
    """Some head's maximum after the first 32-token tile exceeds its first tile's by > 15."""
    return bool(np.any(s[:, 32:].max(axis=1) > s[:, :32].max(axis=1) + 15.0))


def _h16_rescale_taken(s, cache_dtype=0):
    """Some head's running maximum grows by more than 8 after a non-empty tile,
    so its sums are rescaled by a factor other than 0.  The 16-head kernels keep
    that maximum per compute wave over tokens 16 w .. 16 w + 15 of every 64-token
    tile, except the FP8 one, whose waves share one maximum per 128-token tile."""
    H, L = s.shape
    tile, part = (128, 128) if cache_dtype == 5 else (64, 16)
    for w in range(tile // part):
        m = np.full(H, -np.inf)
        for t0 in range(0, L, tile):
            lo, hi = t0 + part * w, min(t0 + part * w + part, L)
            if lo >= hi:
                continue
            mx = s[:, lo:hi].max(axis=1)
            need = mx > m + 8.0
            if np.any(need & np.isfinite(m)):
                return True
            m = np.where(need, mx, m)
    return False


def _check(case, cache_dtype, chunk):
    run, dev = upload(case, cache_dtype)
    out = run_step(run, dev, case.seq_lens, chunk_pages=chunk).float().cpu().numpy()
    assert np.isfinite(out).all()
    for b in range(case.B):
        ref_out, _, _ = oracle_seq(case, b, cache_dtype)
        mx, mean = errors(out[b], ref_out)
        _note("  seq %d L=%d max_rel %.2e mean_rel %.2e" % (b, case.seq_lens[b], mx, mean))
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, mx, mean)


# ------------------------------------------------------------------ softmax branches
def _spread_case(H, case_id=60):
    """Queries scaled by 6: scores span about 50 log2 units; the maximum arrives late."""
    case = mla_synth.small_decode(case_id=case_id, H=H, seq_lens=[1500, 900])
    case.q_nope = _scaled_bits(case.q_nope, 6.0)
    case.q_pe = _scaled_bits(case.q_pe, 6.0)
    return case


def _early_max_case(H, case_id=61):
    """As above, and the first 32 rows of every sequence scaled by 4: for most
    heads the maximum sits in the first tile, and for some later scores fall by
    more than 24 log2 units."""
    case = _spread_case(H, case_id)

    def fn(b, c, r):
        c, r = c.copy(), r.copy()
        c[:32] = _scaled_bits(c[:32], 4.0)
        r[:32] = _scaled_bits(r[:32], 4.0)
        return c, r

    return _with_cache_transform(case, fn)


@pytest.mark.parametrize("cache_dtype", FORMATS)
@pytest.mark.parametrize("H", [16, 128])
def test_late_maximum(H, cache_dtype):
    case = _spread_case(H)
    scores = [_log2_scores(case, b, cache_dtype) for b in range(case.B)]
    taken = _h128_redo_taken if H == 128 else (lambda s: _h16_rescale_taken(s, cache_dtype))
    assert any(taken(s) for s in scores), "case does not reach the branch"
    _note("late max H=%d dtype=%d spread %.1f log2" % (H, cache_dtype, float(np.ptp(scores[0]))))
    _check(case, cache_dtype, chunk=1000)      # one work item per sequence


@pytest.mark.parametrize("cache_dtype", FORMATS)
@pytest.mark.parametrize("H", [16, 128])
def test_early_maximum_then_falling_scores(H, cache_dtype):
    case = _early_max_case(H)
    s = _log2_scores(case, 0, cache_dtype)
    fall = s[:, :32].max(axis=1) - s[:, 32:].max(axis=1)
    assert np.any(fall > 24.0) and np.mean(fall > 0) > 0.5, (float(fall.max()), float(np.mean(fall > 0)))
    _note("early max H=%d dtype=%d largest fall %.1f log2" % (H, cache_dtype, float(fall.max())))
    _check(case, cache_dtype, chunk=1000)


@pytest.mark.parametrize("H", [16, 128])
def test_late_maximum_split_items(H):
    """The same spread with split work items (each item fixes its own reference)."""
    case = _spread_case(H, case_id=62)
    _check(case, 0, chunk=3)


# ------------------------------------------------------------------ dequantisation range
def _shrunk_case(H):
    """Every cached value scaled by 2^-8 (group scales down to about 3e-5)."""
    case = mla_synth.small_decode(case_id=63, H=H, seq_lens=[700, 130], normalise=False, outliers=True)
    return _with_cache_transform(case, lambda b, c, r: (_scaled_bits(c, 2.0 ** -8), _scaled_bits(r, 2.0 ** -8)))


def _tiny_groups_case(H):
    """Latent groups 3 and 9 (channels 96..127, 288..319) scaled by 2^-14 in every
    token: max|x| < 2^-7 inside tokens whose other groups are normal."""
    case = mla_synth.small_decode(case_id=64, H=H, seq_lens=[700, 130], normalise=False, outliers=True)

    def fn(b, c, r):
        c = c.copy()
        for g in (3, 9):
            c[:, 32 * g: 32 * g + 32] = _scaled_bits(c[:, 32 * g: 32 * g + 32], 2.0 ** -14)
        return c, r

    return _with_cache_transform(case, fn)


def _offset_case(H):
    """Latent channels 0..255 shifted by +64: INT4 zero points about 150 times
    their scale."""
    case = mla_synth.small_decode(case_id=65, H=H, seq_lens=[700, 130], normalise=False)

    def fn(b, c, r):
        x = mla_synth.bf16_bits_to_f32(c).copy()
        x[:, :256] += np.float32(64.0)
        return mla_synth.f32_to_bf16_bits(x), r

    return _with_cache_transform(case, fn)


@pytest.mark.parametrize("kind", ["shrunk", "tiny_groups", "offset"])
@pytest.mark.parametrize("cache_dtype", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("H", [16, 128])
def test_dequant_range(H, cache_dtype, kind):
    case = {"shrunk": _shrunk_case, "tiny_groups": _tiny_groups_case, "offset": _offset_case}[kind](H)
    if kind == "tiny_groups" and cache_dtype in (1, 2, 3, 6):
        f = quant.encode_tokens(cache_dtype, *case.seq_cache(0))
        amax_g = np.abs(quant.dequant_fields(cache_dtype, f)[0]).reshape(-1, 16, 32).max(axis=2)
        assert amax_g[:, 3].max() < 2.0 ** -7
    if kind == "offset" and cache_dtype == 2:
        f = quant.encode_tokens(cache_dtype, *case.seq_cache(0))
        assert np.median(np.abs(f["c_zero"][:, :8]) / f["c_scale"][:, :8]) > 100
    _note("dequant %s H=%d dtype=%d" % (kind, H, cache_dtype))
    _check(case, cache_dtype, chunk=4)


# ------------------------------------------------------------------ malformed work items
@pytest.mark.parametrize("H", [16, 128])
def test_item_range_past_the_table_is_empty(H):
    """Items whose first page lies past the block table (2^25: 32-bit token
    arithmetic would wrap negative there; and max_pages + 1) or past the
    sequence write o = 0 and lse = -inf; a normal item beside them is right."""
    case = mla_synth.small_decode(case_id=66, H=H, seq_lens=[200, 130])
    run, dev = upload(case)
    cfg = api.config(H)
    absorb = torch.empty(case.B, H, 576, dtype=torch.float16, device=DEV)
    api.absorb_q(cfg, dev["q_nope"], dev["q_pe"], dev["w_uk"], absorb)
    mp = case.max_pages
    items = torch.tensor([[0, 1 << 25, 4, 0],
                          [1, mp + 1, 2, 1],
                          [0, 3, 1, 2],                 # page 3 of a 4-page sequence: tokens 192..199
                          [1, 3, 1, 3],                 # page 3: past sequence 1's 130 tokens (pages 0-2)
                          [1, 0, (1 << 31) - 1, 4]],    # whole sequence 1, n_pages clipped
                         dtype=torch.int32, device=DEV)
    o_part = torch.full((5, H, 512), float("nan"), dtype=torch.float16, device=DEV)
    lse_part = torch.zeros(5, H, dtype=torch.float32, device=DEV)
    api.decode_attn(cfg, absorb, run.pool, dev["block_table"], dev["seq_lens"], items, o_part, lse_part)
    torch.cuda.synchronize()
    for row in (0, 1, 3):
        assert torch.all(o_part[row] == 0), row
        assert torch.all(torch.isneginf(lse_part[row])), row
    assert torch.isfinite(o_part[2]).all() and torch.isfinite(lse_part[2]).all()
    # row 4 is sequence 1's whole attention: compare its latent with the oracle
    _, ref_lse, ref_olat = oracle_seq(case, 1)
    mx, mean = errors(o_part[4].float().cpu().numpy(), ref_olat)
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    assert np.max(np.abs(lse_part[4].cpu().numpy() - ref_lse)) <= 1e-3 * max(1.0, np.abs(ref_lse).max())

"""Prefill attention (unabsorbed, causal) on the GPU against oracle.prefill.

Tolerance as for the decode: max|out - ref| <= 1e-2 max|ref| and
sum|out - ref| / sum|ref| <= 2e-3 per tensor, ref = the oracle's fp64 result
from the same bf16 inputs; lse within 1e-3 absolute (natural log).  Small cases
compare every row; the full-size prompts (4,096 positions) compare sampled rows,
each computed by the oracle over its own causal prefix.
"""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import DEV, MAX_REL, MEAN_REL, errors, to_dev_bits
from mla_absorbed_latent_amd import api
from oracle import mla_ref, prefill

pytestmark = pytest.mark.gpu


def _run(case):
    cfg = api.config(case.H, 0, case.softmax_scale)
    ws = torch.empty(api.prefill_workspace_bytes(cfg, case.L), dtype=torch.uint8, device=DEV)
    out = torch.empty(case.T, case.H, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(case.T, case.H, dtype=torch.float32, device=DEV)
    api.prefill_attn(cfg, to_dev_bits(case.q_nope), to_dev_bits(case.q_pe), to_dev_bits(case.c),
                     to_dev_bits(case.r), to_dev_bits(case.w_uk), to_dev_bits(case.w_uv), ws, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _oracle_rows(case, rows):
    """Oracle output of query rows `rows` (consecutive), over their causal prefix."""
    f = mla_ref.bf16_to_f64
    i0, i1 = rows[0], rows[-1] + 1
    L_sub = case.L - case.T + i1
    return prefill.prefill_unabsorbed(f(case.q_nope[i0:i1]), f(case.q_pe[i0:i1]), f(case.c[:L_sub]),
                                      f(case.r[:L_sub]), f(case.w_uk), f(case.w_uv), case.softmax_scale)


def _check(got, ref, got_lse, ref_lse, what):
    mx, mean = errors(got, ref)
    assert mx <= MAX_REL and mean <= MEAN_REL, (what, mx, mean)
    assert np.max(np.abs(got_lse - ref_lse)) <= 1e-3, (what, float(np.max(np.abs(got_lse - ref_lse))))


@pytest.mark.parametrize("T,L,H", [(1, 1, 16), (26, 26, 16), (64, 64, 16), (100, 300, 16), (5, 1000, 16),
                                   (300, 300, 16), (512, 600, 16), (77, 77, 128), (130, 200, 128), (1, 65, 128)])
def test_prefill_small(T, L, H):
    """Every row against the oracle.  T = 512 (four query blocks) and T = 130 at
    128 heads take the paired schedule (a work-group runs query blocks
    nqb - 1 - u and u), T = 300 (three blocks) the one-block-per-work-group one."""
    case = mla_synth.prefill_chunk(T, L, H, case_id=43)
    print("prefill T=%d L=%d H=%d" % (T, L, H), flush=True)
    out, lse = _run(case)
    ref, ref_lse = _oracle_rows(case, list(range(T)))
    _check(out, ref, lse, ref_lse, "all rows")


@pytest.mark.parametrize("name", ["v2lite_prefill", "v3_prefill"])
def test_prefill_full_size_sampled(name):
    case = getattr(mla_synth, name)()
    print("prefill %s T=%d H=%d" % (name, case.T, case.H), flush=True)
    out, lse = _run(case)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    T = case.T
    groups = [[0, 1, 2], [63, 64, 65], [T // 2 - 1, T // 2]] + ([[T - 2, T - 1]] if case.H == 16 else [])
    for rows in groups:
        ref, ref_lse = _oracle_rows(case, rows)
        _check(out[rows], ref, lse[rows], ref_lse, rows)


def test_prefill_matches_decode_of_the_last_position():
    """The last row of a chunk is the decode of that position: the prefill's
    unabsorbed kernels and the decode's absorbed kernels must agree (each within
    the tolerance of the oracle; here against each other)."""
    case = mla_synth.prefill_chunk(40, 300, 16, case_id=44)
    out, lse = _run(case)
    from gpu_case import DecodeRunner
    cfg = api.config(16, 0, case.softmax_scale)
    run = DecodeRunner(cfg, 1, 5, DEV)
    run.append(to_dev_bits(case.c), to_dev_bits(case.r), torch.arange(300, dtype=torch.int64, device=DEV))
    run.plan([300], chunk_pages=2)
    dec = run.step(to_dev_bits(case.q_nope[-1:]), to_dev_bits(case.q_pe[-1:]), to_dev_bits(case.w_uk),
                   to_dev_bits(case.w_uv), torch.arange(5, dtype=torch.int32, device=DEV)[None],
                   torch.tensor([300], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    d = dec.float().cpu().numpy()[0]
    mx, mean = errors(out[-1], d.astype(np.float64))
    assert mx <= 2 * MAX_REL and mean <= 2 * MEAN_REL, (mx, mean)
    assert np.max(np.abs(run.lse.cpu().numpy()[0] - lse[-1])) <= 2e-3

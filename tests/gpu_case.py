"""Helpers for the GPU tests: upload a seeded case through the C ABI and compute
the oracle's answer for chosen sequences.  The two sides meet only in the input
bits drawn by mla_synth."""
from __future__ import annotations

import numpy as np
import torch

import mla_synth
from mla_absorbed_latent_amd import api
from mla_absorbed_latent_amd.runner import DecodeRunner
from oracle import mla_ref, quant

DEV = "cuda:0"


def to_dev_bits(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bit patterns -> device tensor of a 2-byte dtype (bits unchanged)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dtype).to(DEV)


def upload(case: mla_synth.DecodeCase, cache_dtype: int = 0, block_table=None, append_batch: int = 1 << 18):
    """Fill a pool through mla_cache_append and upload queries, weights and tables."""
    cfg = api.config(case.H, cache_dtype, case.softmax_scale)
    run = DecodeRunner(cfg, case.B, case.num_pages, DEV)
    bt = case.block_table if block_table is None else block_table
    pend_c, pend_r, pend_s, n = [], [], [], 0

    def flush():
        nonlocal pend_c, pend_r, pend_s, n
        if not pend_c:
            return
        c = to_dev_bits(np.concatenate(pend_c))
        r = to_dev_bits(np.concatenate(pend_r))
        s = torch.from_numpy(np.concatenate(pend_s)).to(DEV)
        run.append(c, r, s)
        pend_c, pend_r, pend_s, n = [], [], [], 0

    for b in range(case.B):
        c, r = case.seq_cache(b)
        L = int(case.seq_lens[b])
        t = np.arange(L, dtype=np.int64)
        slots = bt[b, t // 64].astype(np.int64) * 64 + (t % 64)
        pend_c.append(c)
        pend_r.append(r)
        pend_s.append(slots)
        n += L
        if n >= append_batch:
            flush()
    flush()
    dev = {
        "q_nope": to_dev_bits(case.q_nope),
        "q_pe": to_dev_bits(case.q_pe),
        "w_uk": to_dev_bits(case.w_uk),
        "w_uv": to_dev_bits(case.w_uv),
        "block_table": torch.from_numpy(np.ascontiguousarray(bt)).to(DEV),
        "seq_lens": torch.from_numpy(case.seq_lens.astype(np.int32)).to(DEV),
    }
    return run, dev


def run_step(run: DecodeRunner, dev: dict, seq_lens, chunk_pages: int = 0, num_cus=None):
    run.plan(seq_lens, num_cus=num_cus, chunk_pages=chunk_pages)
    out = run.step(dev["q_nope"], dev["q_pe"], dev["w_uk"], dev["w_uv"], dev["block_table"], dev["seq_lens"])
    torch.cuda.synchronize()
    return out


def lse_bound(case: mla_synth.DecodeCase, b: int):
    """Per-head bound on |lse - lse_ref| for sequence b of a bf16 cache: the scores
    differ from the oracle's by the fp16 rounding of the absorbed query (at most
    2^-11 relative per element) and by fp32 accumulation, both within
    scale * 2^-10 * sum_c |q~_hc| |k_tc| for every token t, and a log-sum-exp moves
    by no more than its largest argument does."""
    c_bits, r_bits = case.seq_cache(b)
    if c_bits.shape[0] == 0:
        return np.zeros(case.H)
    keys = np.abs(np.concatenate([mla_ref.bf16_to_f64(c_bits), mla_ref.bf16_to_f64(r_bits)], axis=1))
    q = np.concatenate([mla_ref.absorb_q(mla_ref.bf16_to_f64(case.q_nope[b])[None], mla_ref.bf16_to_f64(case.w_uk))[0],
                        mla_ref.bf16_to_f64(case.q_pe[b])], axis=1)
    return case.softmax_scale * 2.0 ** -10 * (np.abs(q) @ keys.T).max(axis=1)


def oracle_seq(case: mla_synth.DecodeCase, b: int, cache_dtype: int = 0):
    """fp64 oracle for sequence b: (out [H,128], lse [H], o_lat [H,512])."""
    c_bits, r_bits = case.seq_cache(b)
    if cache_dtype == 0:
        c = mla_ref.bf16_to_f64(c_bits)
        r = mla_ref.bf16_to_f64(r_bits)
    else:
        f = quant.encode_tokens(cache_dtype, c_bits, r_bits)
        c32, r32 = quant.dequant_fields(cache_dtype, f)
        c, r = c32.astype(np.float64), r32.astype(np.float64)
    qn = mla_ref.bf16_to_f64(case.q_nope[b])
    qp = mla_ref.bf16_to_f64(case.q_pe[b])
    wk = mla_ref.bf16_to_f64(case.w_uk)
    wv = mla_ref.bf16_to_f64(case.w_uv)
    if c.shape[0] == 0:
        H = case.H
        return np.zeros((H, 128)), np.full(H, -np.inf), np.zeros((H, 512))
    return mla_ref.absorbed_decode(qn, qp, c, r, wk, wv, case.softmax_scale)


def errors(got: np.ndarray, ref: np.ndarray):
    """(max|d| / max|ref|, sum|d| / sum|ref|) -- the tolerance metrics."""
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-300)), float(d.sum() / max(np.abs(ref).sum(), 1e-300))


MAX_REL = 1e-2      # max|out - ref| <= 1e-2 * max|ref|
MEAN_REL = 2e-3     # sum|out - ref| / sum|ref| <= 2e-3

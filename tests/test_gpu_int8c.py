"""GPU parity of the per-channel INT8 cache over 32-token blocks (the report's
"per-channel INT8 (32 blocks)", "DeepSeek-V2-Lite MLA 吸收式 KV 缓存优化 — 完整实验报告"
§3.2/§4.1), through the C ABI, against the oracle's quantiser and decode.

Append: codes, channel scales, RoPE-key codes and scales bit-exact, and the open
block's bf16 rows bit-exact, whether a sequence arrives in one call (a prompt),
one position per call (decode steps) or in ragged chunks.  Decode: the output
within the usual tolerance of the oracle attending over the dequantised closed
blocks and the bf16 open block.
"""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import DEV, MAX_REL, MEAN_REL, errors, oracle_seq, run_step, to_dev_bits, upload
from mla_absorbed_latent_amd import api
from oracle import quant

pytestmark = pytest.mark.gpu

DT = quant.CACHE_INT8_CHAN
LENS = [1, 31, 32, 33, 64, 95, 130, 200]
CHUNKS = [10, 40, 17, 1, 5, 64, 33, 2]


def _append_calls(case, mode):
    """Lists of (sequence, first position, count) per call."""
    calls = []
    if mode == "one_call":
        calls.append([(b, 0, int(case.seq_lens[b])) for b in range(case.B)])
    elif mode == "token_by_token":
        for t in range(int(case.seq_lens.max())):
            calls.append([(b, t, 1) for b in range(case.B) if t < case.seq_lens[b]])
    else:
        pos = [0] * case.B
        k = 0
        while any(pos[b] < case.seq_lens[b] for b in range(case.B)):
            call = []
            for b in range(case.B):
                n = min(CHUNKS[(k + b) % len(CHUNKS)], int(case.seq_lens[b]) - pos[b])
                if n > 0:
                    call.append((b, pos[b], n))
                    pos[b] += n
            calls.append(call)
            k += 1
    return calls


@pytest.mark.parametrize("mode", ["one_call", "token_by_token", "chunks"])
def test_int8c_append_bitexact(mode):
    case = mla_synth.small_decode(case_id=70, H=16, seq_lens=LENS, paging="shuffled", normalise=False,
                                  outliers=True, extra_pages=2)
    cfg = api.config(16, DT)
    page = api.cache_page_bytes(cfg)
    pool = torch.zeros(case.num_pages * page, dtype=torch.uint8, device=DEV)
    data = [case.seq_cache(b) for b in range(case.B)]
    slots = [case.slots_of(b) for b in range(case.B)]
    calls = _append_calls(case, mode)
    print("int8c append %s: %d calls" % (mode, len(calls)), flush=True)
    for call in calls:
        c = np.concatenate([data[b][0][t: t + n] for b, t, n in call])
        r = np.concatenate([data[b][1][t: t + n] for b, t, n in call])
        s = np.concatenate([slots[b][t: t + n] for b, t, n in call])
        api.cache_append(cfg, pool, to_dev_bits(c), to_dev_bits(r), torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    pages = pool.cpu().numpy().reshape(case.num_pages, page)
    for b in range(case.B):
        L = int(case.seq_lens[b])
        c, r = data[b]
        for p0 in range(0, L, 64):
            n = min(64, L - p0)
            got = quant.page_fields_int8_chan(pages[int(case.block_table[b, p0 // 64])], n)
            ref = quant.encode_tokens(DT, c[p0: p0 + n], r[p0: p0 + n])
            for k in ("codes", "blk_scale", "r_codes", "r_scale", "open"):
                assert np.array_equal(got[k], ref[k]), (mode, b, p0, k)


DEC_LENS = [1, 31, 32, 33, 64, 95, 96, 130, 200, 2000]


@pytest.mark.parametrize("chunk", [0, 1, 3])
@pytest.mark.parametrize("H", [16, 128])
def test_int8c_decode_small(H, chunk):
    """Closed blocks only, open block only, a closed and an open block on one
    page (33, 95, 130, 200), and work items of one page (chunk 1) that hold only
    a closed or only an open block."""
    case = mla_synth.small_decode(case_id=71, H=H, seq_lens=DEC_LENS, paging="shuffled", normalise=False,
                                  outliers=True)
    print("int8c decode H=%d chunk=%d" % (H, chunk), flush=True)
    run, dev = upload(case, DT)
    out = run_step(run, dev, case.seq_lens, chunk_pages=chunk).float().cpu().numpy()
    for b in range(case.B):
        ref_out, _, _ = oracle_seq(case, b, DT)
        mx, mean = errors(out[b], ref_out)
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, int(case.seq_lens[b]), mx, mean)


@pytest.mark.parametrize("H", [16, 128])
def test_int8c_decode_after_token_steps(H):
    """The cache filled one position per call, as decode steps write it, gives
    the same output, bit for bit, as the cache written by one prompt call."""
    case = mla_synth.small_decode(case_id=72, H=H, seq_lens=[33, 64, 100], paging="shuffled")
    run, dev = upload(case, DT)
    ref = run_step(run, dev, case.seq_lens, chunk_pages=1).clone()
    run.pool.zero_()
    for t in range(int(case.seq_lens.max())):
        bs = [b for b in range(case.B) if t < case.seq_lens[b]]
        c = np.stack([case.seq_cache(b)[0][t] for b in bs])
        r = np.stack([case.seq_cache(b)[1][t] for b in bs])
        s = np.array([case.slots_of(b)[t] for b in bs], np.int64)
        run.append(to_dev_bits(c), to_dev_bits(r), torch.from_numpy(s).to(DEV))
    out = run_step(run, dev, case.seq_lens, chunk_pages=1)
    assert torch.equal(out, ref)


@pytest.mark.parametrize("H", [16, 128])
def test_int8c_full_size_sampled(H):
    case = mla_synth.v2lite_quant() if H == 16 else mla_synth.v3_decode()
    print("int8c full H=%d B=%d tokens=%d" % (H, case.B, case.total_tokens), flush=True)
    run, dev = upload(case, DT)
    out = run_step(run, dev, case.seq_lens).float().cpu().numpy()
    lens = case.seq_lens
    for b in sorted({0, case.B // 2, case.B - 1, int(np.argmax(lens)), int(np.argmin(lens))}):
        ref_out, _, _ = oracle_seq(case, b, DT)
        mx, mean = errors(out[b], ref_out)
        print("  seq %d L=%d max_rel %.2e mean_rel %.2e" % (b, lens[b], mx, mean), flush=True)
        assert mx <= MAX_REL and mean <= MEAN_REL, (b, mx, mean)
    assert np.isfinite(out).all()

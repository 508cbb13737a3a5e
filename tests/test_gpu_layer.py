"""The layer front on the GPU and one whole V2-Lite layer through the C ABI.

Chunks under 64 tokens (or a width that is not a multiple of 64) take the
vector-ALU projection, longer ones the matrix-core GEMM; both are covered.

mla_layer_front (projections, RMSNorm, RoPE) is compared with oracle.layer's
layer_front element by element.  Both sides round each output once to bf16; the
GPU's projection sums are fp32 where the oracle's are fp64, so an element may
land one bf16 step away: |got - ref| <= 2^-7 |ref| + 1e-5 per element, and the
usual output tolerance (max|d| <= 1e-2 max|ref|, sum|d| / sum|ref| <= 2e-3) on
each tensor.

The layer test runs the V2-Lite layer of 26 tokens (25 prefill + the decoded
one) wholly on the GPU: front -> cache append of all 26 rows -> absorb the last
token's query -> decode -> merge + W_UV -> W_O, and compares y with the
oracle's layer_decode (its own front, absorbed and unabsorbed forms).
"""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import DEV, MAX_REL, MEAN_REL, errors, to_dev_bits
from mla_absorbed_latent_amd import api
from mla_absorbed_latent_amd.runner import DecodeRunner
from oracle import layer, mla_ref

pytestmark = pytest.mark.gpu


def _gpu_front(case, cache_dtype=0):
    T, H = case.T, case.H
    cfg = api.config(H, cache_dtype, case.softmax_scale)
    ws = torch.empty(api.layer_front_workspace_bytes(cfg, T) // 4, dtype=torch.float32, device=DEV)
    outs = (torch.empty(T, H, 128, dtype=torch.bfloat16, device=DEV),
            torch.empty(T, H, 64, dtype=torch.bfloat16, device=DEV),
            torch.empty(T, 512, dtype=torch.bfloat16, device=DEV),
            torch.empty(T, 64, dtype=torch.bfloat16, device=DEV))
    pos = torch.arange(T, dtype=torch.int32, device=DEV)
    api.layer_front(cfg, to_dev_bits(case.x), to_dev_bits(case.w_q), to_dev_bits(case.w_dkv), pos, ws, *outs,
                    rms_eps=case.rms_eps, rope_base=case.rope_base)
    return cfg, outs


@pytest.mark.parametrize("T,H,hidden", [(26, 16, 2048), (1, 16, 2048), (17, 16, 520), (40, 128, 1024),
                                          (200, 16, 2048), (64, 128, 1024), (100, 16, 520)])
def test_layer_front(T, H, hidden):
    case = mla_synth.v2lite_layer(T=T, H=H, hidden=hidden, case_id=31)
    print("front T=%d H=%d hidden=%d" % (T, H, hidden), flush=True)
    _, outs = _gpu_front(case)
    torch.cuda.synchronize()
    refs = layer.layer_front(case)
    for name, g, r in zip(("q_nope", "q_pe", "c_kv", "k_pe"), outs, refs):
        got = g.float().cpu().numpy().astype(np.float64)
        ref = mla_ref.bf16_to_f64(r)
        assert got.shape == ref.shape, name
        d = np.abs(got - ref)
        bad = d > 2.0 ** -7 * np.abs(ref) + 1e-5
        assert not bad.any(), (name, int(bad.sum()), float(d.max()))
        mx, mean = errors(got, ref)
        assert mx <= MAX_REL and mean <= MEAN_REL, (name, mx, mean)
    # RMSNorm has unit gain: every latent row has RMS 1 up to bf16 rounding.
    c = outs[2].float().cpu().numpy().astype(np.float64)
    assert np.allclose(np.sqrt((c * c).mean(axis=1)), 1.0, atol=4e-3)


@pytest.mark.parametrize("fused", [True, False])
def test_v2lite_layer_end_to_end(fused):
    case = mla_synth.v2lite_layer()
    T, H = case.T, case.H
    print("layer T=%d H=%d fused=%s" % (T, H, fused), flush=True)
    cfg, (qn, qp, c, r) = _gpu_front(case)
    run = DecodeRunner(cfg, 1, 1, DEV)
    run.append(c, r, torch.arange(T, dtype=torch.int64, device=DEV))
    run.plan([T], chunk_pages=0)
    y = torch.empty(1, case.hidden, dtype=torch.bfloat16, device=DEV)
    of = torch.empty(1, H, 128, dtype=torch.float32, device=DEV)
    run.step(qn[T - 1:].contiguous(), qp[T - 1:].contiguous(), to_dev_bits(case.w_uk), to_dev_bits(case.w_uv),
             torch.zeros(1, 1, dtype=torch.int32, device=DEV), torch.tensor([T], dtype=torch.int32, device=DEV),
             w_o=to_dev_bits(case.w_o), y=y, out_f32=of, fused=fused)
    torch.cuda.synchronize()
    ref = layer.layer_decode(case)
    got = y.float().cpu().numpy()[0]
    for key in ("y_absorbed", "y_unabsorbed"):
        mx, mean = errors(got, ref[key])
        assert mx <= MAX_REL and mean <= MEAN_REL, (key, mx, mean)
    mx, mean = errors(of.cpu().numpy()[0], ref["out_absorbed"])
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)


@pytest.mark.parametrize("cache_dtype", [0, 1, 2, 3, 4, 5, 6, 7])
def test_layer_front_append_matches_front_then_append(cache_dtype):
    """mla_layer_front_append against mla_layer_front followed by
    mla_cache_append: every output and every pool byte equal, over two calls
    (positions 0..44, then 45..99: the second call finishes blocks the first one
    opened and takes the matrix-core projection), pages shuffled, one slot
    outside the pool (skipped by both)."""
    H, T = 16, 100
    case = mla_synth.v2lite_layer(T=T, H=H, hidden=2048, case_id=32)
    cfg = api.config(H, cache_dtype, case.softmax_scale)
    page = api.cache_page_bytes(cfg)
    perm = [2, 0, 3, 1]
    slots_all = np.array([perm[p // 64] * 64 + p % 64 for p in range(T)], np.int64)
    slots_all[7] = 4 * 64 + 3                        # past the 4-page pool
    pools = [torch.zeros(4 * page, dtype=torch.uint8, device=DEV) for _ in range(2)]
    x_all = to_dev_bits(case.x)
    w_q, w_dkv = to_dev_bits(case.w_q), to_dev_bits(case.w_dkv)
    print("front+append dtype=%d" % cache_dtype, flush=True)
    for t0, t1 in ((0, 45), (45, T)):
        n = t1 - t0
        x = x_all[t0:t1].contiguous()
        pos = torch.arange(t0, t1, dtype=torch.int32, device=DEV)
        slots = torch.from_numpy(slots_all[t0:t1].copy()).to(DEV)
        ws = torch.empty(api.layer_front_workspace_bytes(cfg, n) // 4, dtype=torch.float32, device=DEV)
        outs = []
        for k in range(2):
            o = (torch.empty(n, H, 128, dtype=torch.bfloat16, device=DEV),
                 torch.empty(n, H, 64, dtype=torch.bfloat16, device=DEV),
                 torch.empty(n, 512, dtype=torch.bfloat16, device=DEV),
                 torch.empty(n, 64, dtype=torch.bfloat16, device=DEV))
            if k == 0:
                api.layer_front(cfg, x, w_q, w_dkv, pos, ws, *o, rms_eps=case.rms_eps, rope_base=case.rope_base)
                api.cache_append(cfg, pools[0], o[2], o[3], slots)
            else:
                api.layer_front_append(cfg, x, w_q, w_dkv, pos, ws, *o, pools[1], slots, rms_eps=case.rms_eps,
                                       rope_base=case.rope_base)
            outs.append(o)
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(pools[0], pools[1]), (t0, int((pools[0] != pools[1]).sum()))
    assert bool(pools[1].any())

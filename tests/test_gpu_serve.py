"""A prompt followed by one decode step through a stack of three V2-Lite layers,
wholly on the GPU, against the stack oracle.

Per layer: the prompt (T = 48 tokens) runs the prompt path
(mla_layer_front_append, which also writes its latent rows into the layer's
paged cache -> mla_prefill_attn -> mla_out_residual); the next token then runs the decode path at position T
(mla_layer_front for one token -> mla_cache_append -> mla_absorb_q ->
mla_decode_attn -> merge + W_UV -> mla_out_residual).  Attention is causal, so
the oracle stack over T + 1 tokens gives both: rows 0..T-1 for the prompt and
row T for the decoded token.  This checks that the two attention forms and the
cache handed between them agree across layers.  Drift bounds as in
test_gpu_stack.py for a bf16 cache; with an INT8 cache the decoded token's
bound allows for the quantisation error.
"""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import DEV, to_dev_bits
from mla_absorbed_latent_amd import api
from mla_absorbed_latent_amd.runner import DecodeRunner, PrefillLayer
from oracle import mla_ref, stack

pytestmark = pytest.mark.gpu


def _drift(got, ref, base, l):
    upd = np.abs(ref - base)
    d = np.abs(got - ref)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(d <= (l + 1) * (ulp + 1e-2 * upd.max())), l
    return d.sum() / upd.sum()


@pytest.mark.parametrize("cache_dtype", [0, 1])
def test_prompt_then_decode_through_three_layers(cache_dtype):
    T, n_layers = 48, 3
    x_all, layers = mla_synth.v2lite_stack(n_layers=n_layers, T=T + 1)
    refs = stack.run_stack(x_all, layers)
    H, hidden = 16, 2048
    cfg = api.config(H, cache_dtype, layers[0].softmax_scale)
    prompt = PrefillLayer(api.config(H, 0, layers[0].softmax_scale), T, hidden, DEV)
    x_p = to_dev_bits(x_all[:T])
    x_d = to_dev_bits(x_all[T:])
    pages = (T + 1 + 63) // 64
    bt = torch.arange(pages, dtype=torch.int32, device=DEV)[None]
    lens = torch.tensor([T + 1], dtype=torch.int32, device=DEV)
    fws = torch.empty(api.layer_front_workspace_bytes(cfg, 1) // 4, dtype=torch.float32, device=DEV)
    rws = torch.empty(hidden, dtype=torch.float32, device=DEV)
    qn = torch.empty(1, H, 128, dtype=torch.bfloat16, device=DEV)
    qp = torch.empty(1, H, 64, dtype=torch.bfloat16, device=DEV)
    c1 = torch.empty(1, 512, dtype=torch.bfloat16, device=DEV)
    r1 = torch.empty(1, 64, dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([T], dtype=torch.int32, device=DEV)
    base_p = mla_ref.bf16_to_f64(x_all[:T])
    base_d = mla_ref.bf16_to_f64(x_all[T:])
    for l, case in enumerate(layers):
        w = [to_dev_bits(a) for a in (case.w_q, case.w_dkv, case.w_uk, case.w_uv, case.w_o)]
        run = DecodeRunner(cfg, 1, pages, DEV)
        # prompt: prefill path; its latent rows go to this layer's cache from the
        # front's own launch (mla_layer_front_append)
        prompt.forward(x_p, *w, x_p, cache=run, slots=torch.arange(T, dtype=torch.int64, device=DEV))
        # decode: one token at position T through the absorbed path
        api.layer_front(cfg, x_d, w[0], w[1], pos, fws, qn, qp, c1, r1)
        run.plan([T + 1])
        out = run.step(qn, qp, w[2], w[3], bt, lens, new_c_kv=c1, new_k_pe=r1,
                       new_slots=torch.tensor([T], dtype=torch.int64, device=DEV))
        api.out_residual(cfg, out, w[4], x_d, x_d, rws)
        torch.cuda.synchronize()
        got_p = x_p.float().cpu().numpy().astype(np.float64)
        got_d = x_d.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(got_d).all()
        ref = mla_ref.bf16_to_f64(refs[l])
        mp = _drift(got_p, ref[:T], base_p, l)
        if cache_dtype == 0:
            md = _drift(got_d, ref[T:], base_d, l)
            assert md <= 4e-3 * (l + 1), (l, md)
        else:
            # the decoded token reads an INT8 cache: its drift includes the
            # quantisation error of the latent rows (about 1 % per element)
            upd = np.abs(ref[T:] - base_d)
            md = np.abs(got_d - ref[T:]).sum() / upd.sum()
            assert md <= 3e-2 * (l + 1), (l, md)
        print("layer %d: prompt drift %.2e, decoded token drift %.2e" % (l, mp, md), flush=True)
        assert mp <= 2e-3 * (l + 1), (l, mp)

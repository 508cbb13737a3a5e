"""A stack of four V2-Lite layers (64 positions, residual connections) on the
GPU against oracle.stack, layer by layer.

Both sides hand each layer a bf16 input; the GPU's attention output is also
rounded to bf16 before W_O and its sums are fp32, so the two sums a layer
rounds differ slightly and now and then round to neighbouring bf16 values.
After layer l (0-based) the drift d = x_gpu - x_ref must stay within: per
element, l + 1 bf16 steps of x_ref plus 1e-2 (l + 1) max|x_l - x_0| (the output
tolerance on the accumulated updates); in sum, sum|d| / sum|x_l - x_0| <=
2e-3 (l + 1).
"""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import DEV, to_dev_bits
from mla_absorbed_latent_amd import api
from mla_absorbed_latent_amd.runner import PrefillLayer
from oracle import mla_ref, stack

pytestmark = pytest.mark.gpu


def test_four_layer_stack():
    x0, layers = mla_synth.v2lite_stack(n_layers=4, T=64)
    refs = stack.run_stack(x0, layers)
    cfg = api.config(16, 0, layers[0].softmax_scale)
    run = PrefillLayer(cfg, 64, 2048, DEV)
    x = to_dev_bits(x0)
    base = mla_ref.bf16_to_f64(x0)
    for l, case in enumerate(layers):
        run.forward(x, to_dev_bits(case.w_q), to_dev_bits(case.w_dkv), to_dev_bits(case.w_uk),
                    to_dev_bits(case.w_uv), to_dev_bits(case.w_o), x)
        torch.cuda.synchronize()
        got = x.float().cpu().numpy().astype(np.float64)
        ref = mla_ref.bf16_to_f64(refs[l])
        upd = np.abs(ref - base)
        d = np.abs(got - ref)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        mean_rel = d.sum() / upd.sum()
        print("layer %d: sum|d|/sum|upd| %.2e  max|d|/max|upd| %.2e" % (l, mean_rel, d.max() / upd.max()), flush=True)
        assert np.all(d <= (l + 1) * (ulp + 1e-2 * upd.max())), l
        assert mean_rel <= 2e-3 * (l + 1), (l, mean_rel)

"""mla_layer_front_noalloc against mla_layer_front, through the C ABI: the same
kernels over the library's own scratch instead of a caller workspace, so every
output must be bitwise equal.  Two calls in a row, the second with fewer tokens
(the scratch keeps the first call's contents), at H = 16 and H = 128; the
largest token count the scratch holds works and one more is rejected."""
import numpy as np
import pytest
import torch

import mla_synth
from gpu_case import DEV, to_dev_bits
from mla_absorbed_latent_amd import api
from mla_absorbed_latent_amd._lib import MLA_ERR_WORKSPACE

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20


def _max_tokens(H):
    return SCRATCH // ((576 + H * 192) * 4)


def _outputs(T, H):
    return [torch.empty(T, H, 128, dtype=torch.bfloat16, device=DEV),
            torch.empty(T, H, 64, dtype=torch.bfloat16, device=DEV),
            torch.empty(T, 512, dtype=torch.bfloat16, device=DEV),
            torch.empty(T, 64, dtype=torch.bfloat16, device=DEV)]


def _both(cfg, layer, T, H, w_q, w_dkv):
    x = to_dev_bits(layer.x[:T])
    pos = torch.arange(3, 3 + T, dtype=torch.int32, device=DEV)
    ws = torch.empty(api.layer_front_workspace_bytes(cfg, T) // 4, dtype=torch.float32, device=DEV)
    ref = _outputs(T, H)
    got = [t.fill_(7.0) for t in _outputs(T, H)]
    api.layer_front(cfg, x, w_q, w_dkv, pos, ws, *ref)
    api.layer_front_noalloc(cfg, x, w_q, w_dkv, pos, *got)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r.view(torch.int16), g.view(torch.int16))
    return got


@pytest.mark.parametrize("H", [16, 128])
def test_noalloc_front_matches_the_workspace_front(H):
    T_max = _max_tokens(H)
    layer = mla_synth.v2lite_layer(T=T_max + 1, H=H, case_id=80 + H)
    cfg = api.config(H)
    w_q, w_dkv = to_dev_bits(layer.w_q), to_dev_bits(layer.w_dkv)
    print("noalloc H=%d T=%d then 9 then %d" % (H, 100, T_max), flush=True)
    _both(cfg, layer, 100, H, w_q, w_dkv)                  # matrix-core projections
    _both(cfg, layer, 9, H, w_q, w_dkv)                    # fewer tokens (vector-ALU projections)
    _both(cfg, layer, T_max, H, w_q, w_dkv)                # the largest count the scratch holds
    x = to_dev_bits(layer.x[:T_max + 1])
    pos = torch.arange(T_max + 1, dtype=torch.int32, device=DEV)
    with pytest.raises(api.MlaError) as e:
        api.layer_front_noalloc(cfg, x, w_q, w_dkv, pos, *_outputs(T_max + 1, H))
    assert e.value.status == MLA_ERR_WORKSPACE

"""Pins of the layer-stack oracle (oracle/stack.py), CPU only.

Special cases: a layer whose W_O is zero passes its input through unchanged
(the residual path); the first position attends only to itself, so its update
is W_O applied to each head's W_UV c_0.  Cross-check with an independent path:
the last position's update equals W_O applied to the absorbed decode of that
position (oracle.layer.layer_decode, pinned by the two decode forms agreeing).
"""
import dataclasses

import numpy as np

import mla_synth
from oracle import layer, mla_ref, stack


def test_zero_output_projection_is_identity():
    x, layers = mla_synth.v2lite_stack(n_layers=2, T=6)
    zero = [dataclasses.replace(c, w_o=np.zeros_like(c.w_o)) for c in layers]
    xs = stack.run_stack(x, zero)
    assert all(np.array_equal(a, x) for a in xs)


def test_first_and_last_positions():
    x, (case,) = mla_synth.v2lite_stack(n_layers=1, T=7)
    y = stack.layer_update(case, x)
    f = mla_ref.bf16_to_f64
    _, _, c, _ = layer.layer_front(case)
    v0 = np.einsum("hdc,c->hd", f(case.w_uv), f(c)[0])
    assert np.allclose(y[0], mla_ref.wo_proj(v0, f(case.w_o)), rtol=1e-10, atol=1e-12)
    ref = layer.layer_decode(case)["y_absorbed"]
    assert np.allclose(y[-1], ref, rtol=1e-9, atol=1e-11)


def test_stack_feeds_each_layer_the_rounded_sum():
    x, layers = mla_synth.v2lite_stack(n_layers=2, T=5)
    xs = stack.run_stack(x, layers)
    y1 = stack.layer_update(layers[1], xs[0])
    assert np.array_equal(xs[1], layer._to_bf16_bits(mla_ref.bf16_to_f64(xs[0]) + y1))
    assert not np.array_equal(xs[0], x)

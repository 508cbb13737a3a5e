"""Oracle: a stack of MLA layers with residual connections.  Test
infrastructure only.

Each layer runs its front (oracle.layer.layer_front: projections, RMSNorm,
RoPE, outputs rounded to bf16), causal attention over all T positions in the
unabsorbed form (oracle.prefill, fp64), the output projection W_O (fp64), and
adds the result to its input; the sum is rounded to bf16, which is the next
layer's input.  Reading where the pages are silent (R23): attention and W_O
form the whole layer (no MLP, no norm on the residual path); the rounding
points are the bf16 tensors a layer hands on.

This is the multi-layer stacking that the pages name as unvalidated
([Tutorial] §六: validated on layer 0 only; [Audit] §9 lists stacking as a next
step): it measures how the GPU path's rounding accumulates over layers.

Pins (tests/test_oracle_stack.py): zero layers and W_O = 0 leave x unchanged;
the last position's update equals W_O applied to the decode oracle's
absorbed result for that position (oracle.layer.layer_decode).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .layer import _to_bf16_bits, layer_front
from .mla_ref import bf16_to_f64, wo_proj
from .prefill import prefill_unabsorbed


def layer_update(case, x_bits):
    """One layer's output y [T, hidden] (fp64, before the residual) for input x."""
    qn, qp, c, r = (bf16_to_f64(a) for a in layer_front(dataclasses.replace(case, x=x_bits)))
    out, _ = prefill_unabsorbed(qn, qp, c, r, bf16_to_f64(case.w_uk), bf16_to_f64(case.w_uv),
                                case.softmax_scale)
    return wo_proj(out, bf16_to_f64(case.w_o))


def run_stack(x_bits, layers):
    """Hidden states after each layer: list of bf16 bit arrays [T, hidden]."""
    xs = []
    x = x_bits
    for case in layers:
        y = layer_update(case, x)
        x = _to_bf16_bits(bf16_to_f64(x) + y)
        xs.append(x)
    return xs

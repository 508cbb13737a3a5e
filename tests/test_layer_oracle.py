"""The single-layer oracle (V2-Lite shapes, 25-token prefill + 1 decode token).

The layer front (projections, RMSNorm, RoPE) has no printed values for synthetic
weights, so it is pinned by properties only; the decode is pinned by the two
forms agreeing (absorbed == unabsorbed, [Audit] "DeepSeek MLA 吸收式缓存：真实权重执行与
FlashMLA 架构边界" §2.2/§2.3)."""
import numpy as np
import pytest

import mla_synth
from oracle import layer, mla_ref


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 64))
    y = layer.rope_interleaved(x, np.zeros(5))
    assert np.array_equal(y, x)
    y = layer.rope_interleaved(x, np.arange(5) * 7)
    pn = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2
    assert np.allclose(pn(y), pn(x), rtol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    def score(m, n):
        return float(layer.rope_interleaved(q, np.array([m]))[0] @ layer.rope_interleaved(k, np.array([n]))[0])
    assert score(10, 3) == pytest.approx(score(7, 0), rel=1e-12)
    assert score(25, 25) == pytest.approx(float(q[0] @ k[0]), rel=1e-12)


def test_rope_pairs_adjacent_channels():
    """Interleaved convention: channel 0 and 1 rotate together at frequency 1."""
    x = np.zeros((1, 64))
    x[0, 0] = 1.0
    y = layer.rope_interleaved(x, np.array([1.0]))
    assert y[0, 0] == pytest.approx(np.cos(1.0)) and y[0, 1] == pytest.approx(np.sin(1.0))
    assert np.count_nonzero(y) == 2


def test_rmsnorm_unit_rms():
    rng = np.random.default_rng(2)
    x = 3 * rng.standard_normal((4, 512))
    y = layer.rmsnorm(x)
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), 1.0, atol=1e-6)


def test_layer_decode_two_forms_agree():
    case = mla_synth.v2lite_layer()
    res = layer.layer_decode(case)
    ya, yu = res["y_absorbed"], res["y_unabsorbed"]
    assert ya.shape == (2048,)
    assert np.max(np.abs(ya - yu)) <= 1e-12 * np.max(np.abs(yu))
    # the decoded token attends to 26 cached positions (25 prefill + itself)
    qn, qp, c, r = layer.layer_front(case)
    assert c.shape == (26, 512) and r.shape == (26, 64)
    assert qn.shape == (26, 16, 128) and qp.shape == (26, 16, 64)

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


def _pair_angles(pos):
    """Angle each of the 32 pairs turns through at position `pos`, read back from
    the rotation of unit vectors (atan2 of the rotated pair)."""
    x = np.zeros((32, 64))
    for i in range(32):
        x[i, 2 * i] = 1.0
    y = layer.rope_interleaved(x[:, None, :], np.full(32, float(pos)))[:, 0, :]
    return np.array([np.arctan2(y[i, 2 * i + 1], y[i, 2 * i]) for i in range(32)])


def test_rope_frequencies_at_round_decades():
    """The frequency ladder of a 64-wide RoPE key with base 10000 spans four
    decades over its 32 pairs: pairs 0, 8, 16 and 24 turn by exactly 1, 0.1,
    0.01 and 0.001 rad per position.  A wrong exponent (e.g. -i/d instead of
    -2i/d) puts pair 16 at 0.1 rad and fails here."""
    ang = _pair_angles(1)
    for pair, rad in ((0, 1.0), (8, 0.1), (16, 0.01), (24, 0.001)):
        assert ang[pair] == pytest.approx(rad, rel=1e-12), (pair, ang[pair])
    # position 100: pair 16 turns through 1 rad, pair 24 through 0.1 rad
    ang = _pair_angles(100)
    assert ang[16] == pytest.approx(1.0, rel=1e-12)
    assert ang[24] == pytest.approx(0.1, rel=1e-12)
    # neighbouring pairs differ by one eighth of a decade
    ang = _pair_angles(1)
    assert np.allclose(ang[1:] / ang[:-1], 10.0 ** -0.125, rtol=1e-12)


def test_wo_orientation_on_a_non_square_projection():
    """W_O [hidden][H*128] with hidden != H*128: a one-hot W_O routes one head
    feature to one output channel, which fixes both the orientation and the
    head-major flattening (feature d of head h is column 128 h + d)."""
    H, hidden = 16, 520
    out = np.arange(H * 128, dtype=np.float64).reshape(H, 128) + 1.0
    w_o = np.zeros((hidden, H * 128))
    w_o[7, 128 * 3 + 5] = 1.0          # y[7] = out[head 3, feature 5]
    w_o[519, 128 * 15 + 127] = 2.0     # y[519] = 2 * out[head 15, feature 127]
    y = mla_ref.wo_proj(out, w_o)
    assert y.shape == (hidden,)
    assert y[7] == out[3, 5] and y[519] == 2.0 * out[15, 127]
    assert np.count_nonzero(y) == 2
    # batched form keeps the leading axes
    yb = mla_ref.wo_proj(np.stack([out, -out]), w_o)
    assert yb.shape == (2, hidden) and yb[1, 7] == -out[3, 5]


def test_rmsnorm_epsilon_inside_the_root():
    """A constant row c gives c / sqrt(c^2 + eps): with c = 1e-3 and eps = 1e-6
    that is 1 / sqrt(2), which places eps inside the square root and fixes its
    value."""
    y = layer.rmsnorm(np.full((1, 512), 1e-3), 1e-6)
    assert np.allclose(y, 2.0 ** -0.5, rtol=1e-12)


def test_front_projection_orientation_and_head_split():
    """A one-hot hidden state x = e_j picks column j of every projection: the
    query of head h is W_q[192 h : 192 h + 192, j] (128 no-RoPE values then 64
    RoPE values), the latent is W_DKV[0:512, j] (RMS-normalised) and the RoPE key
    W_DKV[512:576, j].  At position 0 RoPE is the identity, so these hold
    exactly up to the one bf16 rounding."""
    case = mla_synth.v2lite_layer(T=2)
    j = 37
    x = np.zeros((2, case.hidden), np.float32)
    x[0, j] = 1.0
    x[1, j] = 1.0
    case.x = mla_synth.f32_to_bf16_bits(x)
    qn, qp, c, r = layer.layer_front(case)
    wq = mla_ref.bf16_to_f64(case.w_q)
    wd = mla_ref.bf16_to_f64(case.w_dkv)
    bf = lambda a: mla_ref.bf16_to_f64(mla_synth.f32_to_bf16_bits(np.asarray(a, np.float32)))
    for h in (0, 5, 15):
        assert np.array_equal(mla_ref.bf16_to_f64(qn[0, h]), bf(wq[192 * h: 192 * h + 128, j]))
        assert np.array_equal(mla_ref.bf16_to_f64(qp[0, h]), bf(wq[192 * h + 128: 192 * h + 192, j]))
    lat = wd[:512, j]
    assert np.array_equal(mla_ref.bf16_to_f64(c[0]), bf(lat / np.sqrt(np.mean(lat * lat) + case.rms_eps)))
    assert np.array_equal(mla_ref.bf16_to_f64(r[0]), bf(wd[512:, j]))
    # position 1 rotates pair 0 of the RoPE key by 1 rad
    k = wd[512:, j]
    want0 = k[0] * np.cos(1.0) - k[1] * np.sin(1.0)
    assert mla_ref.bf16_to_f64(r[1, 0]) == bf(want0)

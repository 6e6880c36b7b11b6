"""Pins of the oracle's square-block comparator (§III-C: the method of [25]
extended to convolution, X' quantized once in square blocks after im2col and
saved) and of the per-element activation MSE of Table II (§IV-D)."""
import numpy as np
import pytest

import oracle
from microscaling_quantized_convolution_mxq_amd.workloads import ConvShape

from test_oracle_layout_conv import SMALL, _lossless


@pytest.mark.parametrize("shape", SMALL)
def test_cuyckens_on_lossless_inputs_equals_exact_conv(shape):
    x, w, dy = _lossless(shape, 11)
    xc, xs, n = oracle.cuyckens_im2col_quantize(shape, x, 0)
    assert n == shape.ho * shape.wo * shape.n * shape.cin * shape.kh * shape.kw
    y, _ = oracle.cuyckens_fwd(shape, xc, xs, w, 0, 0)
    np.testing.assert_allclose(y, oracle.conv_fwd(shape, x.astype(np.float64), w.astype(np.float64)),
                               rtol=1e-12, atol=1e-12)
    dx, _ = oracle.cuyckens_dgrad(shape, dy, w, 1, 0)
    np.testing.assert_allclose(dx, oracle.conv_dgrad(shape, dy.astype(np.float64), w.astype(np.float64)),
                               rtol=1e-12, atol=1e-12)
    dw, _ = oracle.cuyckens_wgrad(shape, dy, xc, xs, 1, 0)
    np.testing.assert_allclose(dw, oracle.conv_wgrad(shape, dy.astype(np.float64), x.astype(np.float64)),
                               rtol=1e-12, atol=1e-12)


def test_cuyckens_square_blocks_hand_worked():
    """1x1 convolution with M = K = 64 (two 32-blocks along each direction) and
    Cout = 32: X' holds 256 at [0][0] and a = 1.5 * 2^-12 elsewhere, W is all
    ones, E4M3. The square [0:32][0:32] has shared exponent 0, where a lies
    below half the smallest subnormal and becomes 0; the three other squares
    keep a exactly (exponent -20, a * 2^20 = 384). So Y = 256 + 32a on row 0,
    32a on rows 1..31 (their first K-block is zero) and 64a on rows 32..63;
    line blocks along k would instead give 64a on rows 1..31."""
    a = 1.5 * 2.0 ** -12
    s = ConvShape(1, 64, 1, 64, 32, 1, 1, 1, 0)
    xm = np.full((64, 64), a)
    xm[0, 0] = 256.0
    x = xm.reshape(1, 64, 1, 64).astype(np.float32)
    w = np.ones((32, 1, 1, 64), np.float32)
    xc, xs, _ = oracle.cuyckens_im2col_quantize(s, x, 0)
    y, _ = oracle.cuyckens_fwd(s, xc, xs, w, 0, 0)
    y = y.reshape(64, 32)
    np.testing.assert_array_equal(y[0], 256.0 + 32 * a)
    np.testing.assert_array_equal(y[1:32], 32 * a)
    np.testing.assert_array_equal(y[32:], 64 * a)


def test_cuyckens_counts_table1():
    """Table I, Cuyckens column, 3x3 stride 1 same padding: each activation
    element is quantized 9 times (once per copy in X'), weights and gradients
    once."""
    s = ConvShape(2, 8, 6, 6, 4, 3, 3, 1, 1)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((s.h, s.w, s.n, s.cin)).astype(np.float32)
    w = rng.standard_normal((s.cout, s.kh, s.kw, s.cin)).astype(np.float32)
    dy = rng.standard_normal((s.ho, s.wo, s.n, s.cout)).astype(np.float32)
    _, _, na = oracle.cuyckens_im2col_quantize(s, x, 0)
    _, cw = oracle.cuyckens_fwd(s, *oracle.cuyckens_im2col_quantize(s, x, 0)[:2], w, 0, 0)
    _, cg = oracle.cuyckens_dgrad(s, dy, w, 1, 0)
    assert na == 9 * x.size and cw["W"] == w.size and cg["G"] == dy.size


def test_activation_mse_lossless_is_zero_and_microqonv_weights_copies():
    """On inputs every method represents exactly the MSE is 0; the MicroQonv
    MSE is the error of each X element weighted by its number of in-image
    copies in X' (computed here from the quantized X directly)."""
    s = ConvShape(4, 40, 7, 6, 8, 3, 3, 2, 1)
    x, _, _ = _lossless(s, 13)
    for m in ("microqonv", "naive", "cuyckens"):
        assert oracle.activation_mse(s, x, 0, m) == 0.0
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((s.h, s.w, s.n, s.cin)) * np.exp(rng.uniform(-3, 3, (s.h, s.w, 1, 1)))).astype(np.float32)
    c, sc, _ = oracle.quantize(oracle.ROLE_ACT, 4, 32, x)
    err2 = (oracle.dequantize(oracle.ROLE_ACT, 4, 32, c, sc) - x.astype(np.float64)) ** 2
    # copies of pixel (h, w) in X': number of (output pixel, tap) pairs reading it
    cnt = np.zeros((s.h, s.w))
    for ho in range(s.ho):
        for wo in range(s.wo):
            for kh in range(s.kh):
                for kw in range(s.kw):
                    hi, wi = ho * s.stride + kh - s.pad, wo * s.stride + kw - s.pad
                    if 0 <= hi < s.h and 0 <= wi < s.w:
                        cnt[hi, wi] += 1
    expect = np.sum(err2 * cnt[:, :, None, None]) / (np.sum(cnt) * s.n * s.cin)
    assert oracle.activation_mse(s, x, 4, "microqonv") == pytest.approx(expect, rel=1e-12)

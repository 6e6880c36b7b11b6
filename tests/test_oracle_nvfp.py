"""Pins of the oracle's two-level (NVFP-style) scaling, Eqs. (4)-(6) of the
MicroQonv paper (§II-D, §III-A): FP32 tensor scale T = max|X| / (448 m),
E4M3 block scales rounded to nearest, elements rounded to nearest even,
square 8 x 8 blocks (B = 64, §IV-B)."""
import numpy as np
import pytest

import oracle


def _block(vals):
    """An activation [1][1][8][8] (one pixel, 8 samples x 8 channels)."""
    x = np.zeros((1, 1, 8, 8), np.float32)
    for (n, c), v in vals.items():
        x[0, 0, n, c] = v
    return x


def test_hand_worked_blocks_fp4():
    """Worked by hand: one pixel of N = 8 samples and C = 24 channels, three
    8 x 8 blocks, E2M1 elements (m = 6).
    T = 2688 / (448 * 6) = 1.
    block 0: max 2688 -> B = E4M3(448) = 448 (0x7E); 2688 / 448 = 6 -> code 0x7;
             -1 / 448 rounds to -0 -> code 0x8.
    block 1: max 3 -> B = 0.5 (0x30); 3 / 0.5 = 6 -> 0x7; 1.25 / 0.5 = 2.5 is a
             tie between 2 and 3 -> even mantissa 2 -> 0x4.
    block 2: max 5 -> 5 / 6 = 0.8333 -> nearest E4M3 0.8125 (0x35); 5 / 0.8125 =
             6.15 saturates to 6 -> 0x7; 0.8125 / 0.8125 = 1 -> 0x2."""
    x = np.zeros((1, 1, 8, 24), np.float32)
    x[0, 0, 0, 0], x[0, 0, 1, 1] = 2688.0, -1.0
    x[0, 0, 2, 8], x[0, 0, 3, 9] = 3.0, 1.25
    x[0, 0, 4, 16], x[0, 0, 5, 17] = 5.0, 0.8125
    codes, bs, T = oracle.nvfp_quantize(oracle.ROLE_ACT, 4, x)
    assert T == 1.0
    np.testing.assert_array_equal(bs.reshape(-1), [0x7E, 0x30, 0x35])
    c = codes[0, 0]
    assert (c[0, 0], c[1, 1], c[2, 8], c[3, 9], c[4, 16], c[5, 17]) == (0x7, 0x8, 0x7, 0x4, 0x7, 0x2)
    assert np.count_nonzero(c) == 6


def test_zero_tensor_and_zero_block_scale():
    """An all-zero tensor gets T = 0 and zero codes; a block so small next to
    the tensor maximum that its E4M3 scale rounds to 0 gets zero codes."""
    c, bs, T = oracle.nvfp_quantize(oracle.ROLE_ACT, 4, np.zeros((2, 1, 8, 16), np.float32))
    assert T == 0.0 and not c.any() and not bs.any()
    x = np.zeros((1, 1, 8, 16), np.float32)
    x[0, 0, 0, 0] = 1e6
    x[0, 0, 0, 8] = 1e-3  # 1e-3 / (T * 6) = 2.7e-6 < half the smallest E4M3 subnormal 2^-10
    c, bs, T = oracle.nvfp_quantize(oracle.ROLE_ACT, 4, x)
    assert bs.reshape(-1)[1] == 0 and c[0, 0, 0, 8] == 0


@pytest.mark.parametrize("fmt", range(5))
def test_nearest_grid_point_and_power_of_two_equivariance(fmt):
    """Every non-saturated element dequantizes to the nearest point of the
    element grid scaled by B_i * T; scaling the tensor by 2^k scales T by 2^k
    and leaves codes and block scales unchanged."""
    rng = np.random.default_rng(60 + fmt)
    x = (rng.standard_normal((3, 2, 16, 40)) * np.exp(rng.uniform(-2, 2, (3, 2, 16, 1)))).astype(np.float32)
    codes, bs, T = oracle.nvfp_quantize(oracle.ROLE_ACT, fmt, x)
    deq = oracle.nvfp_dequantize(oracle.ROLE_ACT, fmt, codes, bs, T)
    mx = oracle.elem_max(fmt)
    grid = np.array(sorted({abs(oracle.decode(fmt, c)) for c in range(1 << oracle.ELEM_BITS[fmt])
                            if np.isfinite(oracle.decode(fmt, c))}))
    # per-element scale d = B_i * T, recomputed from the block scales
    bsv = np.vectorize(lambda b: oracle.decode(0, int(b)))(bs.reshape(6, 2, 5))
    d = np.repeat(np.repeat(bsv, 8, axis=1), 8, axis=2)[:, :16, :40].reshape(x.shape) * T
    v = x.astype(np.float64) / d
    inside = np.abs(v) <= mx
    near = grid[np.abs(np.abs(v[inside])[:, None] - grid[None, :]).argmin(axis=1)]
    got = np.abs(deq[inside] / d[inside])
    assert np.all(np.abs(np.abs(v[inside]) - got) <= np.abs(np.abs(v[inside]) - near) * (1 + 1e-12) + 1e-300)
    for k in (-3, 5):
        c2, bs2, T2 = oracle.nvfp_quantize(oracle.ROLE_ACT, fmt, x * np.float32(2.0 ** k))
        assert T2 == pytest.approx(T * 2.0 ** k, rel=0) and np.array_equal(c2, codes) and np.array_equal(bs2, bs)


def test_weight_blocks_are_cin_by_cout_per_tap():
    """Weights [Cout][Kh][Kw][Cin]: a block is 8 Cin x 8 Cout of one tap, so a
    larger value (below the tensor maximum, so T stays) changes the block
    scale of its own (tap, Cout block, Cin block) only."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal((16, 3, 3, 16)).astype(np.float32)
    _, bs0, T0 = oracle.nvfp_quantize(oracle.ROLE_WEIGHT, 4, w)
    w2 = w.copy()
    w2[3, 1, 2, 5] = np.abs(w).max() * np.float32(0.999)  # tap (1, 2) = 5, Cout block 0, Cin block 0
    _, bs1, T1 = oracle.nvfp_quantize(oracle.ROLE_WEIGHT, 4, w2)
    assert T1 == T0
    np.testing.assert_array_equal(np.argwhere(bs0 != bs1), [[0, 5, 0, 0]])

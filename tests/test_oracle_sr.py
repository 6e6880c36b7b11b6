"""Pins of the oracle's stochastic rounding (MicroQonv §III-A: activations and
weights round to nearest, the gradient is rounded stochastically): the
Philox4x32-10 generator against its published known-answer vectors, the
rounding rule on hand-worked values with chosen random words, unbiasedness,
and the block rule it shares with round-to-nearest."""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    for line in open(os.path.join(GOLD, "philox_kat.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            w = [int(t, 16) for t in line.split()]
            rows.append((w[:4], w[4:6], w[6:]))
    return rows


@pytest.mark.parametrize("ctr,key,out", _kat())
def test_philox_known_answers(ctr, key, out):
    assert [int(v) for v in oracle.philox4x32_10(ctr, key)] == out


def test_sr_word_selection():
    """Element (row, c) takes word c mod 4 of the block at counter
    (row, c // 4, 0, 0) under key (seed low, seed high)."""
    seed = 0x0123456789ABCDEF
    for row, c in [(0, 0), (5, 3), (7, 4), (123456, 45), (2**31 - 1, 127)]:
        words = oracle.philox4x32_10([row & 0xFFFFFFFF, c // 4, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.sr_word(seed, row, c) == int(words[c % 4])


# (format, scaled value, lower grid point code, upper grid point code, T = floor(2^32 * frac))
# worked by hand from the element grids:
#   E4M3 at 1.03125: binade [1, 2) has spacing 1/8, frac = 0.25 -> 2^30; codes 0x38 (1.0), 0x39 (1.125)
#   E4M3 at -0.0029296875 = -(1.5 * 2^-9): subnormal spacing 2^-9, frac = 0.5 -> 2^31; codes 0x81, 0x82
#   E2M1 at 2.5: binade [2, 4) spacing 1, frac = 0.5 -> 2^31; codes 0x4 (2), 0x5 (3)
#   E2M1 at 0.125: subnormal spacing 0.5, frac = 0.25 -> 2^30; codes 0x0, 0x1 (0.5)
#   E3M2 at 27.0: binade [16, 32) spacing 4, frac = 0.75 -> 3 * 2^30; codes 0x1E (24), 0x1F (28)
HAND = [
    (0, 1.03125, 0x38, 0x39, 1 << 30),
    (0, -0.0029296875, 0x81, 0x82, 1 << 31),
    (4, 2.5, 0x4, 0x5, 1 << 31),
    (4, 0.125, 0x0, 0x1, 1 << 30),
    (3, 27.0, 0x1E, 0x1F, 3 << 30),
]


@pytest.mark.parametrize("fmt,v,lo,hi,T", HAND)
def test_sr_rounds_up_exactly_when_word_below_threshold(fmt, v, lo, hi, T):
    assert oracle.encode_sr(fmt, v, 0) == hi
    assert oracle.encode_sr(fmt, v, T - 1) == hi
    assert oracle.encode_sr(fmt, v, T) == lo
    assert oracle.encode_sr(fmt, v, 0xFFFFFFFF) == lo


@pytest.mark.parametrize("fmt", range(5))
def test_sr_keeps_grid_points_and_saturates(fmt):
    """Grid points (signed zeros included) never move, whatever the word;
    above the largest normal the result is the largest normal."""
    bits = oracle.ELEM_BITS[fmt]
    mx = oracle.elem_max(fmt)
    for code in range(1 << bits):
        v = oracle.decode(fmt, code)
        if not np.isfinite(v):
            continue
        for r in (0, 1, 1 << 31, 0xFFFFFFFF):
            assert oracle.encode_sr(fmt, v, r) == code
    top = oracle.encode(fmt, mx)
    for r in (0, 0xFFFFFFFF):
        assert oracle.encode_sr(fmt, mx * 1.01, r) == top
        assert oracle.encode_sr(fmt, -mx * 1.2, r) == top | (1 << (bits - 1))


@pytest.mark.parametrize("fmt", range(5))
def test_sr_is_floor_or_ceil_and_unbiased(fmt):
    """Every stochastic code is one of the two grid neighbours, and the mean of
    the dequantized values over many random words is the value itself (within
    4 standard deviations), while round-to-nearest is biased on the same value."""
    mx = oracle.elem_max(fmt)
    rng = np.random.default_rng(40 + fmt)
    v = float(mx * 0.37 + 0.013)
    words = rng.integers(0, 1 << 32, 20000, dtype=np.uint64)
    vals = np.array([oracle.decode(fmt, oracle.encode_sr(fmt, v, int(r))) for r in words])
    lo, hi = vals.min(), vals.max()
    assert set(np.unique(vals)) <= {lo, hi} and lo <= v <= hi
    p = (v - lo) / (hi - lo)
    sd = (hi - lo) * np.sqrt(p * (1 - p) / len(vals))
    assert abs(vals.mean() - v) < 4 * sd
    rne = oracle.decode(fmt, oracle.encode(fmt, v))
    assert abs(rne - v) > 8 * sd


@pytest.mark.parametrize("role,bp,shape", [(0, 32, (3, 2, 33, 45)), (2, 1, (2, 3, 5, 70)),
                                           (1, 32, (40, 3, 3, 20))])
def test_quantize_sr_block_rule(role, bp, shape):
    """Stochastic quantization of a tensor keeps the round-to-nearest block
    scales, picks each code from the two grid neighbours of the scaled value
    with that element's own random word, and is reproducible from the seed."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-5, 5, shape[:-1] + (1,)))).astype(np.float32)
    c_rne, s_rne, _ = oracle.quantize(role, 1, bp, x)
    c1, s1, n = oracle.quantize_sr(role, 1, bp, x, seed=77)
    c2, s2, _ = oracle.quantize_sr(role, 1, bp, x, seed=77)
    c3, _, _ = oracle.quantize_sr(role, 1, bp, x, seed=78)
    assert n == x.size
    np.testing.assert_array_equal(s1, s_rne)
    np.testing.assert_array_equal(c1, c2)
    assert np.count_nonzero(c1 != c3) > 0.2 * x.size
    d_sr = oracle.dequantize(role, 1, bp, c1, s1)
    d_rne = oracle.dequantize(role, 1, bp, c_rne, s_rne)
    # the stochastic value is within one grid step of x: never farther than
    # twice the nearest value's distance plus the nearest value's own step
    assert np.all(np.abs(d_sr - x) <= 2 * np.abs(d_rne - x) + np.abs(d_rne) * 2.0 ** -2 + 1e-30)
    # element (row, c) uses word (row, c): recompute a few codes one by one
    flat = x.reshape(-1, shape[-1])
    scl = 2.0 ** (s1.astype(np.int64) - 127)
    for row, c in [(0, 0), (1, 44 % shape[-1]), (flat.shape[0] - 1, shape[-1] - 1)]:
        if role == 1:  # [Cout][Kh][Kw][Cin]: scale of (co, kh, kw) at [kh][kw][co // bp]
            co, t = divmod(row, shape[1] * shape[2])
            kh, kw = divmod(t, shape[2])
            s = scl[kh, kw, co // bp, c // 32]
        else:  # [H][W][N][C]
            hw, nn = divmod(row, shape[2])
            hh, ww = divmod(hw, shape[1])
            s = scl[hh, ww, nn // bp, c // 32]
        code = oracle.encode_sr(1, float(flat[row, c]) / s, oracle.sr_word(77, row, c))
        assert code == c1.reshape(-1, shape[-1])[row, c]

"""Pins of the oracle's element codec and block quantizer against facts fixed
outside the oracle: values printed in the MicroQonv paper, the OCP element
value tables, torch's own float8 casts, hand-worked blocks and brute force.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
BITS = {0: 8, 1: 8, 2: 6, 3: 6, 4: 4}
MBITS = {0: 3, 1: 2, 2: 3, 3: 2, 4: 1}


def _read_rows(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line)
    return rows


def _grid(fmt):
    """Non-negative values by magnitude code, from sources independent of
    the oracle: torch's float8 dtypes for the 8-bit formats, the OCP value
    tables for the 6- and 4-bit formats."""
    if fmt == 0:
        v = torch.arange(128, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
        return v[:127]  # code 127 is NaN
    if fmt == 1:
        v = torch.arange(128, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
        return v[:124]  # exponent 31 is Inf/NaN
    for row in _read_rows("subbyte_values.txt"):
        parts = row.split()
        if int(parts[0]) == fmt:
            return np.array([float(t) for t in parts[1:]])
    raise KeyError(fmt)


@pytest.mark.parametrize("fmt", range(5))
def test_decode_matches_independent_tables(fmt):
    grid = _grid(fmt)
    sign = 1 << (BITS[fmt] - 1)
    for code, val in enumerate(grid):
        assert oracle.decode(fmt, code) == val
        assert oracle.decode(fmt, code | sign) == -val


def test_printed_maxima():
    for row in _read_rows("format_maxima.txt"):
        fmt, mx = row.split()
        fmt = int(fmt)
        assert oracle.elem_max(fmt) == float(mx)
        assert _grid(fmt).max() == float(mx)


@pytest.mark.parametrize("fmt", range(5))
def test_encode_roundtrip_every_code(fmt):
    grid = _grid(fmt)
    sign = 1 << (BITS[fmt] - 1)
    for code, val in enumerate(grid):
        assert oracle.encode(fmt, val) == code
        assert oracle.encode(fmt, -val) == code | sign  # includes -0 -> sign bit only


@pytest.mark.parametrize("fmt", range(5))
def test_encode_is_nearest_grid_point_ties_even(fmt):
    """Brute force: the nearest non-negative grid value, ties to the even
    magnitude code (= even mantissa), saturation above the maximum."""
    grid = _grid(fmt)
    mx = grid[-1]
    rng = np.random.default_rng(100 + fmt)
    mids = (grid[:-1] + grid[1:]) / 2  # exact ties
    v = np.concatenate([
        rng.uniform(-1.3 * mx, 1.3 * mx, 300_000),
        np.exp(rng.uniform(np.log(grid[1] / 8), np.log(mx * 1.2), 300_000)) * rng.choice([-1, 1], 300_000),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
        [mx * 1.001, -mx * 1e3, grid[1] / 2, grid[1] / 2 * 0.999],
    ])
    got = oracle.encode_array(fmt, v)
    a = np.minimum(np.abs(v), mx)
    d = np.abs(a[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    codes = np.arange(len(grid))[None, :]
    # among the (one or two) nearest codes take the even one
    best = np.where(cand & (codes % 2 == 0), codes, 10_000).min(axis=1)
    single = cand.sum(axis=1) == 1
    best = np.where(single, np.argmax(cand, axis=1), best)
    expect = best | (np.signbit(v).astype(np.int64) << (BITS[fmt] - 1))
    np.testing.assert_array_equal(got.astype(np.int64), expect)


@pytest.mark.parametrize("fmt,torch_dtype", [(0, torch.float8_e4m3fn), (1, torch.float8_e5m2)])
def test_encode_matches_torch_float8_inside_range(fmt, torch_dtype):
    """torch's float8 casts round to nearest-even but do not saturate; inside
    the representable range they must agree with the oracle bit for bit."""
    mx = oracle.elem_max(fmt)
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(200_000) * mx / 8,
                        np.exp(rng.uniform(-25, np.log(mx), 200_000)) * rng.choice([-1, 1], 200_000)])
    v = v[np.abs(v) <= mx].astype(np.float32)
    ref = torch.from_numpy(v).to(torch_dtype).view(torch.uint8).numpy()
    got = oracle.encode_array(fmt, v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def _parse_blocks():
    out = []
    for row in _read_rows("hand_blocks.txt"):
        f, xs, s, cs = [t.strip() for t in row.split("|")]
        out.append((int(f), [float(t) for t in xs.split(",")], int(s),
                    [int(t, 16) for t in cs.split(",")]))
    return out


@pytest.mark.parametrize("fmt,xs,scale,codes", _parse_blocks())
def test_hand_worked_blocks(fmt, xs, scale, codes):
    x = np.array(xs, np.float32)
    c, s, n = oracle.quantize_view(fmt, 1, x, 1, 1, 1, len(x))
    assert n == len(x)
    assert int(s.reshape(-1)[0]) == scale
    assert [int(t) for t in c] == codes


@pytest.mark.parametrize("fmt", range(5))
def test_scale_rule_invariants(fmt):
    """Shared exponent: the block maximum lands in the element format's top
    binade [2^emax, 2^(emax+1)) before saturation; scaling a block by 2^k
    leaves the codes unchanged and adds k to the scale byte."""
    emax = oracle.elem_emax(fmt)
    rng = np.random.default_rng(11 + fmt)
    for _ in range(200):
        x = (rng.standard_normal(32) * np.exp(rng.uniform(-20, 20))).astype(np.float32)
        c, s, _ = oracle.quantize_view(fmt, 1, x, 1, 1, 1, 32)
        S = int(s.reshape(-1)[0])
        v = np.abs(x.astype(np.float64)).max() * 2.0 ** (127 - S)
        assert 2.0 ** emax <= v < 2.0 ** (emax + 1)
        k = int(rng.integers(-10, 11))
        c2, s2, _ = oracle.quantize_view(fmt, 1, (x * np.float32(2.0 ** k)), 1, 1, 1, 32)
        np.testing.assert_array_equal(c, c2)
        assert int(s2.reshape(-1)[0]) == S + k


def test_scale_clamps_and_zero_and_nonfinite():
    # all-zero block: scale byte 0, codes 0 (with the sign of zero)
    c, s, _ = oracle.quantize_view(0, 1, np.zeros(32, np.float32), 1, 1, 1, 32)
    assert s.reshape(-1)[0] == 0 and not c.any()
    # tiny block: exponent clamped at -127, values kept where representable
    x = np.full(32, 2.0 ** -130, np.float32)  # an fp32 subnormal
    x[1] = 2.0 ** -140
    c, s, _ = oracle.quantize_view(0, 1, x, 1, 1, 1, 32)
    assert s.reshape(-1)[0] == 0
    assert oracle.decode(0, int(c[0])) == 2.0 ** -3  # 2^-130 * 2^127
    assert c[1] == 0  # 2^-13 is below half the smallest E4M3 subnormal (2^-9)
    # non-finite input: scale 0xFF and codes 0 for that block only
    x = np.ones(64, np.float32)
    x[3] = np.inf
    c, s, _ = oracle.quantize_view(0, 1, x, 1, 1, 1, 64)
    assert list(s.reshape(-1)) == [255, 127 - 8]
    assert not c[:32].any() and (c[32:] == 0x78).all()  # 1.0 * 2^8 = 256 -> 0.1111.000


def test_square_block_geometry_and_partial_blocks():
    """bp = 32 blocks span 32 channels x 32 partner indices; the last blocks
    are truncated; one large element only affects its own block."""
    H, W, N, C = 2, 1, 40, 45
    x = np.ones((H, W, N, C), np.float32)
    x[1, 0, 33, 40] = 64.0  # inside block (pixel 1, nb 1, cb 1)
    codes, scales, n = oracle.quantize(oracle.ROLE_ACT, 0, 32, x)
    assert n == x.size
    assert scales.shape == (2, 1, 2, 2)
    want = np.full((2, 1, 2, 2), 127 - 8)
    want[1, 0, 1, 1] = 127 - 8 + 6
    np.testing.assert_array_equal(scales, want)
    # weights: partner is Cout, blocks inside one tap
    w = np.ones((40, 3, 3, 45), np.float32)
    w[35, 2, 1, 10] = 256.0
    codes, scales, n = oracle.quantize(oracle.ROLE_WEIGHT, 0, 32, w)
    assert scales.shape == (3, 3, 2, 2)
    want = np.full((3, 3, 2, 2), 127 - 8)
    want[2, 1, 1, 0] = 127 - 8 + 8
    np.testing.assert_array_equal(scales, want)


def test_pack_layout_independent_construction():
    rng = np.random.default_rng(3)
    for fmt in range(5):
        C = 45
        lg = rng.integers(0, 1 << BITS[fmt], size=(3, C)).astype(np.uint8)
        pk = oracle.pack(fmt, lg)
        run = 32 * BITS[fmt] // 8
        assert pk.shape == (3, 2 * run)
        for r in range(3):
            for cb in range(2):
                word = 0
                for j in range(32):
                    c = 32 * cb + j
                    code = int(lg[r, c]) if c < C else 0
                    word |= code << (BITS[fmt] * j)
                want = word.to_bytes(run, "little")
                assert bytes(pk[r, cb * run:(cb + 1) * run]) == want
        np.testing.assert_array_equal(oracle.unpack(fmt, pk, C), lg)
    # 8-bit: identity bytes; 4-bit: code 2i in the low nibble of byte i
    lg = rng.integers(0, 16, size=(1, 32)).astype(np.uint8)
    pk = oracle.pack(4, lg)
    np.testing.assert_array_equal(pk[0], lg[0, 0::2] | (lg[0, 1::2] << 4))


def test_eq7_block_dot_product_identity():
    """Eq. (7): the dot product of two dequantized vectors equals the sum over
    blocks of the two block scales times the dot product of the code values."""
    rng = np.random.default_rng(5)
    for fa, fb in [(0, 0), (4, 0), (3, 1), (2, 4)]:
        S = 160
        r = (rng.standard_normal(S) * 3).astype(np.float32)
        t = (rng.standard_normal(S) * 1e-3).astype(np.float32)
        rc, rs, _ = oracle.quantize_view(fa, 1, r, 1, 1, 1, S)
        tc, ts, _ = oracle.quantize_view(fb, 1, t, 1, 1, 1, S)
        rh = oracle.dequant_view(fa, 1, rc, rs, 1, 1, 1, S)
        th = oracle.dequant_view(fb, 1, tc, ts, 1, 1, 1, S)
        lhs = float(np.dot(rh, th))
        rhs = 0.0
        for j in range(S // 32):
            sr = 2.0 ** (int(rs.reshape(-1)[j]) - 127)
            st = 2.0 ** (int(ts.reshape(-1)[j]) - 127)
            inner = sum(oracle.decode(fa, int(rc[32 * j + i])) * oracle.decode(fb, int(tc[32 * j + i]))
                        for i in range(32))
            rhs += sr * st * inner
        assert lhs == pytest.approx(rhs, rel=1e-15, abs=0)

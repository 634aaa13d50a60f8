"""Pins for the oracle's codecs (oracle/quant.py) against hand-worked examples,
exact rational arithmetic, exhaustive fp16 sweeps and closed-form bounds.

Nothing here re-types the oracle's formulas: every expected value comes from
a different route (integer arithmetic on the exact fp16 values, Fractions, or
literal numbers worked out by hand in tests/golden/quant_examples.json).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ALL_FP16_BITS = np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. max finite
ALL_POS_FP16 = ALL_FP16_BITS[1:].view(np.float16)               # 31743 values


def _fp16_rne(fr: Fraction) -> Fraction:
    """Round a non-negative rational to the nearest fp16 (ties to even),
    computed with exact integers."""
    if fr == 0:
        return Fraction(0)
    e = math.floor(math.log2(fr))
    # correct a possible off-by-one of the float log2
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    e = max(e, -14)                       # subnormal spacing below 2^-14
    spacing = Fraction(2) ** (e - 10)
    m = fr / spacing
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * spacing


def _rne_div_int(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """Round-half-even of num/den for int64 arrays, den > 0, exactly."""
    q = np.floor_divide(num, den)
    rem = num - q * den                    # 0 <= rem < den
    twice = 2 * rem
    up = (twice > den) | ((twice == den) & (q % 2 == 1))
    return q + up.astype(np.int64)


def _fp16_to_int24(x16: np.ndarray) -> np.ndarray:
    """Exact value * 2^24 as int64 (every fp16 is a multiple of 2^-24)."""
    return np.round(x16.astype(np.float64) * 2.0 ** 24).astype(np.int64)


# ---------------------------------------------------------------- golden ---

def test_int8_hand_examples():
    g = json.load(open(os.path.join(GOLDEN, "quant_examples.json")))
    for ex in g["int8"]:
        codes, scale = quant.quantize_int8_sym(np.array(ex["x"], np.float16))
        assert float(scale) == ex["scale"], ex["why"]
        assert codes.tolist() == ex["codes"], ex["why"]


def test_int4_hand_examples():
    g = json.load(open(os.path.join(GOLDEN, "quant_examples.json")))
    for ex in g["int4"]:
        codes, scale, zp = quant.quantize_int4_asym(np.array(ex["x"], np.float16))
        assert float(scale) == ex["scale"], ex["why"]
        assert int(zp) == ex["zero_point"], ex["why"]
        assert codes.tolist() == ex["codes"], ex["why"]


def test_int4_packing_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "quant_examples.json")))["int4_packing"]
    assert quant.pack_int4(np.array(g["codes"])).tolist() == g["bytes"]
    assert quant.unpack_int4(np.array(g["bytes"], np.uint8)).tolist() == g["codes"]


# ------------------------------------------------------------ exhaustive ---

def test_scale_single_rounding_all_fp16():
    """fp16(fp32(a)/127) equals the single nearest-even rounding of the exact
    a/127 for every finite positive fp16 absmax a (so the two-step rounding
    of the scale never differs from the mathematical one)."""
    got = (ALL_POS_FP16.astype(np.float32) / np.float32(127)).astype(np.float16)
    bad = []
    for a, s in zip(ALL_POS_FP16.tolist(), got.astype(np.float64).tolist()):
        if Fraction(s) != _fp16_rne(Fraction(a) / 127):
            bad.append(a)
    assert not bad, bad[:5]


def test_int4_scale_single_rounding_sample():
    """Same for the INT4 step (hi - lo) / 15 on exact fp16 ranges."""
    rng = np.random.default_rng(7)
    span = rng.choice(ALL_POS_FP16, 3000)
    got = (span.astype(np.float32) / np.float32(15)).astype(np.float16)
    for a, s in zip(span.tolist(), got.astype(np.float64).tolist()):
        assert Fraction(s) == _fp16_rne(Fraction(a) / 15), a


def _scale_sample():
    rng = np.random.default_rng(11)
    picks = [1, 2, 3, 0x03FF, 0x0400, 0x0401, 0x1000, 0x2E66, 0x3C00, 0x3C01,
             0x4000, 0x5BF8, 0x6000, 0x7000, 0x7BFF]
    return np.concatenate([np.array(picks, np.uint16).view(np.float16),
                           rng.choice(ALL_POS_FP16, 120)])


@pytest.mark.parametrize("chunk", range(3))
def test_int8_element_map_exact(chunk):
    """For sampled fp16 scales and EVERY fp16 x (both signs), the oracle's
    fp32 route gives clamp(RNE(exact x/s), -127, 127)."""
    scales = _scale_sample()[chunk::3]
    xs = np.concatenate([ALL_FP16_BITS.view(np.float16),
                         (ALL_FP16_BITS[1:] | 0x8000).view(np.float16)])
    xi = _fp16_to_int24(xs)
    for s in scales:
        si = _fp16_to_int24(np.array([s], np.float16))[0]
        expect = np.clip(_rne_div_int(xi, np.full_like(xi, si)), -127, 127)
        got = quant.int8_codes(xs.astype(np.float32), s).astype(np.int64)
        assert np.array_equal(got, expect), float(s)


@pytest.mark.parametrize("zp", [0, 1, 5, 8, 15])
def test_int4_element_map_exact(zp):
    """clamp(RNE(exact x/s + zp), 0, 15) for sampled scales and every fp16 x
    whose code is not clamped far away; the rounding happens after adding
    the zero point."""
    scales = _scale_sample()[::2]
    xs = np.concatenate([ALL_FP16_BITS.view(np.float16),
                         (ALL_FP16_BITS[1:] | 0x8000).view(np.float16)])
    xi = _fp16_to_int24(xs)
    for s in scales:
        si = _fp16_to_int24(np.array([s], np.float16))[0]
        expect = np.clip(_rne_div_int(xi + zp * si, np.full_like(xi, si)), 0, 15)
        got = quant.int4_codes(xs.astype(np.float32), s, zp).astype(np.int64)
        assert np.array_equal(got, expect), (float(s), zp)


# --------------------------------------------------------------- bounds ---

def _rand_tiles(rng, n, rows, d, spread=1.0):
    return (rng.standard_normal((n, rows, d)) * spread).astype(np.float16)


def test_int8_roundtrip_bound_and_range():
    rng = np.random.default_rng(3)
    for tile in _rand_tiles(rng, 300, 16, 128, 2.0):
        codes, s = quant.quantize_int8_sym(tile)
        assert codes.min() >= -127 and codes.max() <= 127
        xhat = quant.dequantize_int8_sym(codes, s)
        err = np.abs(tile.astype(np.float64) - xhat)
        assert err.max() <= 0.5 * float(s)
        # the absmax element maps to +-127 exactly
        i = np.unravel_index(np.argmax(np.abs(tile.astype(np.float32))), tile.shape)
        assert abs(int(codes[i])) == 127


def test_int8_special_cases():
    c, s = quant.quantize_int8_sym(np.full((5, 8), -0.75, np.float16))
    assert np.all(c == -127) and float(s) > 0
    c, s = quant.quantize_int8_sym(np.zeros((3, 8), np.float16))
    assert float(s) == 0.0 and not c.any()
    one = np.zeros((1, 8), np.float16)
    one[0, 3] = 5.0
    c, s = quant.quantize_int8_sym(one)
    assert c[0, 3] == 127 and np.count_nonzero(c) == 1


def test_int8_tiny_absmax_clamps():
    """A subnormal scale can push |x|/s above 127; the code clamps (the
    reading for tiny blocks)."""
    x = np.array([[np.float16(2.0 ** -14) * np.float16(1.0009765625)]], np.float16)
    c, s = quant.quantize_int8_sym(x)
    exact = Fraction(float(x[0, 0])) / Fraction(float(s))
    assert exact > 127 and c[0, 0] == 127


def test_int4_roundtrip_bound_zero_exact():
    rng = np.random.default_rng(5)
    tiles = _rand_tiles(rng, 300, 32, 128)
    mask = rng.random(tiles.shape) < 0.01
    tiles = np.where(mask, tiles * np.float16(8), tiles).astype(np.float16)
    for tile in tiles:
        codes, s, zp = quant.quantize_int4_asym(tile)
        assert codes.max() <= 15 and 0 <= int(zp) <= 15
        xhat = quant.dequantize_int4_asym(codes, s, zp)
        err = np.abs(tile.astype(np.float64) - xhat)
        assert err.max() <= (0.5 + 15 * 2.0 ** -11) * float(s) * 1.0001
        # zero is represented exactly
        zc = quant.int4_codes(np.zeros(1, np.float32), s, zp)
        assert quant.dequantize_int4_asym(zc, s, zp)[0] == 0.0


def test_int4_zero_block_and_constant():
    c, s, z = quant.quantize_int4_asym(np.zeros((4, 8), np.float16))
    assert float(s) == 0 and int(z) == 0 and not c.any()
    c, s, z = quant.quantize_int4_asym(np.full((4, 8), 3.0, np.float16))
    assert int(z) == 0 and np.all(c == 15)
    c, s, z = quant.quantize_int4_asym(np.full((4, 8), -3.0, np.float16))
    assert int(z) == 15 and np.all(c == 0)


def test_pack_unpack_identity():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (7, 5, 128), dtype=np.uint8)
    assert np.array_equal(quant.unpack_int4(quant.pack_int4(codes)), codes)
    with pytest.raises(ValueError):
        quant.pack_int4(np.array([16, 0], np.uint8))


def test_page_literal_rule_differs_from_reading():
    """The page's literal store (fp16 quotient, truncation toward zero)
    disagrees with round-to-nearest on a large share of codes and has a larger
    mean error; recorded to justify the rounding reading."""
    rng = np.random.default_rng(1)
    tiles = _rand_tiles(rng, 50, 16, 128)
    diff, e_lit, e_rne = 0, 0.0, 0.0
    for t in tiles:
        codes, s = quant.quantize_int8_sym(t)
        lit = np.trunc(t / np.float16(s)).astype(np.int64)       # fp16 quotient
        diff += np.count_nonzero(lit != codes)
        e_lit += np.abs(lit * float(s) - t.astype(np.float64)).mean()
        e_rne += np.abs(codes * float(s) - t.astype(np.float64)).mean()
    assert diff / tiles.size > 0.3
    assert e_lit > 1.5 * e_rne


# ------------------------------------------------------------ FP8 E4M3 ---

def test_e4m3_table_hand_values_and_torch():
    """Code values from the format's definition at hand-checked points, and
    the whole table equal to torch's float8_e4m3fn decoding."""
    import torch
    T = quant.E4M3_TABLE
    assert T[0x38] == 1.0 and T[0x7E] == 448.0 and T[0x01] == 2.0 ** -9
    assert T[0x08] == 2.0 ** -6 and T[0x07] == 7 * 2.0 ** -9 and T[0x39] == 1.125
    assert T[0xB8] == -1.0 and T[0x80] == 0.0 and np.signbit(T[0x80])
    assert np.isnan(T[0x7F]) and np.isnan(T[0xFF])
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.nan_to_num(ref, nan=7.0), np.nan_to_num(T, nan=7.0))
    pos = T[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # codes 0..0x7E increase


def test_e4m3_hand_examples():
    """Ties go to the even code, beyond 448 saturates, the sign of zero stays."""
    cases = [(1.0625, 0x38),        # halfway 1 (0x38) / 1.125 (0x39): even 0x38
             (1.1875, 0x3A),        # halfway 1.125 / 1.25: even 0x3A
             (2.0 ** -10, 0x00),    # halfway 0 / 2^-9: even 0x00
             (3 * 2.0 ** -10, 0x02),   # halfway 2^-9 / 2^-8: even 0x02
             (432.0, 0x7E),         # halfway 416 (0x7D) / 448 (0x7E): even 0x7E
             (440.0, 0x7E), (500.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),
             (-0.0, 0x80), (0.0, 0x00), (-1.0, 0xB8), (2.0 ** -11, 0x00), (-(2.0 ** -11), 0x80)]
    for x, c in cases:
        assert int(quant.e4m3_codes(np.float32(x))) == c, x


def test_e4m3_codes_match_torch_and_exact_nearest():
    """Every fp16 value in [-448, 448] and random fp32 quotients: the code
    equals torch's float8_e4m3fn cast (round to nearest even), and on a
    sample equals the nearest value found with exact rationals."""
    import torch
    xs = np.concatenate([ALL_FP16_BITS.view(np.float16), (ALL_FP16_BITS[1:] | 0x8000).view(np.float16)])
    xs = xs[np.abs(xs.astype(np.float32)) <= 448].astype(np.float32)
    r = np.random.default_rng(3).uniform(-448, 448, 200000).astype(np.float32)
    for x in (xs, r):
        want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(quant.e4m3_codes(x), want)
    vals = [Fraction(v) for v in quant.E4M3_TABLE[:0x7F].tolist()]
    for x in r[:3000].tolist():
        a = abs(Fraction(x))
        best = min(range(0x7F), key=lambda c: (abs(vals[c] - a), c % 2))
        assert quant.e4m3_codes(np.float32(x)) & 0x7F == best, x


def test_fp8_tile_range_and_roundtrip_bound():
    """The tile's largest element maps to +-448; |x_hat - x| is at most half
    a step of the E4M3 grid at x / s (2^-4 relative, 2^-10 absolute below
    2^-6) times s, plus the fp32 quotient's rounding."""
    rng = np.random.default_rng(5)
    for spread in (1.0, 1e-3, 300.0):
        for tile in _rand_tiles(rng, 40, 16, 64, spread):
            codes, s = quant.quantize_fp8_e4m3(tile)
            x = tile.astype(np.float64)
            assert float(s) > 0
            vmax = np.max(np.abs(quant.E4M3_TABLE[codes]))
            assert vmax == 448.0
            xh = quant.dequantize_fp8_e4m3(codes, s)
            t = np.abs(x) / float(s)
            bound = float(s) * np.maximum(t * 2.0 ** -4, 2.0 ** -10) + np.abs(x) * 2.0 ** -22
            assert np.all(np.abs(xh - x) <= bound)


def test_fp8_zero_and_tiny_tiles():
    z = np.zeros((4, 8), np.float16)
    codes, s = quant.quantize_fp8_e4m3(z)
    assert float(s) == 0 and not codes.any()
    tiny = np.full((2, 8), np.float16(2.0 ** -24))      # absmax/448 rounds to fp16 zero
    codes, s = quant.quantize_fp8_e4m3(tiny)
    assert float(s) == 0 and not codes.any()
    # a scale that rounds down makes |x| / s exceed 448: saturated, not NaN
    x = np.array([[449.0, 1.0]], np.float16)
    codes, s = quant.quantize_fp8_e4m3(x)
    assert float(x[0, 0]) / float(s) > 448 and int(codes[0, 0]) == 0x7E


# ------------------------------------------------------- INT8 asymmetric ---

@pytest.mark.parametrize("zp", [0, 1, 100, 128, 255])
def test_int8_asym_element_map_exact(zp):
    """clamp(RNE(exact x/s + zp), 0, 255) for sampled scales and every fp16 x,
    by exact integer arithmetic (the fp32 route rounds only where it cannot
    change the result)."""
    scales = _scale_sample()[1::2]
    xs = np.concatenate([ALL_FP16_BITS.view(np.float16),
                         (ALL_FP16_BITS[1:] | 0x8000).view(np.float16)])
    xi = _fp16_to_int24(xs)
    for s in scales:
        si = _fp16_to_int24(np.array([s], np.float16))[0]
        expect = np.clip(_rne_div_int(xi + zp * si, np.full_like(xi, si)), 0, 255)
        got = quant.int8_asym_codes(xs.astype(np.float32), s, zp).astype(np.int64)
        assert np.array_equal(got, expect), (float(s), zp)


def test_int8_asym_scale_zero_point_and_bound():
    """scale = fp16 of the widened range / 255 (exact rationals), zero point
    = RNE(-lo / s), 0 maps to the zero point exactly, and every in-range
    value comes back within s / 2."""
    rng = np.random.default_rng(9)
    for spread, shift in ((1.0, 0.0), (0.01, 0.5), (50.0, -20.0), (1.0, 3.0)):
        for tile in (rng.standard_normal((30, 16, 64)) * spread + shift).astype(np.float16):
            codes, s, zp = quant.quantize_int8_asym(tile)
            x = tile.astype(np.float64)
            lo, hi = min(0.0, x.min()), max(0.0, x.max())
            assert Fraction(float(s)) == _fp16_rne((Fraction(hi) - Fraction(lo)) / 255)
            assert int(zp) == int(np.clip(_rne_div_int(np.array([_fp16_to_int24(np.array([-lo], np.float16))[0]]),
                                                        _fp16_to_int24(np.array([s], np.float16)))[0], 0, 255))
            assert int(quant.int8_asym_codes(np.float32([0.0]), s, zp)[0]) == int(zp)
            xh = quant.dequantize_int8_asym(codes, s, zp)
            inside = (x / float(s) + int(zp) >= -0.5) & (x / float(s) + int(zp) <= 255.5)
            assert np.all(np.abs(xh - x)[inside] <= float(s) / 2 * (1 + 2.0 ** -10))
            assert inside.mean() > 0.99

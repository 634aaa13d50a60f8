"""GPU parity of the store kernel on the codecs' extreme cases, bit for bit
against the oracle (codes, fp16 scale bits, zero points), through the C ABI.

* One tile per positive finite fp16 absmax (all 31,743 of them) for every
  codec pair: subnormal fp16 scales (absmax below 127 * 2^-14 for INT8), the
  codes that then clamp at 127 (reading R6: |x| / s can reach 190), FP8
  quotients that the scale's rounding pushes past 448 (reading R28: they
  saturate), and asymmetric tiles whose ranges sweep every zero point.
  (yunthe.com "quantization principle": Q(x) = clamp(round(x / scale +
  zero_point), 0, 2^bits - 1); tbr8.org §4 store_kv: absmax / 127.)
* Element sweeps: every finite fp16 value as an element of tiles under fixed
  absmax values, among them 448 for FP8 (scale 1, so every quotient is the
  fp16 value itself: every E4M3 rounding midpoint and its fp16 neighbours
  reach the conversion) and absmax values whose scales are not powers of two
  (quotients off the fp16 grid), and subnormal-scale absmax values for INT8.
* A decode over the absmax sweep: every scale, subnormal ones included,
  through the dequantizing attention, in bands of similar magnitude.
"""

import numpy as np
import pytest
import torch

from gpu_util import SmallCase, announce, assert_close, assert_pool_equal, codecs

pytestmark = pytest.mark.gpu

BS, D, H = 16, 64, 8
F16 = np.float16
# codec names (gpu_util.codecs): INT8 K with each V codec, FP8 K and V, and
# INT4 K with INT4 or INT8 V
CODECS = ["i8", "i4", "i8a", "fp8", "k4i4", "k4i8"]


def _finite_positive_f16():
    return np.arange(1, 0x7C00, dtype=np.uint16).view(F16)


def _tiles_to_history(tiles):
    """A list of [BS, D] fp16 tiles -> one sequence's token-major [T, H, D]
    rows, tile i in (block i // H, head i % H); unused heads of the last
    block are zero tiles."""
    n_blk = (len(tiles) + H - 1) // H
    hist = np.zeros((n_blk * BS, H, D), F16)
    for i, t in enumerate(tiles):
        b, g = divmod(i, H)
        hist[b * BS:(b + 1) * BS, g, :] = t
    return hist


def _sym_tile(a, rng, with_ties):
    """Elements in [-a, a] with +-a at element 0: uniform fractions of a, and
    (with_ties) values exactly halfway between codes of the INT8 grid of the
    scale fp16(a / 127) where fp16 holds them."""
    x = (rng.uniform(-1.0, 1.0, BS * D) * np.float64(a)).astype(F16)
    x[0] = F16(a) if rng.integers(2) else -F16(a)
    if with_ties:
        s = np.float64(F16(np.float32(a) / np.float32(127.0)))
        if s > 0:
            k = rng.integers(-127, 127, 64)
            t = (k + 0.5) * s
            ok = (t.astype(F16).astype(np.float64) == t) & (np.abs(t) <= np.float64(a))
            x[1:1 + int(ok.sum())] = t[ok].astype(F16)
    return x.reshape(BS, D)


def _asym_tile(a, i, rng):
    """Elements in [lo, hi] with both ends present; the range's shape cycles
    so that zero points run from 0 (all >= 0) to the top code (all <= 0)."""
    kind = i % 4
    f = ((i // 4) % 17) / 16.0
    a = np.float64(a)
    lo, hi = {0: (0.0, a), 1: (-a, 0.0), 2: (-a * f, a), 3: (-a, a * f)}[kind]
    x = rng.uniform(lo, hi, BS * D).astype(F16)
    x[0], x[1] = F16(lo), F16(hi)
    return x.reshape(BS, D)


def _sweep_tiles(spec, rng):
    """One K and one V tile per positive finite fp16 absmax: symmetric tiles
    for symmetric codecs, range-sweeping tiles for asymmetric ones."""
    kc, vc = codecs(spec)
    amax = _finite_positive_f16()
    if kc == "i4":
        ktiles = [_asym_tile(a, i + 1, rng) for i, a in enumerate(amax)]
    else:
        ktiles = [_sym_tile(a, rng, kc != "fp8") for a in amax]
    if vc in ("i4", "i8a"):
        vtiles = [_asym_tile(a, i, rng) for i, a in enumerate(amax)]
    else:
        vtiles = [_sym_tile(a, rng, vc == "i8") for a in amax]
    return ktiles, vtiles


def _absmax_case(vc, seed):
    rng = np.random.default_rng(seed)
    ktiles, vtiles = _sweep_tiles(vc, rng)
    hk, hv = _tiles_to_history(ktiles), _tiles_to_history(vtiles)
    n_blocks = hk.shape[0] // BS
    q = (rng.standard_normal((1, H, D)) * 2.0 ** -10).astype(F16)
    return SmallCase([hk], [hv], q, H, H, D, BS, vc, n_blocks, rng.permutation(n_blocks))


@pytest.mark.parametrize("vc", CODECS)
def test_every_fp16_absmax(vc):
    announce("absmax sweep", vc)
    case = _absmax_case(vc, seed=11 + CODECS.index(vc))
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    g = case.pool.k_scale.cpu().numpy().view(np.uint16)
    kc_name, vc_name = codecs(vc)
    # the sweep reached subnormal scales and (INT8) codes clamped at +-127
    assert np.any((g > 0) & (g < 0x0400)), "no subnormal K scale"
    if kc_name == "i8":
        kc = case.opool.k_codes
        assert np.any(np.abs(kc.astype(np.int32)) == 127)
    if vc_name in ("i4", "i8a"):
        zp = case.opool.v_zp
        top = 15 if vc_name == "i4" else 255
        assert zp.min() == 0 and zp.max() == top
        if vc_name == "i4":
            assert len(np.unique(zp)) == 16, "every INT4 zero point"
    if kc_name == "i4":
        assert len(np.unique(case.opool.k_zp)) == 16, "every INT4 K zero point"


@pytest.mark.parametrize("vc", CODECS)
def test_decode_over_every_absmax(vc):
    """The attention over the absmax sweep's tiles, every scale (subnormal
    ones included) dequantized inside the kernel.  The tiles are cut into 62
    sequences of 64 blocks, so that each sequence's tiles have absmax values
    within about one binade; each sequence's outputs are compared with the
    oracle relative to its largest V magnitude (attention is linear in V:
    the kernel's error scales with the V values, not with an output that
    happens to be near zero)."""
    announce("absmax sweep decode", vc)
    rng = np.random.default_rng(21 + CODECS.index(vc))
    ktiles, vtiles = _sweep_tiles(vc, rng)
    hk, hv = _tiles_to_history(ktiles), _tiles_to_history(vtiles)
    per = 64 * BS
    n_seq = hk.shape[0] // per
    hks = [hk[i * per:(i + 1) * per] for i in range(n_seq)]
    hvs = [hv[i * per:(i + 1) * per] for i in range(n_seq)]
    # queries small enough that the scores of the largest tiles stay moderate
    q = (rng.standard_normal((n_seq, H, D)) * 2.0 ** -10).astype(F16)
    n_blocks = n_seq * 64
    case = SmallCase(hks, hvs, q, H, H, D, BS, vc, n_blocks, rng.permutation(n_blocks))
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    ref = case.reference()
    for part in (0, 256):
        out = case.decode(part)
        for s_ in range(n_seq):
            sigma = float(np.max(np.abs(hvs[s_].astype(np.float64)))) or 1.0
            assert_close(out[s_] / sigma, ref[s_] / sigma, f"absmax sweep decode {vc} seq {s_} part {part}")


def _all_f16_upto(a):
    """Every finite fp16 value x with |x| <= a (both signs, +-0)."""
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(F16)
    pos = pos[pos.astype(np.float64) <= np.float64(a)]
    return np.concatenate([pos, -pos])


def _element_tiles(values, first):
    """Tiles of BS*D elements: `first` (the values fixing the tile's scale
    and range) at the start of every tile, then the values in order."""
    first = np.asarray(first, F16)
    per = BS * D - len(first)
    tiles = []
    for i in range(0, len(values), per):
        t = np.zeros(BS * D, F16)
        chunk = values[i:i + per]
        t[:len(first)] = first
        t[len(first):len(first) + len(chunk)] = chunk
        tiles.append(t.reshape(BS, D))
    return tiles


# absmax values: FP8 scale exactly 1 (448) or off the power-of-two grid;
# INT8 scales subnormal (a < 127 * 2^-14), exactly 1 (127) and the largest
SWEEP_ABSMAX = {
    "fp8": [448.0, 449.0, 447.75, 1.0, 3.0, 1000.0, 65504.0, 0.01, 2.0 ** -12],
    "i8": [127.0, 100.0, 1.0, 65504.0, 0.005, 2.0 ** -10, 3 * 2.0 ** -14, 2.0 ** -17],
}


@pytest.mark.parametrize("vc", CODECS)
def test_every_fp16_element(vc):
    """Every finite fp16 value inside tiles of fixed absmax (symmetric
    codecs) or fixed range (asymmetric), as K and as V."""
    announce("element sweep", vc)
    kc_name, vc_name = codecs(vc)
    kind = "fp8" if vc == "fp8" else "i8"
    sym = []
    for a in SWEEP_ABSMAX[kind]:
        sym += _element_tiles(_all_f16_upto(a), [a])
    asym = []
    for lo, hi in [(-1.0, 3.0), (-100.0, 1.0), (0.0, 7.5), (-2.0 ** -10, 2.0 ** -11), (-60000.0, 1000.0)]:
        vals = _all_f16_upto(max(-lo, hi))
        vals = vals[(vals.astype(np.float64) >= lo) & (vals.astype(np.float64) <= hi)]
        asym += _element_tiles(vals, [lo, hi])
    ktiles = list(asym) if kc_name == "i4" else list(sym)
    vtiles = list(asym) if vc_name in ("i4", "i8a") else list(sym)
    n = max(len(ktiles), len(vtiles))
    zero = np.zeros((BS, D), F16)
    ktiles += [zero] * (n - len(ktiles))
    vtiles += [zero] * (n - len(vtiles))
    hk, hv = _tiles_to_history(ktiles), _tiles_to_history(vtiles)
    n_blocks = hk.shape[0] // BS
    rng = np.random.default_rng(31)
    q = rng.standard_normal((1, H, D)).astype(F16)
    case = SmallCase([hk], [hv], q, H, H, D, BS, vc, n_blocks, rng.permutation(n_blocks))
    case.store_all()
    assert_pool_equal(case.pool, case.opool)

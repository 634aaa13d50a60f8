"""Per-(block, head) KV codecs (test infrastructure only).

What the pages fix
------------------
* Each block is quantized on its own (tbr8.org §3), K with one fp16 scale per
  (block, head) (tbr8.org §4: ``k_scales`` is [num_blocks, num_heads, 1, 1]
  fp16), the scale being the absolute maximum divided by 127 (tbr8.org §4
  ``store_kv``).
* The general quantizer is Q(x) = clamp(round(x / scale + zero_point), 0,
  2^bits - 1) and the dequantizer x_hat = (Q(x) - zero_point) * scale
  (yunthe.com, "quantization principle", both formulas).
* K in INT8, V may go to INT4 (tbr8.org §5, point 1).

Readings where the pages are silent, garbled or contradictory
-------------------------------------------------------------
* Granularity: ``store_kv`` takes one maximum over the whole block (all
  heads) while the scale tensor it writes has a slot per head; the scale is
  taken per (block, head), as the tensor's shape says.
* Rounding: ``store_kv`` casts with truncation while the yunthe.com formula
  rounds; codes round to nearest with ties to even.
* Precision: the quotient x / scale is taken in fp32, correctly rounded, with
  the *stored* fp16 scale as divisor, so codes agree with what dequantization
  multiplies back.  Codes are integers decided by floating point, so they are
  decided in the precision the kernel uses (fp32).  The scale itself is
  fp16(fp32(absmax) / 127) with both roundings to nearest-even.
* INT8 symmetric codes are the yunthe.com formula with bits = 8 and
  zero_point = 128, stored as the signed value Q - 128 in [-127, 127]
  (-128 never occurs because |x| <= absmax).
* All-zero block: scale 0 and all codes 0, so dequantization gives 0.
* INT4 asymmetric scale and zero point are not given by the pages; they
  follow the usual affine recipe in which the range is widened to contain 0
  and the zero point is an integer, so that 0 is exactly representable:
  lo = min(0, min x), hi = max(0, max x), scale = fp16(fp32(hi - lo) / 15),
  zero_point = clamp(rint(fp32(-lo) / scale), 0, 15).  The code is
  clamp(rint(fp32(fp32(x / scale) + zero_point)), 0, 15): division and
  addition each rounded in fp32, no fused multiply-add.
* INT4 packing: two codes per byte along the last axis, the even index in the
  low nibble (V tiles are dim-major, so the last axis is the block's tokens).
* Only the rows a block actually holds take part in the statistics; rows not
  yet written are stored as zero bytes.
Inputs must be finite fp16.

Further codecs (yunthe.com "vLLM deployment": the cache may be stored as
fp8 in the E4M3 format, or int8; yunthe.com "quantization principle" with
bits = 8 and a free zero point for INT8 asymmetric):
* FP8 E4M3 (the OCP 8-bit format with 4 exponent bits of bias 7, 3 mantissa
  bits, subnormals, no infinities, largest finite value 448).  The pages fix
  the format only.  Readings: one fp16 scale per (block, head),
  scale = fp16(fp32(absmax) / 448), so that the largest element maps to the
  top of the range; code = E4M3 of the fp32 quotient x / scale (correctly
  rounded, as for INT8), rounded to nearest with ties to the even code and
  saturated at +-448 (a quotient can exceed 448 only through the scale's
  rounding); the sign of a zero quotient is kept (-0 -> 0x80).  Scale 0 ->
  all codes 0.  x_hat = value(code) * scale.
* INT8 asymmetric: the INT4 asymmetric recipe with 255 in place of 15, codes
  0..255 stored as u8, the zero point u8 beside them.

INT4 K (tbr8.org §3: a block may go to INT8 or even INT4; yunthe.com Q(x)
with bits = 4): K tiles use ``quantize_int4_asym`` unchanged; only their
packing differs (paged.py: along head_dim, K tiles being token-major).
"""

import numpy as np

F32 = np.float32
F16 = np.float16


def int8_codes(x32: np.ndarray, scale) -> np.ndarray:
    """Per-element INT8 map for a nonzero fp16 ``scale``:
    clamp(rint(fp32(x) / fp32(scale)), -127, 127), the quotient correctly
    rounded in fp32 and ties going to even."""
    t = np.asarray(x32, F32) / F32(F16(scale))
    return np.clip(np.rint(t), -127, 127).astype(np.int8)


def int4_codes(x32: np.ndarray, scale, zero_point) -> np.ndarray:
    """Per-element INT4 map for a nonzero fp16 ``scale`` (yunthe.com Q(x) with
    bits = 4): clamp(rint(fp32(fp32(x / scale) + zero_point)), 0, 15)."""
    t = np.asarray(x32, F32) / F32(F16(scale))
    u = t + F32(zero_point)
    return np.clip(np.rint(u), 0, 15).astype(np.uint8)


def quantize_int8_sym(x16: np.ndarray):
    """INT8 symmetric codes and fp16 scale for one (block, head) tile.

    ``x16``: fp16 array [rows, head_dim] of the rows present (rows >= 1).
    Returns (codes int8 [rows, head_dim], scale float16 scalar).
    """
    x16 = np.asarray(x16, dtype=F16)
    x32 = x16.astype(F32)
    absmax = F32(np.max(np.abs(x32))) if x32.size else F32(0)
    scale = F16(absmax / F32(127.0))
    if scale == 0:
        return np.zeros(x16.shape, np.int8), scale
    return int8_codes(x32, scale), scale


def dequantize_int8_sym(codes: np.ndarray, scale) -> np.ndarray:
    """x_hat = code * scale in float64 (exact)."""
    return np.asarray(codes, np.float64) * np.asarray(scale, F16).astype(np.float64)


def quantize_int4_asym(x16: np.ndarray):
    """INT4 asymmetric codes (0..15), fp16 scale and u8 zero point for one
    (block, head) tile of the rows present."""
    x16 = np.asarray(x16, dtype=F16)
    x32 = x16.astype(F32)
    lo = min(F32(0), F32(np.min(x32))) if x32.size else F32(0)
    hi = max(F32(0), F32(np.max(x32))) if x32.size else F32(0)
    scale = F16((F32(hi) - F32(lo)) / F32(15.0))
    if scale == 0:
        return np.zeros(x16.shape, np.uint8), scale, np.uint8(0)
    zp = np.uint8(np.clip(np.rint(F32(-lo) / F32(scale)), 0, 15))
    return int4_codes(x32, scale, zp), scale, zp


def dequantize_int4_asym(codes: np.ndarray, scale, zero_point) -> np.ndarray:
    """x_hat = (code - zero_point) * scale in float64 (exact)."""
    c = np.asarray(codes, np.float64)
    return (c - np.asarray(zero_point, np.float64)) * np.asarray(scale, F16).astype(np.float64)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """[..., n] codes in 0..15 -> [..., n/2] bytes, even index in the low nibble."""
    c = np.asarray(codes, np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("head_dim must be even")
    if np.any(c > 15):
        raise ValueError("INT4 code out of range")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_int4``."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


# ---- FP8 E4M3 ----------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code byte from the format's definition (NaN for
    S.1111.111): sign bit 7, exponent bits 6..3 with bias 7, mantissa bits
    2..0; exponent field 0 is subnormal (m / 8 * 2^-6)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], np.float64)
# non-negative finite values in code order (codes 0x00 .. 0x7E), increasing
_E4M3_POS = E4M3_TABLE[:0x7F]


def e4m3_codes(t32: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3 code bytes: nearest value, ties to the even code,
    magnitudes beyond 448 saturate to 448, the sign bit taken from t (so -0
    gives 0x80)."""
    t = np.asarray(t32, np.float32).astype(np.float64)
    a = np.minimum(np.abs(t), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")      # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    mag = np.where(a == _E4M3_POS[hi], hi, mag).astype(np.uint8)   # exact values
    sign = np.signbit(t).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def quantize_fp8_e4m3(x16: np.ndarray):
    """FP8 E4M3 codes (u8) and fp16 scale for one (block, head) tile of the
    rows present."""
    x16 = np.asarray(x16, dtype=F16)
    x32 = x16.astype(F32)
    absmax = F32(np.max(np.abs(x32))) if x32.size else F32(0)
    scale = F16(absmax / F32(E4M3_MAX))
    if scale == 0:
        return np.zeros(x16.shape, np.uint8), scale
    return e4m3_codes(x32 / F32(scale)), scale


def dequantize_fp8_e4m3(codes: np.ndarray, scale) -> np.ndarray:
    """x_hat = value(code) * scale in float64 (exact)."""
    return E4M3_TABLE[np.asarray(codes, np.uint8)] * np.asarray(scale, F16).astype(np.float64)


# ---- INT8 asymmetric -----------------------------------------------------------

def int8_asym_codes(x32: np.ndarray, scale, zero_point) -> np.ndarray:
    """clamp(rint(fp32(fp32(x / scale) + zero_point)), 0, 255) (yunthe.com
    Q(x) with bits = 8)."""
    t = np.asarray(x32, F32) / F32(F16(scale))
    u = t + F32(zero_point)
    return np.clip(np.rint(u), 0, 255).astype(np.uint8)


def quantize_int8_asym(x16: np.ndarray):
    """INT8 asymmetric codes (0..255), fp16 scale and u8 zero point for one
    (block, head) tile of the rows present: the INT4 recipe with 255 levels."""
    x16 = np.asarray(x16, dtype=F16)
    x32 = x16.astype(F32)
    lo = min(F32(0), F32(np.min(x32))) if x32.size else F32(0)
    hi = max(F32(0), F32(np.max(x32))) if x32.size else F32(0)
    scale = F16((F32(hi) - F32(lo)) / F32(255.0))
    if scale == 0:
        return np.zeros(x16.shape, np.uint8), scale, np.uint8(0)
    zp = np.uint8(np.clip(np.rint(F32(-lo) / F32(scale)), 0, 255))
    return int8_asym_codes(x32, scale, zp), scale, zp


def dequantize_int8_asym(codes: np.ndarray, scale, zero_point) -> np.ndarray:
    """x_hat = (code - zero_point) * scale in float64 (exact)."""
    c = np.asarray(codes, np.float64)
    return (c - np.asarray(zero_point, np.float64)) * np.asarray(scale, F16).astype(np.float64)

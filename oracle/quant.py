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
    return np.asarray(codes, np.float64) * np.float64(F16(scale))


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
    return (c - np.float64(zero_point)) * np.float64(F16(scale))


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

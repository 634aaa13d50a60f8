"""Block pool contents: storing a sequence into scattered blocks and gathering
it back (test infrastructure only).

What the pages fix
------------------
* Physical storage is a pool of blocks shaped [num_blocks, num_heads,
  block_size, head_dim] of int8 codes with a [num_blocks, num_heads] fp16
  scale beside it (tbr8.org §4, ``PagedKVCacheManager.__init__``).
* Blocks of a sequence need not be contiguous; the block table maps logical
  block j to its physical block (tbr8.org §2; yunthe.com "PagedAttention
  mechanism").  Token t of a sequence therefore lives in physical block
  table[t // bs] at row t % bs.
* The per-layer contiguous KV shape is [batch, heads, seq_len, head_dim]
  (yunthe.com, "quantization principle"); ``quantize_contiguous`` quantizes
  that layout in consecutive row chunks of block_size, which must give the
  same values as the paged store followed by the gather.

Readings
--------
* A block is always (re)quantized from the exact fp16 rows it holds, never
  from earlier codes: storing tokens into a partially filled block quantizes
  that block again over all of its rows.  Unfilled rows are zero bytes.
* The pages show only the K pool; the V pool's layout is open.  V tiles are
  stored dim-major, [head_dim, block_size] per (block, head), so that a sum
  over a block's tokens reads one contiguous row per dimension: the V pool is
  [num_blocks, heads, head_dim, block_size] int8, or for INT4
  [num_blocks, heads, head_dim, block_size / 2] bytes holding two consecutive
  tokens per byte (the earlier token in the low nibble), with a u8 zero point
  per (block, head).
* Codecs by name: K "i8" (INT8 symmetric), "fp8" (E4M3) or "i4" (INT4
  asymmetric); V "i8", "i4" (INT4 asymmetric), "i8a" (INT8 asymmetric, u8
  codes) or "fp8".  FP8 and INT8-asymmetric tiles are u8 arrays of the INT8
  tiles' shape; the asymmetric V codecs keep their zero point in ``v_zp``.
* INT4 K (tbr8.org §3: blocks may be quantized to INT8 or even INT4;
  yunthe.com "quantization principle": Q(x) with bits = 4): the same
  per-(block, head) affine recipe as INT4 V, applied to the K tile; K tiles
  stay token-major, so the two codes of a byte are consecutive head dims of
  one token (the even dim in the low nibble): [num_blocks, heads,
  block_size, head_dim / 2] bytes, with the zero point in ``k_zp``.
"""

import numpy as np

from . import quant


class PoolArrays:
    """Host mirror of the device pool arrays, same shapes and dtypes."""

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim,
                 v_int4=False, k_codec="i8", v_codec=None):
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.block_size = block_size
        self.head_dim = head_dim
        self.k_codec = k_codec
        self.v_codec = v_codec if v_codec is not None else ("i4" if v_int4 else "i8")
        assert self.k_codec in ("i8", "fp8", "i4") and self.v_codec in ("i8", "i4", "i8a", "fp8")
        self.v_int4 = self.v_codec == "i4"
        self.k_int4 = self.k_codec == "i4"
        if self.k_int4:
            self.k_codes = np.zeros((num_blocks, num_kv_heads, block_size, head_dim // 2), np.uint8)
        else:
            self.k_codes = np.zeros((num_blocks, num_kv_heads, block_size, head_dim),
                                    np.int8 if k_codec == "i8" else np.uint8)
        if self.v_int4:
            self.v_codes = np.zeros((num_blocks, num_kv_heads, head_dim, block_size // 2), np.uint8)
        else:
            self.v_codes = np.zeros((num_blocks, num_kv_heads, head_dim, block_size),
                                    np.int8 if self.v_codec == "i8" else np.uint8)
        self.k_scale = np.zeros((num_blocks, num_kv_heads), np.float16)
        self.v_scale = np.zeros((num_blocks, num_kv_heads), np.float16)
        self.v_zp = np.zeros((num_blocks, num_kv_heads), np.uint8)
        self.k_zp = np.zeros((num_blocks, num_kv_heads), np.uint8)


def quantize_tile(codec: str, x16):
    """(codes, scale, zero point) of one tile's rows under a codec name."""
    if codec == "i8":
        c, s = quant.quantize_int8_sym(x16)
        return c, s, np.uint8(0)
    if codec == "fp8":
        c, s = quant.quantize_fp8_e4m3(x16)
        return c, s, np.uint8(0)
    if codec == "i4":
        return quant.quantize_int4_asym(x16)
    if codec == "i8a":
        return quant.quantize_int8_asym(x16)
    raise ValueError(codec)


def dequantize_tile(codec: str, codes, scale, zero_point):
    """float64 values of codes under a codec name (zero point for i4/i8a)."""
    if codec == "i8":
        return quant.dequantize_int8_sym(codes, scale)
    if codec == "fp8":
        return quant.dequantize_fp8_e4m3(codes, scale)
    if codec == "i4":
        return quant.dequantize_int4_asym(codes, scale, zero_point)
    if codec == "i8a":
        return quant.dequantize_int8_asym(codes, scale, zero_point)
    raise ValueError(codec)


def store_block(pool: PoolArrays, phys: int, k_rows, v_rows):
    """Quantize the rows a block holds (k_rows, v_rows: fp16 [n, H, D],
    1 <= n <= block_size) into physical block ``phys``, head by head."""
    k_rows = np.asarray(k_rows, np.float16)
    v_rows = np.asarray(v_rows, np.float16)
    n = k_rows.shape[0]
    assert 1 <= n <= pool.block_size
    for h in range(pool.num_kv_heads):
        kc, ks, kz = quantize_tile(pool.k_codec, k_rows[:, h, :])
        pool.k_codes[phys, h] = 0
        # INT4 K: two consecutive head dims of a token per byte
        pool.k_codes[phys, h, :n] = quant.pack_int4(kc) if pool.k_int4 else kc
        pool.k_scale[phys, h] = ks
        pool.k_zp[phys, h] = kz
        # V tile, dim-major: codes[d, t]; tokens >= n stay zero bytes
        vc, vs, vz = quantize_tile(pool.v_codec, v_rows[:, h, :])
        tile = np.zeros((pool.head_dim, pool.block_size), vc.dtype)
        tile[:, :n] = vc.T
        pool.v_codes[phys, h] = quant.pack_int4(tile) if pool.v_int4 else tile
        pool.v_zp[phys, h] = vz
        pool.v_scale[phys, h] = vs


def store_range(pool: PoolArrays, table, k_hist, v_hist, start: int, end: int):
    """Requantize every logical block touched by positions [start, end) of a
    sequence whose fp16 history (rows 0..end-1) is k_hist / v_hist [>=end, H, D].
    """
    bs = pool.block_size
    if end <= start:
        return
    for j in range(start // bs, (end - 1) // bs + 1):
        lo, hi = j * bs, min((j + 1) * bs, end)
        store_block(pool, int(table[j]), k_hist[lo:hi], v_hist[lo:hi])


def gather_dequant(pool: PoolArrays, table, ctx: int):
    """Dequantized K and V of the first ``ctx`` tokens of a sequence, read
    through its block table: float64 [H, ctx, D] each."""
    bs = pool.block_size
    t = np.arange(ctx)
    phys = np.asarray(table, np.int64)[t // bs]
    row = t % bs
    kc = pool.k_codes[phys, :, row, :]                            # [ctx, H, D] (INT4: D / 2 bytes)
    if pool.k_int4:
        kc = quant.unpack_int4(kc)
    ks = pool.k_scale[phys, :]                                    # [ctx, H]
    kz = pool.k_zp[phys, :]
    khat = np.stack([dequantize_tile(pool.k_codec, kc[:, h], ks[:, h][:, None],
                                     kz[:, h][:, None].astype(np.float64))
                     for h in range(pool.num_kv_heads)], axis=1)
    if pool.v_int4:
        tiles = quant.unpack_int4(pool.v_codes[phys])             # [ctx, H, D, bs]
    else:
        tiles = pool.v_codes[phys]
    vc = tiles[np.arange(ctx), :, :, row]                         # [ctx, H, D]
    vz = pool.v_zp[phys, :]
    vs = pool.v_scale[phys, :]
    vhat = np.stack([dequantize_tile(pool.v_codec, vc[:, h], vs[:, h][:, None],
                                     vz[:, h][:, None].astype(np.float64))
                     for h in range(pool.num_kv_heads)], axis=1)
    return khat.transpose(1, 0, 2), vhat.transpose(1, 0, 2)


def quantize_contiguous(x16, block_size: int, int4: bool = False, codec=None):
    """Quantize a contiguous [H, ctx, D] fp16 tensor in row chunks of
    ``block_size`` and return the dequantized float64 values."""
    codec = codec or ("i4" if int4 else "i8")
    x16 = np.asarray(x16, np.float16)
    H, ctx, D = x16.shape
    out = np.zeros((H, ctx, D), np.float64)
    for h in range(H):
        for lo in range(0, ctx, block_size):
            hi = min(lo + block_size, ctx)
            c, s, z = quantize_tile(codec, x16[h, lo:hi])
            out[h, lo:hi] = dequantize_tile(codec, c, s, z)
    return out

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
"""

import numpy as np

from . import quant


class PoolArrays:
    """Host mirror of the device pool arrays, same shapes and dtypes."""

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim,
                 v_int4=False):
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.block_size = block_size
        self.head_dim = head_dim
        self.v_int4 = v_int4
        self.k_codes = np.zeros((num_blocks, num_kv_heads, block_size, head_dim), np.int8)
        if v_int4:
            self.v_codes = np.zeros((num_blocks, num_kv_heads, head_dim, block_size // 2), np.uint8)
        else:
            self.v_codes = np.zeros((num_blocks, num_kv_heads, head_dim, block_size), np.int8)
        self.k_scale = np.zeros((num_blocks, num_kv_heads), np.float16)
        self.v_scale = np.zeros((num_blocks, num_kv_heads), np.float16)
        self.v_zp = np.zeros((num_blocks, num_kv_heads), np.uint8)


def store_block(pool: PoolArrays, phys: int, k_rows, v_rows):
    """Quantize the rows a block holds (k_rows, v_rows: fp16 [n, H, D],
    1 <= n <= block_size) into physical block ``phys``, head by head."""
    k_rows = np.asarray(k_rows, np.float16)
    v_rows = np.asarray(v_rows, np.float16)
    n = k_rows.shape[0]
    assert 1 <= n <= pool.block_size
    for h in range(pool.num_kv_heads):
        kc, ks = quant.quantize_int8_sym(k_rows[:, h, :])
        pool.k_codes[phys, h] = 0
        pool.k_codes[phys, h, :n] = kc
        pool.k_scale[phys, h] = ks
        # V tile, dim-major: codes[d, t]; tokens >= n stay zero
        if pool.v_int4:
            vc, vs, vz = quant.quantize_int4_asym(v_rows[:, h, :])
            tile = np.zeros((pool.head_dim, pool.block_size), np.uint8)
            tile[:, :n] = vc.T
            pool.v_codes[phys, h] = quant.pack_int4(tile)
            pool.v_zp[phys, h] = vz
        else:
            vc, vs = quant.quantize_int8_sym(v_rows[:, h, :])
            tile = np.zeros((pool.head_dim, pool.block_size), np.int8)
            tile[:, :n] = vc.T
            pool.v_codes[phys, h] = tile
            pool.v_zp[phys, h] = 0
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
    kc = pool.k_codes[phys, :, row, :].astype(np.float64)        # [ctx, H, D]
    ks = pool.k_scale[phys, :].astype(np.float64)                # [ctx, H]
    khat = kc * ks[:, :, None]
    if pool.v_int4:
        tiles = quant.unpack_int4(pool.v_codes[phys])                # [ctx, H, D, bs]
        vc = tiles[np.arange(ctx), :, :, row].astype(np.float64)      # [ctx, H, D]
        vz = pool.v_zp[phys, :].astype(np.float64)
        vhat = (vc - vz[:, :, None]) * pool.v_scale[phys, :].astype(np.float64)[:, :, None]
    else:
        vc = pool.v_codes[phys][np.arange(ctx), :, :, row].astype(np.float64)
        vhat = vc * pool.v_scale[phys, :].astype(np.float64)[:, :, None]
    return khat.transpose(1, 0, 2), vhat.transpose(1, 0, 2)


def quantize_contiguous(x16, block_size: int, int4: bool = False):
    """Quantize a contiguous [H, ctx, D] fp16 tensor in row chunks of
    ``block_size`` and return the dequantized float64 values."""
    x16 = np.asarray(x16, np.float16)
    H, ctx, D = x16.shape
    out = np.zeros((H, ctx, D), np.float64)
    for h in range(H):
        for lo in range(0, ctx, block_size):
            hi = min(lo + block_size, ctx)
            if int4:
                c, s, z = quant.quantize_int4_asym(x16[h, lo:hi])
                out[h, lo:hi] = quant.dequantize_int4_asym(c, s, z)
            else:
                c, s = quant.quantize_int8_sym(x16[h, lo:hi])
                out[h, lo:hi] = quant.dequantize_int8_sym(c, s)
    return out

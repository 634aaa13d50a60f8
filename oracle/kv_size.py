"""Closed-form KV-cache sizes and block counts (test infrastructure only).

* Dense KV size: each layer keeps a K and a V tensor shaped
  [batch, heads, seq_len, head_dim] (yunthe.com, "quantization principle").
  The deepinsea.top "pain points" section and the yunthe.com opening paragraph
  quote sizes for Llama-2-7B and LLaMA-70B that these formulas reproduce or
  refute; the tests record which.
* Blocks for n tokens: the smallest count of block_size-token blocks holding
  them, i.e. ceil(n / block_size) (tbr8.org §4 ``allocate_for_request``;
  deepinsea.top "paging mechanism design" ``allocate``).
* Block-quantized size: every (block, head) stores bs*D codes of k_bits for K
  and v_bits for V, plus its own metadata: one fp16 scale for K, one fp16
  scale for V and, when V is asymmetric, one byte of zero point (tbr8.org §4
  keeps one fp16 scale per (block, head); yunthe.com's formula adds a zero
  point).  Codes are counted for the tokens present only; metadata for every
  allocated block.
* Pool sizing: yunthe.com "PagedAttention mechanism" sizes the pool as memory
  divided by (block_size * bytes per token).  With per-(block, head) metadata
  the unit is a whole block, so the divisor is the bytes of one block.
"""


def num_blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks needed for ``num_tokens`` tokens: ceil(n / bs), written as the
    integer form used on deepinsea.top, (n + bs - 1) // bs."""
    if block_size <= 0 or num_tokens < 0:
        raise ValueError("block_size must be > 0 and num_tokens >= 0")
    return (num_tokens + block_size - 1) // block_size


def kv_bytes_dense(num_layers: int, num_kv_heads: int, head_dim: int,
                   seq_len: int, batch: int, bytes_per_elem: int = 2) -> int:
    """Bytes of an unquantized KV cache: K and V per layer, each
    [batch, num_kv_heads, seq_len, head_dim] of ``bytes_per_elem``."""
    per_tensor = batch * num_kv_heads * seq_len * head_dim * bytes_per_elem
    return 2 * num_layers * per_tensor


def meta_bytes_per_block_head(v_asymmetric: bool, k_asymmetric: bool = False) -> int:
    """fp16 K scale + fp16 V scale (+ one u8 zero point for asymmetric V, and
    one for asymmetric K)."""
    return 2 + 2 + (1 if v_asymmetric else 0) + (1 if k_asymmetric else 0)


def kv_bytes_block_quantized(seq_len: int, batch: int, num_kv_heads: int,
                             head_dim: int, block_size: int, k_bits: int,
                             v_bits: int, v_asymmetric: bool,
                             num_layers: int = 1) -> int:
    """Bytes of a block-quantized KV cache for ``batch`` sequences of
    ``seq_len`` tokens: codes of the present tokens plus metadata of every
    allocated (block, head)."""
    code_bits = seq_len * num_kv_heads * head_dim * (k_bits + v_bits)
    if code_bits % 8:
        raise ValueError("code bits do not fill whole bytes")
    blocks = num_blocks_for(seq_len, block_size)
    meta = blocks * num_kv_heads * meta_bytes_per_block_head(v_asymmetric)
    return num_layers * batch * (code_bits // 8 + meta)


def pool_block_bytes(num_kv_heads: int, head_dim: int, block_size: int,
                     k_bits: int, v_bits: int, v_asymmetric: bool, k_asymmetric: bool = False) -> int:
    """Bytes one physical pool block occupies over all KV heads."""
    codes = block_size * head_dim * (k_bits + v_bits) // 8
    return num_kv_heads * (codes + meta_bytes_per_block_head(v_asymmetric, k_asymmetric))


def pool_num_blocks(budget_bytes: int, num_kv_heads: int, head_dim: int,
                    block_size: int, k_bits: int, v_bits: int,
                    v_asymmetric: bool) -> int:
    """Whole blocks that fit a memory budget (floor division)."""
    return budget_bytes // pool_block_bytes(num_kv_heads, head_dim, block_size,
                                            k_bits, v_bits, v_asymmetric)


def compression_ratio(head_dim: int, block_size: int, k_bits: int,
                      v_bits: int, v_asymmetric: bool) -> float:
    """Quantized bytes / fp16 bytes for one full (block, head)."""
    fp16 = 2 * block_size * head_dim * 2
    q = (block_size * head_dim * (k_bits + v_bits) // 8
         + meta_bytes_per_block_head(v_asymmetric))
    return q / fp16

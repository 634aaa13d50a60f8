"""CPU oracle for block-quantized paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code, header, table or constant with
the HIP library; the two meet only through the seeded synthetic inputs.

Sources (web pages; cited by site, title and section):

* tbr8.org, "How PagedAttention combined with block-wise quantization solves
  long-text OOM caused by memory fragmentation on mobile" -- §2 (PagedAttention
  block virtualisation), §3 (block-wise quantization), §4 (the
  ``PagedKVCacheManager`` code: pool tensors, ``allocate_for_request``,
  ``store_kv``, demo), §5 (mixed INT8/INT4, fused quantized paged attention,
  pre-allocated pool with reference counts).
* deepinsea.top, "PagedAttention memory management in depth" -- "pain points"
  (Llama-2-7B example), "paging mechanism design" (``BlockManager.allocate`` /
  ``free``), "block size choice" (table), "Copy-on-Write", "Swap".
* yunthe.com, "LLM inference memory optimisation: KV-cache quantization and
  PagedAttention" -- "quantization principle" (per-layer KV shape, the
  quantize formula Q(x) and the dequantize formula), "PagedAttention
  mechanism" (block_size / num_blocks / block_table structure, prefix sharing,
  copy-on-write fork), "monitoring and evaluation" (4xA100 figures).

Modules
-------
``kv_size``    closed-form KV-cache sizes and block counts.
``allocator``  a list/dict model of the block pool and its block tables.
``quant``      per-(block, head) INT8 symmetric and INT4 asymmetric codecs.
``paged``      storing a sequence's history into pool blocks; gathering back.
``attention``  single-query softmax attention in float64.

Every function states which passage it follows.  Points where the pages are
silent or contradict each other are resolved by the readings listed in each
module docstring.  Parity status: every function is pinned by a CPU test
(``tests/test_oracle_*.py``) against closed forms, exhaustive sweeps, exact
rational arithmetic, brute force or library routines; see each module.
"""

from . import kv_size, allocator, quant, paged, attention  # noqa: F401

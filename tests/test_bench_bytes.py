"""The algorithmic byte and flop counts the benchmark divides by, against
their closed forms at the workloads' sizes (no GPU)."""

import numpy as np

from paged_block_quantized_amd import runner, workloads as W


def test_llama7b_decode_bytes():
    # 32 sequences x 4096 tokens, 32 KV heads x 128 dims, INT8 K and V:
    # codes 2 x 32 x 4096 x 32 x 128 B, two fp16 scales per (block of 16, head),
    # fp16 Q and O rows, one int32 table entry per block, one length per sequence
    w = W.WORKLOADS["llama7b"]
    ctx = W.context_lengths(w)
    codes = 2 * 32 * 4096 * 32 * 128
    scales = 32 * (4096 // 16) * 32 * 4
    qo = 2 * 32 * 32 * 128 * 2
    tables = 32 * (4096 // 16) * 4 + 32 * 4
    assert codes + scales + qo + tables == 1_075_347_584
    assert runner.decode_bytes(w, ctx) == 1_075_347_584


def test_shared_prefix_decode_bytes_count_the_prefix_once():
    # 32 x 32768 tokens, INT8 K + INT4 V (1.5 B per element), fp16 scale pair
    # and u8 zero point per (block of 32, head); the 4096-token prefix's codes
    # and metadata once, the tables and lengths per sequence
    w = W.WORKLOADS["shared_prefix"]
    ctx = W.context_lengths(w)
    tokens = 4096 + 32 * (32768 - 4096)
    blocks = 4096 // 32 + 32 * (32768 - 4096) // 32
    expect = (tokens * 32 * 128 * 3 // 2 + blocks * 32 * 5 + 2 * 32 * 32 * 128 * 2
              + 32 * (32768 // 32) * 4 + 32 * 4)
    assert runner.decode_bytes(w, ctx) == expect == 5_667_573_888
    per_sequence = dict(vars(w))
    per_sequence.pop("extra", None)
    per_sequence["prefix"] = 0
    assert runner.decode_bytes(W.Workload(**per_sequence), ctx) == 6_448_349_312


def test_prefill_store_bytes():
    # 64 prompts x 2048 tokens, 32 KV heads x 128 dims: fp16 K and V read,
    # INT8 codes written, two fp16 scales per (block of 16, head), the tables
    w = W.WORKLOADS["prefill_store"]
    expect = 64 * 2048 * 32 * 128 * 2 * 2 + 64 * 2048 * 32 * 128 * 2 + 64 * 128 * 32 * 4 + 64 * 128 * 4
    assert runner.prefill_store_bytes(w) == expect == 3_222_306_816


def test_prefill_chunk_flops():
    # the last 512 of 4096 tokens query causally: query i (0-based) sees
    # 3584 + i + 1 tokens; 4 x head_dim x heads flops per (query, token)
    w = W.WORKLOADS["prefill_chunk"]
    ctx = W.context_lengths(w)
    seen = sum(3584 + i + 1 for i in range(512))
    assert runner.multi_flops(w, ctx) == 32 * seen * 4 * 128 * 32 == 1_030_926_368_768


def test_store_step_bytes_one_token():
    # one token per sequence at position ctx - 1: the block's held rows read
    # (fp16 K and V), the whole tile's codes and metadata written, the tail
    # rows of a partial block written back, four int32 arrays per sequence
    w = W.WORKLOADS["llama7b"]
    ctx = np.array([4096] * 32)
    rows = 16   # position 4095 fills its block
    expect = 32 * rows * 32 * 128 * 4 + 32 * 32 * (16 * 128 * 2 + 4) + 32 * 16
    assert runner.store_step_bytes(w, ctx) == expect
    # the same token stored again (the benchmark's repeated step): the scale
    # is unchanged, so only the token's K row and V entries are written and
    # the metadata is read
    expect_row = 32 * rows * 32 * 128 * 4 + 32 * 32 * (128 * 2 + 4) + 32 * 16
    assert runner.store_step_bytes(w, ctx, rewrite_tiles=False) == expect_row
    # INT4 V: half a byte per V code
    w4 = W.WORKLOADS["gqa70b"]
    ctx4 = np.array([33, 64])
    rows4 = np.array([1, 32])
    expect4 = (int(rows4.sum()) * 8 * 128 * 4 + 2 * 8 * (128 * 12 // 8 + 5) + 1 * 8 * 128 * 4 + 2 * 16)
    assert runner.store_step_bytes(w4, ctx4, rewrite_tiles=False) == expect4


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; asking for more ends with a message and
    # status 2 before any device is touched
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_int4_k_decode_bytes():
    # llama7b shape with INT4 K and V: 4 + 4 bits per (token, head, dim) and
    # per block and head two fp16 scales and two u8 zero points; INT4 K with
    # INT8 V: 12 bits and one zero point
    ctx = np.array([4096] * 32)
    qo_tables = 2 * 32 * 32 * 128 * 2 + 32 * 256 * 4 + 32 * 4
    w44 = W.WORKLOADS["llama7b_k4v4"]
    assert runner.decode_bytes(w44, ctx) == 32 * 4096 * 32 * 128 + 32 * 256 * 32 * 6 + qo_tables
    w48 = W.WORKLOADS["llama7b_k4v8"]
    assert runner.decode_bytes(w48, ctx) == 32 * 4096 * 32 * 192 + 32 * 256 * 32 * 5 + qo_tables

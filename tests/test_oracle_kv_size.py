"""Pins for oracle/kv_size.py against the figures the pages print
(tests/golden/page_figures.json, each value derived by hand)."""

import json
import os
from fractions import Fraction

from oracle import kv_size

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _dense(entry):
    s = entry["shape"]
    return kv_size.kv_bytes_dense(s["layers"], s["kv_heads"], s["head_dim"],
                                  s["seq_len"], s["batch"], s["bytes_per_elem"])


def test_llama2_7b_dense_and_page_discrepancy():
    e = G["llama2_7b_fp16_kv"]
    assert kv_size.kv_bytes_dense(32, 32, 128, 1, 1) == e["bytes_per_token"]
    assert _dense(e) == e["bytes"] == 2 ** 36
    # the page's "about 16 GB" is a factor 4 below the arithmetic
    assert _dense(e) // (16 * 2 ** 30) == 4


def test_llama2_7b_int8_blocks():
    e = G["llama2_7b_int8_blocks16_kv"]
    got = kv_size.kv_bytes_block_quantized(4096, 32, 32, 128, 16, 8, 8, False, 32)
    assert got == e["bytes"]


def test_llama70b_two_readings():
    g = G["llama70b_gqa_fp16_kv"]
    m = G["llama70b_mha_fp16_kv"]
    assert kv_size.kv_bytes_dense(80, 8, 128, 1, 1) == g["bytes_per_token"]
    assert _dense(g) == g["bytes"] and _dense(g) < 40e9
    assert _dense(m) == m["bytes"] and _dense(m) > 40e9


def test_memory_ratios():
    e = G["int8_memory_ratio"]
    a, b = e["k8v8_bs16_d128_ratio"]
    assert Fraction(kv_size.compression_ratio(128, 16, 8, 8, False)).limit_denominator(10 ** 6) == Fraction(a, b)
    a, b = e["k8v4_bs32_d128_ratio"]
    assert Fraction(kv_size.compression_ratio(128, 32, 8, 4, True)).limit_denominator(10 ** 6) == Fraction(a, b)
    assert kv_size.compression_ratio(128, 32, 8, 4, True) < 0.5


def test_num_blocks_for_is_ceiling():
    for bs in (1, 2, 3, 8, 16, 32):
        for n in range(0, 200):
            k = kv_size.num_blocks_for(n, bs)
            assert (k - 1) * bs < n <= k * bs or (n == 0 and k == 0)


def test_pool_sizing():
    # one C2-shaped block over 32 heads: 32 * (16*128*2 + 2 + 2) bytes
    assert kv_size.pool_block_bytes(32, 128, 16, 8, 8, False) == 32 * 4100
    # INT4 V at bs 32: 32 * (4096 + 2048 + 5)
    assert kv_size.pool_block_bytes(32, 128, 32, 8, 4, True) == 32 * 6149
    # INT4 K and V at bs 16, D 128: 16 x 128 x (4 + 4) / 8 = 2048 code bytes,
    # two fp16 scales and two u8 zero points = 2054 per head; INT4 K with
    # INT8 V: 16 x 128 x 12 / 8 = 3072 + 2 + 2 + 1 = 3077
    assert kv_size.pool_block_bytes(32, 128, 16, 4, 4, True, True) == 32 * 2054
    assert kv_size.pool_block_bytes(32, 128, 16, 4, 8, False, True) == 32 * 3077
    assert kv_size.pool_num_blocks(32 * 4100 * 1000 + 5, 32, 128, 16, 8, 8, False) == 1000

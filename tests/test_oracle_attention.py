"""Pins for oracle/paged.py and oracle/attention.py: paging indirection
against the contiguous layout, pool-permutation invariance, closed-form
special cases, a pure-Python brute force and torch's float64 SDPA."""

import math

import numpy as np
import pytest
import torch

from oracle import allocator as A
from oracle import attention, paged, quant


def _fill(rng, ctx_lens, hkv, d, bs, n_blocks, v_int4, perm, k_codec="i8", v_codec=None):
    pool = paged.PoolArrays(n_blocks, hkv, bs, d, v_int4, k_codec, v_codec)
    m = A.BlockPoolModel(n_blocks, bs, len(ctx_lens), perm)
    tables, hist = [], []
    for s, c in enumerate(ctx_lens):
        t = m.alloc(s, c)
        k = rng.standard_normal((c, hkv, d)).astype(np.float16)
        v = rng.standard_normal((c, hkv, d)).astype(np.float16)
        paged.store_range(pool, t, k, v, 0, c)
        tables.append(t)
        hist.append((k, v))
    return pool, tables, hist


@pytest.mark.parametrize("kc,vc", [("i8", "i8"), ("i8", "i4"), ("i8", "i8a"), ("fp8", "fp8"),
                                   ("i4", "i4"), ("i4", "i8")])
def test_gather_equals_contiguous(kc, vc):
    rng = np.random.default_rng(0)
    ctx = [1, 17, 50, 100]
    pool, tables, hist = _fill(rng, ctx, 2, 64, 16, 64, False, rng.permutation(64), kc, vc)
    for s, c in enumerate(ctx):
        kh, vh = paged.gather_dequant(pool, tables[s], c)
        k, v = hist[s]
        assert np.array_equal(kh, paged.quantize_contiguous(k.transpose(1, 0, 2), 16, codec=kc))
        assert np.array_equal(vh, paged.quantize_contiguous(v.transpose(1, 0, 2), 16, codec=vc))
        # and every tile by hand: codes of the rows, zero bytes past them
        for j, b in enumerate(tables[s]):
            n = min(16, c - 16 * j)
            for h in range(2):
                rows = v[16 * j:16 * j + n, h]
                codes = (quant.quantize_int8_asym(rows)[0] if vc == "i8a" else
                         quant.quantize_fp8_e4m3(rows)[0] if vc == "fp8" else None)
                if codes is not None:
                    assert np.array_equal(pool.v_codes[b, h][:, :n], codes.T)
                    assert not pool.v_codes[b, h][:, n:].any()


def test_int4_k_tile_hand_example_and_layout():
    """INT4 K: the hand-worked tile of tests/golden/quant_examples.json stored
    through the pool -- codes packed along head_dim (two consecutive dims of
    one token per byte, even dim low), scale and zero point -- rows past the
    tile zero bytes, and gathered back as (code - zp) * scale."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_examples.json")))["int4_k_tile"]
    x = np.array(g["x"], np.float16)
    k = x[:, None, :]
    v = np.zeros_like(k)
    pool = paged.PoolArrays(3, 1, 16, 4, k_codec="i4", v_codec="i8")
    paged.store_block(pool, 2, k, v)
    assert float(pool.k_scale[2, 0]) == g["scale"] and int(pool.k_zp[2, 0]) == g["zero_point"]
    assert pool.k_codes.shape == (3, 1, 16, 2)
    assert pool.k_codes[2, 0, :2].tolist() == g["bytes"]
    assert not pool.k_codes[2, 0, 2:].any()
    kh, _ = paged.gather_dequant(pool, [2], 2)
    expect = (np.array(g["codes"], np.float64) - g["zero_point"]) * g["scale"]
    assert np.array_equal(kh[0], expect)


@pytest.mark.parametrize("kc,vc", [("i4", "i4"), ("i4", "i8")])
def test_int4_k_permutation_invariance_and_append(kc, vc):
    """INT4 K pools: outputs unchanged under a permuted pool, and one-token
    appends from exact rows end with the bytes of one prefill."""
    rng = np.random.default_rng(12)
    ctx = [3, 40, 33]
    q = rng.standard_normal((3, 4, 64)).astype(np.float16)
    outs = []
    for perm_seed in (10, 11):
        r2 = np.random.default_rng(5)
        pool, tables, _ = _fill(r2, ctx, 2, 64, 16, 16, False,
                                np.random.default_rng(perm_seed).permutation(16), kc, vc)
        outs.append(attention.paged_decode(pool, tables, ctx, q, 0.125))
    assert np.array_equal(outs[0], outs[1])
    k = rng.standard_normal((40, 2, 64)).astype(np.float16)
    v = rng.standard_normal((40, 2, 64)).astype(np.float16)
    pre = paged.PoolArrays(8, 2, 16, 64, k_codec=kc, v_codec=vc)
    app = paged.PoolArrays(8, 2, 16, 64, k_codec=kc, v_codec=vc)
    table = [4, 1, 6]
    paged.store_range(pre, table, k, v, 0, 40)
    paged.store_range(app, table, k, v, 0, 3)
    for p in range(3, 40):
        paged.store_range(app, table, k, v, p, p + 1)
    for arr in ("k_codes", "v_codes", "k_scale", "v_scale", "v_zp", "k_zp"):
        assert np.array_equal(getattr(pre, arr), getattr(app, arr)), arr


def test_rows_beyond_context_are_zero_and_ignored():
    rng = np.random.default_rng(1)
    pool, tables, hist = _fill(rng, [5], 1, 64, 16, 4, True, None)
    b = tables[0][0]
    assert not pool.k_codes[b, :, 5:].any()
    vt = quant.unpack_int4(pool.v_codes[b])          # [H, D, bs], dim-major V tile
    assert not vt[:, :, 5:].any() and vt[:, :, :5].any()


def test_permutation_invariance():
    rng = np.random.default_rng(2)
    ctx = [3, 40, 33]
    q = rng.standard_normal((3, 4, 64)).astype(np.float16)
    outs = []
    for perm_seed in (10, 11):
        r2 = np.random.default_rng(5)
        pool, tables, _ = _fill(r2, ctx, 2, 64, 16, 16, False,
                                np.random.default_rng(perm_seed).permutation(16))
        outs.append(attention.paged_decode(pool, tables, ctx, q, 0.125))
    assert np.array_equal(outs[0], outs[1])


def test_append_equals_prefill():
    """Re-quantizing a partial block from its exact rows after each one-token
    append ends with the same bytes as quantizing the full block once."""
    rng = np.random.default_rng(3)
    bs, h, d = 16, 2, 64
    k = rng.standard_normal((40, h, d)).astype(np.float16)
    v = rng.standard_normal((40, h, d)).astype(np.float16)
    pre = paged.PoolArrays(8, h, bs, d, True)
    app = paged.PoolArrays(8, h, bs, d, True)
    table = [4, 1, 6]
    paged.store_range(pre, table, k, v, 0, 40)
    paged.store_range(app, table, k, v, 0, 3)
    for p in range(3, 40):
        paged.store_range(app, table, k, v, p, p + 1)
    for arr in ("k_codes", "v_codes", "k_scale", "v_scale", "v_zp"):
        assert np.array_equal(getattr(pre, arr), getattr(app, arr)), arr


def test_ctx1_identical_keys_dominant_key():
    rng = np.random.default_rng(4)
    d = 64
    v = rng.standard_normal((1, 9, d))
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, 9, d))
    # ctx = 1: the output is the single value row
    assert np.array_equal(attention.decode_attention(q, k[:, :1], v[:, :1], 0.3)[0], v[0, 0])
    # identical keys: uniform weights -> mean of the values
    ksame = np.repeat(k[:, :1], 9, axis=1)
    out = attention.decode_attention(q, ksame, v, 0.3)[0]
    assert np.allclose(out, v[0].mean(0), rtol=0, atol=1e-12)
    # one dominant key: weight ~1 on its row
    kdom = np.zeros((1, 9, d))
    kdom[0, 4] = 1000.0 * q[0] / np.linalg.norm(q[0])
    out = attention.decode_attention(q, kdom, v, 1.0)[0]
    assert np.allclose(out, v[0, 4], rtol=0, atol=1e-12)
    # empty context -> zeros
    assert not attention.decode_attention(q, k[:, :0], v[:, :0], 1.0).any()


def test_brute_force_pure_python_tiny():
    rng = np.random.default_rng(6)
    hq, hkv, ctx, d = 4, 2, 7, 8
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, ctx, d))
    v = rng.standard_normal((hkv, ctx, d))
    out = attention.decode_attention(q, k, v, 0.7)
    for h in range(hq):
        g = h // 2
        sc = [0.7 * sum(q[h][i] * k[g][t][i] for i in range(d)) for t in range(ctx)]
        w = [math.exp(x - max(sc)) for x in sc]
        z = sum(w)
        for i in range(d):
            ref = sum(w[t] * v[g][t][i] for t in range(ctx)) / z
            assert abs(out[h][i] - ref) < 1e-12


@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2), (64, 8)])
def test_against_torch_sdpa_float64(hq, hkv):
    rng = np.random.default_rng(hq)
    ctx, d = 70, 128
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, ctx, d))
    v = rng.standard_normal((hkv, ctx, d))
    out = attention.decode_attention(q, k, v, 1 / math.sqrt(d))
    rep = hq // hkv
    kt = torch.from_numpy(np.repeat(k, rep, axis=0))[None]
    vt = torch.from_numpy(np.repeat(v, rep, axis=0))[None]
    qt = torch.from_numpy(q)[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_tiny_config_end_to_end_quantized():
    """The tiny decode shape: 4 sequences {1,17,50,100}, 2 heads, D=64,
    bs=16 over a permuted 64-block pool; the paged result equals attention
    over the contiguous quantize->dequantize of each sequence."""
    rng = np.random.default_rng(8)
    ctx = [1, 17, 50, 100]
    pool, tables, hist = _fill(rng, ctx, 2, 64, 16, 64, False, rng.permutation(64))
    q = rng.standard_normal((4, 2, 64)).astype(np.float16)
    out = attention.paged_decode(pool, tables, ctx, q, 1 / 8)
    for s, c in enumerate(ctx):
        k, v = hist[s]
        kh = paged.quantize_contiguous(k.transpose(1, 0, 2), 16)
        vh = paged.quantize_contiguous(v.transpose(1, 0, 2), 16)
        assert np.array_equal(out[s], attention.decode_attention(q[s], kh, vh, 1 / 8))
    # ctx = 1 sequence: output equals its dequantized single V row
    k0, v0 = hist[0]
    c, sc = quant.quantize_int8_sym(v0[:, 0, :])
    assert np.array_equal(out[0, 0], quant.dequantize_int8_sym(c, sc)[0])


def test_v_tile_layout_dim_major():
    """V tiles are stored [head_dim, block_size] per (block, head); INT4 packs
    two consecutive tokens per byte with the earlier token in the low nibble.
    Values are chosen so that the scale is exactly 1 and the codes are known."""
    bs, d = 16, 64
    k = np.zeros((bs, 1, d), np.float16)
    v = np.zeros((bs, 1, d), np.float16)
    v[0, 0, 0] = 127.0                          # absmax 127 -> INT8 scale 1
    v[:, 0, 3] = np.arange(1, bs + 1)           # dim 3 holds token index + 1
    pool = paged.PoolArrays(2, 1, bs, d, False)
    paged.store_block(pool, 1, k, v)
    assert float(pool.v_scale[1, 0]) == 1.0
    assert pool.v_codes[1, 0, 3].tolist() == list(range(1, bs + 1))
    assert pool.v_codes[1, 0, 0, 0] == 127 and not pool.v_codes[1, 0, 0, 1:].any()
    v4 = np.zeros((bs, 1, d), np.float16)
    v4[:, 0, 5] = np.arange(bs) % 16            # lo 0, hi 15 -> scale 1, zp 0
    pool4 = paged.PoolArrays(2, 1, bs, d, True)
    paged.store_block(pool4, 0, k, v4)
    assert float(pool4.v_scale[0, 0]) == 1.0 and int(pool4.v_zp[0, 0]) == 0
    assert pool4.v_codes[0, 0, 5].tolist() == [(2 * j) | ((2 * j + 1) << 4) for j in range(bs // 2)]
    assert not pool4.v_codes[0, 0, 4].any()


@pytest.mark.parametrize("n,ctx,hq,hkv", [(5, 5, 2, 2), (7, 20, 4, 2), (1, 9, 3, 1), (16, 16, 8, 1)])
def test_multi_query_matches_torch_causal_sdpa(n, ctx, hq, hkv):
    """The last n tokens attending causally equal torch's float64 SDPA with
    a causal mask shifted by ctx - n (is_causal itself when n == ctx)."""
    rng = np.random.default_rng(n * 100 + ctx)
    d = 32
    k = rng.standard_normal((hkv, ctx, d))
    v = rng.standard_normal((hkv, ctx, d))
    q = rng.standard_normal((n, hq, d)).astype(np.float16)
    sm = 0.3
    got = attention.multi_query_attention(q, k, v, sm)
    g = hq // hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)              # [Hq, n, D]
    kt = torch.from_numpy(k).repeat_interleave(g, 0)
    vt = torch.from_numpy(v).repeat_interleave(g, 0)
    mask = torch.ones(n, ctx, dtype=torch.bool).tril(diagonal=ctx - n)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sm)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    if n == ctx:
        ref2 = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=sm)
        assert np.allclose(got, ref2.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    # the last query sees everything: the single-query definition
    assert np.allclose(got[-1], attention.decode_attention(q[-1], k, v, sm), rtol=0, atol=0)

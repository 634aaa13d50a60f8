"""CPU tests of libpbq's C ABI: the library loads and exports every entry
point include/pbq.h declares; its host allocator matches the oracle's model
bit for bit; sizing and argument validation behave as documented.  No device
computation is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as hst

from oracle import allocator as A
from oracle import kv_size

from alloc_harness import apply_op, random_ops, run_golden_trace

pbq = pytest.importorskip("paged_block_quantized_amd")
from paged_block_quantized_amd import _lib as L  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "pbq.h")).read()
    return re.findall(r"^(?:kv_status|void|size_t|int32_t|const char\*)\s+(\w+)\(", text, re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libpbq.so is not built (run python -m paged_block_quantized_amd.build)")
    return L.lib()


def test_exports_every_header_symbol(lib):
    names = _header_functions()
    assert len(names) >= 17
    assert sorted(names) == sorted(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


class CAdapter:
    """The C allocator behind the same interface as the oracle model."""

    def __init__(self, n, bs, max_seqs, free_order):
        desc = L.make_desc(n, bs, 1, 1, max_seqs=max_seqs)
        self.h = L.kv_pool_create(desc, free_order)

    def alloc(self, s, n):
        L.kv_seq_alloc(self.h, s, n)
        return L.kv_seq_table(self.h, s)[0]

    def alloc_prefix(self, s, toks):
        cached = L.kv_seq_alloc_prefix(self.h, s, toks)
        return L.kv_seq_table(self.h, s)[0], cached

    def fork(self, p, c):
        return L.kv_seq_fork(self.h, p, c)

    def append(self, s, n):
        return L.kv_seq_append(self.h, s, n)

    def release(self, s):
        return L.kv_seq_free(self.h, s)

    def set_swap_space(self, hb, hs):
        L.kv_pool_set_swap_space(self.h, hb, hs)

    def swap_out(self, seqs):
        return L.kv_seq_swap_out(self.h, seqs)

    def swap_in(self, seqs):
        return L.kv_seq_swap_in(self.h, seqs)

    def table(self, s):
        return L.kv_seq_table(self.h, s)

    def stats(self):
        return L.kv_pool_stats(self.h)

    def free_list(self):
        return L.kv_pool_free_list(self.h)

    def __del__(self):
        L.kv_pool_destroy(self.h)


def test_golden_trace_c(lib):
    run_golden_trace(CAdapter, L.PBQError)


@settings(max_examples=80, deadline=None)
@given(seed=hst.integers(0, 2 ** 31 - 1), n_blocks=hst.integers(1, 24),
       bs=hst.sampled_from([1, 2, 4, 16, 32]))
def test_c_allocator_matches_model(lib, seed, n_blocks, bs):
    """Every operation, prefix-cached allocation included, bit for bit."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_blocks)
    model = A.BlockPoolModel(n_blocks, bs, 6, perm)
    c = CAdapter(n_blocks, bs, 6, perm)
    for op in random_ops(rng, 120, prefix=True):
        a = apply_op(model, op, A.AllocError)
        b = apply_op(c, op, L.PBQError)
        assert a == b, op
        assert model.free == c.free_list()
        assert model.stats() == c.stats()
    for sid, st in model.seqs.items():
        assert (st.table, st.num_tokens, st.slot) == tuple(c.table(sid))


@settings(max_examples=80, deadline=None)
@given(seed=hst.integers(0, 2 ** 31 - 1), n_blocks=hst.integers(1, 24),
       bs=hst.sampled_from([1, 2, 4, 16]), host_blocks=hst.integers(0, 16))
def test_c_swap_matches_model(lib, seed, n_blocks, bs, host_blocks):
    """Swap-out / swap-in plans, tables (host blocks as -1 - h), slots, free
    stacks and stats equal the model's after every op, failures included."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_blocks)
    model = A.BlockPoolModel(n_blocks, bs, 6, perm)
    c = CAdapter(n_blocks, bs, 6, perm)
    model.set_swap_space(host_blocks, 3)
    c.set_swap_space(host_blocks, 3)
    for op in random_ops(rng, 160, max_seq_id=6, prefix=True, swap=True):
        a = apply_op(model, op, A.AllocError)
        b = apply_op(c, op, L.PBQError)
        assert a == b, op
        assert model.free == c.free_list()
        assert model.stats() == c.stats()
        for sid, st in model.seqs.items():
            assert (st.table, st.num_tokens, st.slot) == tuple(c.table(sid))


def test_swap_allocator_errors(lib):
    c = CAdapter(8, 4, 2, None)
    c.set_swap_space(2, 1)
    c.alloc(0, 5)
    with pytest.raises(L.PBQError) as e:
        c.swap_in([0])
    assert e.value.kind == "state"
    buf = (L.kv_swap * 1)()
    n = ctypes.c_int32()
    sq = (ctypes.c_int64 * 1)(0)
    with pytest.raises(L.PBQError, match="cap"):       # two blocks and a slot need 3 entries
        L._check(L.lib().kv_seq_swap_out(c.h, sq, 1, buf, 1, ctypes.byref(n)))
    assert c.stats()["swapped"] == 0
    assert c.swap_out([0]) == [(L.KV_SWAP_BLOCK_OUT, 7, 1, 0), (L.KV_SWAP_BLOCK_OUT, 6, 0, 0),
                               (L.KV_SWAP_SLOT_OUT, 0, 0, 1)]
    with pytest.raises(L.PBQError) as e:
        L.kv_batch_tables(c.h, [0], 4)
    assert e.value.kind == "state"
    with pytest.raises(L.PBQError) as e:
        c.set_swap_space(4, 4)
    assert e.value.kind == "state"
    assert c.table(0) == ([-2, -1], 5, -1)
    c.release(0)
    assert c.stats()["host_free"] == 2 and c.stats()["swapped"] == 0


def test_swap_blocks_validates_plan_on_host(lib):
    """kv_swap_blocks checks every plan entry before anything reaches HIP;
    host memory that HIP does not know as pinned is refused."""
    desc = L.make_desc(8, 16, 2, 64, max_seqs=2)
    hdesc = L.make_desc(4, 16, 2, 64, max_seqs=1)
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 15) & ~15
    mem = L.kv_pool_mem(base, base, base, base, None, base, base)

    def run(entries, hd=hdesc):
        plan = (L.kv_swap * max(1, len(entries)))(*[L.kv_swap(*e) for e in entries])
        L.kv_swap_blocks(desc, mem, hd, mem, ctypes.addressof(plan), len(entries), 0)

    O, I, SO, SI = L.KV_SWAP_BLOCK_OUT, L.KV_SWAP_BLOCK_IN, L.KV_SWAP_SLOT_OUT, L.KV_SWAP_SLOT_IN
    with pytest.raises(L.PBQError, match="unknown kind"):
        run([(7, 0, 0, 0)])
    with pytest.raises(L.PBQError, match="out of range"):
        run([(O, 8, 0, 0)])                  # device block 8 of 8
    with pytest.raises(L.PBQError, match="out of range"):
        run([(O, 0, 4, 0)])                  # host block 4 of 4
    with pytest.raises(L.PBQError, match="out of range"):
        run([(SI, 1, 0, 3)])                 # host slot 1 of 1
    with pytest.raises(L.PBQError, match="rows"):
        run([(SO, 0, 0, 0)])
    with pytest.raises(L.PBQError, match="rows"):
        run([(SO, 0, 0, 17)])
    with pytest.raises(L.PBQError, match="rows"):
        run([(O, 0, 0, 1)])
    with pytest.raises(L.PBQError, match="written twice"):
        run([(O, 0, 1, 0), (O, 2, 1, 0)])
    with pytest.raises(L.PBQError, match="written twice or also read"):
        run([(O, 3, 1, 0), (I, 2, 3, 0)])    # device block 3 read and written
    with pytest.raises(L.PBQError, match="written twice or also read"):
        run([(SO, 1, 0, 2), (SI, 0, 1, 2)])  # host slot 0 written, then read
    with pytest.raises(L.PBQError, match="host_desc"):
        run([(O, 0, 0, 0)], L.make_desc(4, 32, 2, 64, max_seqs=1))
    with pytest.raises(L.PBQError, match="pinned"):
        run([(O, 0, 0, 0), (I, 1, 2, 0), (SO, 0, 0, 5)])
    run([])                                  # nothing to do: no device work

    c = CAdapter(16, 4, 4, None)
    c.alloc(7, 9)
    c.alloc(3, 1)
    t, ctx, slots = L.kv_batch_tables(c.h, [3, 7], 5)
    assert t.tolist() == [c.table(3)[0] + [0] * 4, c.table(7)[0] + [0] * 2]
    assert ctx.tolist() == [1, 9] and slots.tolist() == [1, 0]
    with pytest.raises(L.PBQError):
        L.kv_batch_tables(c.h, [7], 2)
    with pytest.raises(L.PBQError) as e:
        L.kv_batch_tables(c.h, [8], 5)
    assert e.value.kind == "unknown_seq"


def test_pool_bytes_match_closed_form(lib):
    for bs, D, H, v4, k4, N in [(16, 128, 32, False, False, 8192), (32, 128, 8, True, False, 1000),
                                (16, 64, 2, False, False, 64), (16, 128, 32, True, True, 8192),
                                (32, 64, 3, False, True, 77)]:
        desc = L.make_desc(N, bs, H, D, L.KV_CODEC_I4_ASYM if v4 else L.KV_CODEC_I8_SYM, 3,
                           k_codec=L.KV_CODEC_I4_ASYM if k4 else L.KV_CODEC_I8_SYM)
        sz = L.kv_pool_bytes(desc)
        per_block = sum(sz[n] for n in ("k_codes", "v_codes", "k_scale", "v_scale", "v_zp", "k_zp")) // N
        assert per_block == kv_size.pool_block_bytes(H, D, bs, 4 if k4 else 8, 4 if v4 else 8, v4, k4)
        assert sz["tail_k"] == sz["tail_v"] == 3 * H * bs * D * 2
        assert sz["k_zp"] == (N * H if k4 else 0)


def test_create_rejects_bad_arguments(lib):
    with pytest.raises(L.PBQError) as e:
        L.kv_pool_create(L.make_desc(4, 16, 1, 64), [0, 1, 1, 2])
    assert e.value.kind == "invalid"
    with pytest.raises(L.PBQError):
        L.kv_pool_create(L.make_desc(0, 16, 1, 64))
    with pytest.raises(L.PBQError):
        L.kv_pool_bytes(L.make_desc(4, 8, 1, 64))      # block_size 8 has no kernel
    with pytest.raises(L.PBQError):
        L.kv_pool_bytes(L.make_desc(4, 16, 1, 96))     # head_dim 96 has no kernel
    with pytest.raises(L.PBQError):
        L.kv_pool_bytes(L.make_desc(4, 16, 1, 64, v_codec=7))
    # codec pairs: FP8 K goes with FP8 V only, FP8 V with FP8 K only, INT4 K
    # with INT4 or INT8 V
    for kc, vc in ((L.KV_CODEC_I8_SYM, L.KV_CODEC_FP8_E4M3), (L.KV_CODEC_FP8_E4M3, L.KV_CODEC_I4_ASYM),
                   (L.KV_CODEC_I4_ASYM, L.KV_CODEC_I8_ASYM), (L.KV_CODEC_I4_ASYM, L.KV_CODEC_FP8_E4M3),
                   (L.KV_CODEC_I8_ASYM, L.KV_CODEC_I8_ASYM)):
        with pytest.raises(L.PBQError, match="unsupported"):
            L.kv_pool_bytes(L.make_desc(4, 16, 1, 64, v_codec=vc, k_codec=kc))


def test_codec_pair_sizes(lib):
    """Byte codecs (FP8, INT8 asymmetric) take one byte per value; the
    asymmetric ones add a zero point per (block, head)."""
    N, H, bs, D = 10, 3, 32, 128
    f8 = L.kv_pool_bytes(L.make_desc(N, bs, H, D, L.KV_CODEC_FP8_E4M3, 2, k_codec=L.KV_CODEC_FP8_E4M3))
    i8a = L.kv_pool_bytes(L.make_desc(N, bs, H, D, L.KV_CODEC_I8_ASYM, 2))
    for sz in (f8, i8a):
        assert sz["k_codes"] == sz["v_codes"] == N * H * bs * D
        assert sz["k_scale"] == sz["v_scale"] == N * H * 2
    assert f8["v_zp"] == 0 and i8a["v_zp"] == N * H


def test_device_calls_validate_before_launch(lib):
    """Invalid arguments are rejected on the host; nothing reaches HIP."""
    desc = L.make_desc(8, 16, 2, 64)
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 15) & ~15
    mem = L.kv_pool_mem(base, base, base, base, None, base, base)
    with pytest.raises(L.PBQError, match="multiple of num_kv_heads"):
        L.paged_attn_decode(desc, mem, base, base, 1, 3, base, 4, base, 64, 0.1, 0, None, 0, 0)
    with pytest.raises(L.PBQError, match="partition_size"):
        L.paged_attn_decode(desc, mem, base, base, 1, 2, base, 4, base, 64, 0.1, 24, None, 0, 0)
    with pytest.raises(L.PBQError, match="max_blocks_per_seq"):
        L.paged_attn_decode(desc, mem, base, base, 1, 2, base, 2, base, 64, 0.1, 0, None, 0, 0)
    with pytest.raises(L.PBQError, match="workspace"):
        L.paged_attn_decode(desc, mem, base, base, 1, 2, base, 64, base, 1024, 0.1, 16, None, 0, 0)
    with pytest.raises(L.PBQError, match="aligned"):
        L.paged_attn_decode(desc, mem, base + 2, base, 1, 2, base, 4, base, 64, 0.1, 0, None, 0, 0)
    with pytest.raises(L.PBQError, match="finite"):
        L.paged_attn_decode(desc, mem, base, base, 1, 2, base, 4, base, 64, float("nan"), 0, None, 0, 0)
    bad = L.kv_pool_mem(base + 1, base, base, base, None, base, base)
    with pytest.raises(L.PBQError, match="aligned"):
        L.kv_quantize_store(desc, bad, base, base, 1, base, base, base, 4, base, 1, 0)
    desc4 = L.make_desc(8, 16, 2, 64, L.KV_CODEC_I4_ASYM)
    with pytest.raises(L.PBQError, match="v_zp"):
        L.kv_copy_blocks(desc4, mem, base, 1, 0)
    # the fused store + decode checks its new-token arguments as well
    with pytest.raises(L.PBQError, match="k_new"):
        L.paged_attn_decode_append(desc, mem, None, base, base, base, base, 1, 2, base, 4, base,
                                   64, 0.1, 0, None, 0, 0)
    with pytest.raises(L.PBQError, match="k_new"):
        L.paged_attn_decode_append(desc, mem, base + 4, base, base, base, base, 1, 2, base, 4,
                                   base, 64, 0.1, 0, None, 0, 0)
    with pytest.raises(L.PBQError, match="tail_slots"):
        L.paged_attn_decode_append(desc, mem, base, base, None, base, base, 1, 2, base, 4, base,
                                   64, 0.1, 0, None, 0, 0)
    no_tail = L.kv_pool_mem(base, base, base, base, None, None, None)
    with pytest.raises(L.PBQError, match="tail slots"):
        L.paged_attn_decode_append(desc, no_tail, base, base, base, base, base, 1, 2, base, 4,
                                   base, 64, 0.1, 0, None, 0, 0)
    with pytest.raises(L.PBQError, match="multiple of num_kv_heads"):
        L.paged_attn_decode_append(desc, mem, base, base, base, base, base, 1, 3, base, 4, base,
                                   64, 0.1, 0, None, 0, 0)
    # the shared-prefix form checks its prefix and partition arguments
    sp = L.paged_attn_decode_shared_prefix
    with pytest.raises(L.PBQError, match="shared_tokens must be >= 0"):
        sp(desc, mem, None, None, None, base, base, 1, 2, base, 8, base, 128, 0.1, 64, -64, None, 0, 0)
    with pytest.raises(L.PBQError, match="explicit partition_size"):
        sp(desc, mem, None, None, None, base, base, 1, 2, base, 8, base, 128, 0.1, 0, 64, None, 0, 0)
    with pytest.raises(L.PBQError, match="multiple of 32"):
        sp(desc, mem, None, None, None, base, base, 1, 2, base, 8, base, 128, 0.1, 48, 96, None, 0, 0)
    with pytest.raises(L.PBQError, match="multiple of partition_size"):
        sp(desc, mem, None, None, None, base, base, 1, 2, base, 8, base, 128, 0.1, 64, 96, None, 0, 0)
    with pytest.raises(L.PBQError, match="below max_context_len"):
        sp(desc, mem, None, None, None, base, base, 1, 2, base, 8, base, 128, 0.1, 64, 128, None, 0, 0)
    with pytest.raises(L.PBQError, match="all NULL"):
        sp(desc, mem, None, base, None, base, base, 1, 2, base, 8, base, 128, 0.1, 64, 64, None, 0, 0)
    # zero-sized work is a no-op that succeeds without touching the device
    L.kv_quantize_store(desc, mem, base, base, 0, base, base, base, 4, base, 0, 0)
    L.paged_attn_decode_append(desc, mem, base, base, base, base, base, 0, 2, base, 4, base, 64,
                               0.1, 0, None, 0, 0)
    L.kv_copy_blocks(desc, mem, None, 0, 0)


def test_multi_query_validates_before_launch(lib):
    """paged_attn_multi_query checks its sizes, pointers, partition and
    workspace on the host; zero tokens is a no-op."""
    desc = L.make_desc(8, 16, 2, 64)
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 15) & ~15
    mem = L.kv_pool_mem(base, base, base, base, None, base, base)
    def mq(*args):
        args = list(args) + [0] * (15 - len(args))       # partition_size 0 by default
        return L.paged_attn_multi_query(*args, workspace=None, workspace_bytes=0, stream=0)
    with pytest.raises(L.PBQError, match="multiple of num_kv_heads"):
        mq(desc, mem, base, base, 1, 3, base, 4, 4, base, 4, base, 64, 0.1)
    with pytest.raises(L.PBQError, match="max_q_len"):
        mq(desc, mem, base, base, 1, 2, base, 4, 0, base, 4, base, 64, 0.1)
    with pytest.raises(L.PBQError, match="max_q_len"):
        mq(desc, mem, base, base, 1, 2, base, 4, 65, base, 8, base, 64, 0.1)
    with pytest.raises(L.PBQError, match="multiple of 32"):
        mq(desc, mem, base, base, 1, 2, base, 4, 4, base, 4, base, 64, 0.1, 48)
    with pytest.raises(L.PBQError, match="max_blocks_per_seq"):
        mq(desc, mem, base, base, 1, 2, base, 4, 4, base, 2, base, 64, 0.1)
    with pytest.raises(L.PBQError, match="aligned"):
        mq(desc, mem, base + 2, base, 1, 2, base, 4, 4, base, 4, base, 64, 0.1)
    with pytest.raises(L.PBQError, match="workspace"):
        mq(desc, mem, base, base, 1, 2, base, 4, 4, base, 64, base, 1024, 0.1, 32)
    with pytest.raises(L.PBQError, match="tiles"):
        mq(L.make_desc(8, 16, 1, 64), mem, base, base, 1, 64, base, 40000, 40000, base, 2500, base,
           40000, 0.1, 64)
    mq(desc, mem, base, base, 1, 2, base, 0, 0, base, 4, base, 64, 0.1)   # nothing to do
    # workspace: one row of (D + 2) floats per query token, head and partition
    assert L.paged_attn_multi_query_workspace_bytes(desc, 2, 10, 2, 5, 1024, 256) == 10 * 2 * 4 * (64 * 4 + 8)
    assert L.paged_attn_multi_query_workspace_bytes(desc, 2, 10, 2, 5, 256, 256) == 0


def test_workspace_bytes(lib):
    desc = L.make_desc(8192, 16, 32, 128)
    # 32 seqs x 32 heads x 8 partitions x (128 floats + max + sum)
    assert L.paged_attn_workspace_bytes(desc, 32, 32, 4096, 512) == 32 * 32 * 8 * (128 * 4 + 8)
    assert L.paged_attn_workspace_bytes(desc, 32, 32, 512, 512) == 0
    assert L.paged_attn_default_partition(desc, 32, 32, 4096) % 32 == 0


def test_default_partition_policy(lib):
    """One pass when the sequence x head units fill the GPU (four work
    groups per compute unit; 256 when no device can be queried) and contexts
    fit in 4096 tokens; otherwise 2048-token partitions, halved to 256 while
    the grid is small."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    mha = L.make_desc(8192, 16, 32, 128)
    gqa = L.make_desc(8192, 32, 8, 128)
    target = 4 * cus
    if 32 * 32 >= target:
        assert L.paged_attn_default_partition(mha, 32, 32, 4096) == 4096
    assert L.paged_attn_default_partition(mha, 32, 32, 4000) % 32 == 0
    # long contexts: 2048-token partitions when the grid is large enough
    assert L.paged_attn_default_partition(mha, 32, 32, 32768) == 2048
    # one sequence, one head: the smallest partition
    assert L.paged_attn_default_partition(mha, 1, 32, 4096) == 256
    # grouped query heads count KV heads x 16-head tiles
    p = L.paged_attn_default_partition(gqa, 128, 64, 1968)
    assert p == (1984 if 128 * 8 >= target else p) and p % 32 == 0
    assert lib.paged_attn_default_partition(None, 1, 1, 1) == 0


def test_stream_read_validates_before_launch(lib):
    """kv_stream_read_tiles checks tile size, sizes, pointers and the sink on
    the host; zero tiles is a no-op."""
    buf = ctypes.create_string_buffer(1 << 14)
    base = (ctypes.addressof(buf) + 15) & ~15
    f = lib.kv_stream_read_tiles
    assert f(base, 4, 3000, None, 4, base, 1024, None) == L.KV_ERR_INVALID
    assert "tile_bytes" in lib.kv_last_error().decode()
    assert f(base, 4, 2048, None, 5, base, 1024, None) == L.KV_ERR_INVALID
    assert "n_src_tiles" in lib.kv_last_error().decode()
    assert f(base + 4, 4, 2048, None, 4, base, 1024, None) == L.KV_ERR_INVALID
    assert f(base, 4, 2048, None, 4, None, 1024, None) == L.KV_ERR_INVALID
    assert f(base, 4, 2048, None, 4, base, 0, None) == L.KV_ERR_INVALID
    assert "sink" in lib.kv_last_error().decode()
    assert f(base, 4, 2048, None, 0, base, 0, None) == L.KV_OK
    assert lib.kv_stream_read_sink_words(0) == 0
    assert lib.kv_stream_read_sink_words(1) >= 1


def test_noalloc_validates_before_touching_the_device(lib):
    """paged_attn_decode_append_noalloc checks its arguments, and that the
    call's workspace fits the library's 64 MiB scratch, before it looks up
    the scratch or launches anything; zero sequences is a no-op."""
    desc = L.make_desc(8, 16, 2, 64)
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 15) & ~15
    mem = L.kv_pool_mem(base, base, base, base, None, base, base)
    f = L.paged_attn_decode_append_noalloc
    with pytest.raises(L.PBQError, match="multiple of num_kv_heads"):
        f(desc, mem, base, base, base, base, base, 1, 3, base, 4, base, 64, 0.1, 0, 0)
    with pytest.raises(L.PBQError, match="k_new"):
        f(desc, mem, None, base, base, base, base, 1, 2, base, 4, base, 64, 0.1, 0, 0)
    with pytest.raises(L.PBQError, match="partition_size"):
        f(desc, mem, base, base, base, base, base, 1, 2, base, 4, base, 64, 0.1, 24, 0)
    # 4096 sequences x 2 heads x 256 partitions x (64 x 4 + 8) bytes > 64 MiB
    assert L.paged_attn_workspace_bytes(desc, 4096, 2, 65536, 256) > 64 << 20
    with pytest.raises(L.PBQError, match="scratch"):
        f(desc, mem, base, base, base, base, base, 4096, 2, base, 4096, base, 65536, 0.1, 256, 0)
    f(desc, mem, base, base, base, base, base, 0, 2, base, 4, base, 64, 0.1, 0, 0)


def test_debug_checks_toggle(lib):
    """kv_set_debug_checks returns the previous setting; the checks are off
    unless PBQ_DEBUG_CHECKS asks for them."""
    env_on = os.environ.get("PBQ_DEBUG_CHECKS", "0") not in ("", "0")
    first = L.kv_set_debug_checks(True)
    assert first == (1 if env_on else 0)
    assert L.kv_set_debug_checks(False) == 1
    assert L.kv_set_debug_checks(first) == 0

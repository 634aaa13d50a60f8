"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
small and ragged cases: quantized codes, fp16 scale bits, zero points and
block tables bit-exact; attention outputs within |d| <= 2e-3 + 1e-2 |ref|."""

import numpy as np
import pytest
import torch

from oracle import allocator as A
from oracle import attention, paged

from gpu_util import (SmallCase, announce, assert_close, assert_pool_equal, codecs, make_pool, normal_case,
                      opool_for, zp_arrays)

pytestmark = pytest.mark.gpu


def _tiny_inputs():
    from paged_block_quantized_amd import workloads as W
    w = W.WORKLOADS["tiny"]
    ctx = W.context_lengths(w)
    hk, hv = [], []
    for s, c in enumerate(ctx):
        k, v = W.kv_tokens(w, s, int(c), "cpu")
        hk.append(k.numpy())
        hv.append(v.numpy())
    q = W.queries(w, "cpu").numpy()
    return w, hk, hv, q


@pytest.mark.parametrize("partition", [0, 16, 32, 48])
def test_tiny_workload(partition):
    announce("tiny", partition)
    w, hk, hv, q = _tiny_inputs()
    from paged_block_quantized_amd import workloads as W
    case = SmallCase(hk, hv, q, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                     w.v_codec, w.pool_blocks, W.free_order(w, w.pool_blocks))
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    out = case.decode(partition)
    assert_close(out, case.reference(), "tiny")
    # ctx = 1: the output is that token's dequantized V row (fp16-rounded)
    vrow = paged.gather_dequant(case.opool, case.model.table(0)[0], 1)[1][:, 0, :]
    assert np.array_equal(out[0], vrow.astype(np.float16))


SHAPES = [(bs, d, vc) for bs in (16, 32) for d in (64, 128) for vc in ("i8", "i4", "i8a", "fp8", "k4i4", "k4i8")]


@pytest.mark.parametrize("bs,d,vc", SHAPES)
def test_shapes_ragged(bs, d, vc):
    announce("ragged", bs, d, vc)
    ctx = [1, bs - 1, bs, bs + 1, 3 * bs + 5, 700, 257, 2100]
    case = normal_case(ctx, 3, 3, d, bs, vc, seed=bs * 1000 + d + (vc == "i4"))
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    ref = case.reference()
    # 64 * bs: partitions of 64 blocks take the 8-wave kernel, with a reduce
    for part in (0, bs, 4 * bs, 128 if bs == 16 else 256, 64 * bs):
        assert_close(case.decode(part), ref, f"ragged bs{bs} d{d} {vc} part{part}")


def test_zero_context_and_zero_blocks():
    announce("zero")
    rng = np.random.default_rng(5)
    d, bs = 128, 16
    hk = [np.zeros((0, 1, d), np.float16), np.zeros((20, 1, d), np.float16),
          rng.standard_normal((33, 1, d)).astype(np.float16)]
    hv = [np.zeros((0, 1, d), np.float16), np.zeros((20, 1, d), np.float16),
          rng.standard_normal((33, 1, d)).astype(np.float16)]
    hv[2][16:32] = 0           # an all-zero V block between non-zero ones
    hk[2][:16] = np.float16(0.5)  # a constant K block
    q = rng.standard_normal((3, 1, d)).astype(np.float16)
    for vc in ("i8", "i4", "i8a", "fp8", "k4i4", "k4i8"):
        case = SmallCase(hk, hv, q, 1, 1, d, bs, vc, 8, rng.permutation(8))
        case.store_all()
        assert_pool_equal(case.pool, case.opool)
        out = case.decode(16)
        assert not out[0].any(), "ctx 0 must give a zero row"
        assert not out[1].any(), "all-zero K/V must give a zero row"
        assert_close(out, case.reference(), f"zero {vc}")


def test_rounding_ties():
    """Values that sit exactly on half-way points of the code grid."""
    announce("ties")
    d, bs = 64, 16
    base = np.arange(-64, 64, dtype=np.float64)[:d]
    rows = []
    for r in range(bs):
        x = (base + 0.5) * (1.0 if r % 2 else 0.25)
        x[0] = 127.0 if r % 3 else -127.0        # absmax -> scale 1 or a round value
        rows.append(x)
    k = np.array(rows, np.float16)[:, None, :]
    v = np.array(rows, np.float16)[::-1][:, None, :].copy()
    v4 = np.array([[-5.0, 10.0, 2.5, -0.5, 3.5] * 12 + [0.5, 1.5, -4.5, 7.5]] * bs, np.float16)[:, None, :]
    # INT8 asymmetric: range 8 - (-7.9375) = 255/16, so scale 1/16 and zero
    # point 127; (m + 1/2)/16 lands x/s + zp on half-integers
    v8 = np.array([[8.0, -7.9375] + [(m + 0.5) / 16 for m in range(-31, 31)]] * bs, np.float16)[:, None, :]
    # FP8: absmax 448 gives scale 1; midpoints of the E4M3 grid, normal and
    # subnormal, and the 416/448 midpoint
    mids = [1.0625, 1.1875, -1.3125, 3 * 2.0 ** -10, 2.0 ** -10, -5 * 2.0 ** -10, 432.0, 2.25, -2.75, 0.15625]
    f8 = np.array([[448.0] + mids * 6 + [0.0, -0.0, 1.0]] * bs, np.float16)[:, None, :]
    k8 = f8.copy()
    q = np.ones((2, 1, d), np.float16)
    # INT4 K: the INT4 V rows as K (scale 1, zero point 5, half-integer ties)
    for vc, kk, vv in (("i8", k, v), ("i4", k, v4), ("i8a", k, v8), ("fp8", k8, f8), ("k4i4", v4, v4),
                       ("k4i8", v4, v)):
        case = SmallCase([kk, kk[:7]], [vv, vv[:7]], q, 1, 1, d, bs, vc, 4, None)
        case.store_all()
        assert_pool_equal(case.pool, case.opool)


def test_permutation_invariance_bitwise():
    announce("perm-invariance")
    rng = np.random.default_rng(9)
    ctx = [300, 45, 1000]
    hk = [rng.standard_normal((c, 2, 128)).astype(np.float16) for c in ctx]
    hv = [rng.standard_normal((c, 2, 128)).astype(np.float16) for c in ctx]
    q = rng.standard_normal((3, 2, 128)).astype(np.float16)
    outs = []
    for seed in (1, 2):
        n = sum((c + 15) // 16 for c in ctx) + 5
        case = SmallCase(hk, hv, q, 2, 2, 128, 16, "i8", n, np.random.default_rng(seed).permutation(n))
        case.store_all()
        outs.append(case.decode(128))
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))


def test_partition_size_invariance():
    announce("partition-invariance")
    case = normal_case([2000, 513, 1], 2, 2, 128, 32, "i4", seed=11)
    case.store_all()
    outs = [case.decode(p) for p in (32, 256, 512, 1024, 2048)]
    for o in outs[1:]:
        assert_close(o, outs[-1], "partition sizes")
    assert_close(outs[-1], case.reference(), "single partition")


def _store_chunk(pool, k, v, s, start, tables, slots):
    cu = torch.tensor([0, k.shape[0]], dtype=torch.int32, device="cuda")
    st = torch.tensor([start], dtype=torch.int32, device="cuda")
    pool.quantize_store(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), cu, st,
                        tables[s:s + 1], slots[s:s + 1], k.shape[0])


@pytest.mark.parametrize("vc", ["i8", "i4", "i8a", "fp8", "k4i4", "k4i8"])
def test_append_requantize_from_tail(vc):
    """One-token appends re-quantize the partial block from the exact rows in
    the tail slot; the result equals the oracle's quantization of the rows."""
    announce("append", vc)
    from paged_block_quantized_amd import KVPool
    rng = np.random.default_rng(21)
    bs, d, h = 16, 128, 2
    total = 40
    hk = rng.standard_normal((total, h, d)).astype(np.float16)
    hv = rng.standard_normal((total, h, d)).astype(np.float16)
    pool = make_pool(8, bs, h, d, vc, max_seqs=2, free_order=rng.permutation(8))
    model = A.BlockPoolModel(8, bs, 2, pool.free_list())
    opool = opool_for(8, h, bs, d, vc)
    pool.alloc(0, 3)
    model.alloc(0, 3)
    tables, _, slots = pool.batch_tables([0], 3)
    tables, slots = tables.cuda(), slots.cuda()
    _store_chunk(pool, hk[:3], hv[:3], 0, 0, tables, slots)
    for p in range(3, total):
        assert pool.append(0, 1) == model.append(0, 1) == []
        tables, _, slots = pool.batch_tables([0], 3)
        tables, slots = tables.cuda(), slots.cuda()
        _store_chunk(pool, hk[p:p + 1], hv[p:p + 1], 0, p, tables, slots)
        paged.store_range(opool, model.table(0)[0], hk, hv, 0, p + 1)
        if p % 7 == 0 or p == total - 1:
            torch.cuda.synchronize()
            assert_pool_equal(pool, opool)
    # tail slot holds the exact rows of the partial last block
    slot = pool.table(0)[2]
    n_tail = total % bs
    tk = pool.tail_k[slot].cpu().numpy()            # [H, bs, D]
    assert np.array_equal(tk[:, :n_tail].transpose(1, 0, 2).view(np.uint16),
                          hk[total - n_tail:].view(np.uint16))
    # append-built blocks equal a prefill of the same rows
    pre = opool_for(8, h, bs, d, vc)
    paged.store_range(pre, model.table(0)[0], hk, hv, 0, total)
    assert_pool_equal(pool, pre)


@pytest.mark.parametrize("vc", ["i8", "i4", "i8a", "fp8", "k4i4", "k4i8"])
def test_fork_copy_on_write(vc):
    """An unaligned shared prefix: fork copies the tail slot; each child's
    first append copies only the shared partial block; shared prefix blocks
    are unchanged; outputs equal the oracle's."""
    announce("fork-cow", vc)
    from paged_block_quantized_amd import KVPool
    rng = np.random.default_rng(31)
    bs, d, h = 32, 128, 2
    pre, n_children, extra = 72, 2, 50        # 72 = 2.25 blocks
    hp_k = rng.standard_normal((pre, h, d)).astype(np.float16)
    hp_v = rng.standard_normal((pre, h, d)).astype(np.float16)
    N = 16
    order = rng.permutation(N)
    pool = make_pool(N, bs, h, d, vc, max_seqs=4, free_order=order)
    model = A.BlockPoolModel(N, bs, 4, order)
    opool = opool_for(N, h, bs, d, vc)
    parent = 9
    pool.alloc(parent, pre)
    model.alloc(parent, pre)
    t, _, sl = pool.batch_tables([parent], 8)
    _store_chunk(pool, hp_k, hp_v, 0, 0, t.cuda(), sl.cuda())
    paged.store_range(opool, model.table(parent)[0], hp_k, hp_v, 0, pre)
    hist = {}
    for c in range(n_children):
        cp = pool.fork(parent, c)
        assert cp == model.fork(parent, c) == [(A.COPY_SLOT, 0, c + 1)]
        keep = pool.copy_blocks(cp)
        ck = rng.standard_normal((extra, h, d)).astype(np.float16)
        cv = rng.standard_normal((extra, h, d)).astype(np.float16)
        cp = pool.append(c, extra)
        assert cp == model.append(c, extra)
        if c == 0:
            assert len(cp) == 1 and cp[0][0] == A.COPY_BLOCK
        keep2 = pool.copy_blocks(cp)   # the oracle re-quantizes dst in full below
        t, _, sl = pool.batch_tables([c], 8)
        _store_chunk(pool, ck, cv, 0, pre, t.cuda(), sl.cuda())
        torch.cuda.synchronize()
        del keep, keep2
        hk, hv = np.concatenate([hp_k, ck]), np.concatenate([hp_v, cv])
        paged.store_range(opool, model.table(c)[0], hk, hv, pre, pre + extra)
        hist[c] = (hk, hv)
    assert_pool_equal(pool, opool)
    # decode the parent and both children together
    seqs = [parent] + list(range(n_children))
    tables, ctx_h, _ = pool.batch_tables(seqs, 8)
    q = rng.standard_normal((3, h, d)).astype(np.float16)
    qd = torch.from_numpy(q).cuda()
    out = torch.empty_like(qd)
    pool.decode(qd, out, tables.cuda(), ctx_h.cuda(), int(ctx_h.max()), 1 / np.sqrt(d), 64)
    ref = attention.paged_decode(opool, [model.table(s)[0] for s in seqs], ctx_h.numpy(), q, 1 / np.sqrt(d))
    assert_close(out.cpu().numpy(), ref, "fork")
    # the shared blocks were not modified by the children's stores
    shared = [b for b in model.table(parent)[0] if model.refcount[b] > 1]
    assert len(shared) == 2
    ref_parent = opool_for(N, h, bs, d, vc)
    paged.store_range(ref_parent, model.table(parent)[0], hp_k, hp_v, 0, pre)
    assert_pool_equal(pool, ref_parent, blocks=model.table(parent)[0])


GQA_SHAPES = [
    # (block_size, head_dim, v codec, query heads per KV head, KV heads)
    (32, 128, "i4", 8, 2),
    (16, 128, "i8", 4, 2),
    (32, 64, "i8", 16, 1),
    (16, 64, "i4", 2, 3),
    (32, 128, "i8", 32, 1),
    (16, 128, "i4", 7, 2),
    (32, 128, "fp8", 8, 2),
    (16, 64, "fp8", 4, 1),
    (32, 128, "i8a", 8, 2),
    (16, 128, "i8a", 7, 2),
    (32, 128, "k4i4", 8, 2),
    (16, 64, "k4i8", 4, 1),
    (16, 128, "k4i4", 7, 2),
    (32, 64, "k4i8", 16, 1),
]


@pytest.mark.parametrize("bs,d,vc,g,hkv", GQA_SHAPES)
def test_gqa_ragged(bs, d, vc, g, hkv):
    """Grouped-query heads (the MFMA path), ragged contexts, several
    partition sizes including ones that split inside a 32-token step."""
    announce("gqa", bs, d, vc, g, hkv)
    ctx = [1, 31, 32, 33, bs + 7, 300, 1027]
    case = normal_case(ctx, g * hkv, hkv, d, bs, vc, seed=7 * bs + d + g)
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    ref = case.reference()
    # 2048: one partition per sequence (the 2-wave single-pass launch)
    for part in (0, 32, 96, 256, 2048):
        assert_close(case.decode(part), ref, f"gqa bs{bs} d{d} {vc} g{g} part{part}")


def test_gqa_rejects_partition_not_multiple_of_32():
    announce("gqa-partition-check")
    from paged_block_quantized_amd import PBQError
    case = normal_case([40], 4, 2, 64, 16, "i8", seed=3)
    case.store_all()
    with pytest.raises(PBQError, match="multiple of 32"):
        case.decode(16)


APPEND_SHAPES = [(bs, d, vc, 1) for bs in (16, 32) for d in (64, 128)
                 for vc in ("i8", "i4", "i8a", "fp8", "k4i4", "k4i8")] + [
    (32, 128, "i4", 8), (16, 128, "i8", 4), (32, 128, "fp8", 8), (16, 64, "fp8", 4), (32, 128, "i8a", 8),
    (16, 128, "i8a", 2), (32, 128, "k4i4", 8), (16, 64, "k4i8", 4), (16, 128, "k4i4", 2)]


@pytest.mark.parametrize("bs,d,vc,g", APPEND_SHAPES)
def test_decode_append_equals_store_then_decode(bs, d, vc, g):
    """paged_attn_decode_append (the current token's store fused into the
    decode) leaves the pool bit-identical to kv_quantize_store followed by
    paged_attn_decode -- codes, scales, zero points and tail slots -- and both
    outputs agree with the oracle.  Context lengths put the new token at the
    start, the middle and the end of a block."""
    announce("decode-append", bs, d, vc, g)
    ctx = [1, 2, bs - 1, bs, bs + 1, 2 * bs, 3 * bs + 5, 700, 1100]
    # 2048 covers every context: one partition (the fused kernel)
    check_decode_append(bs, d, vc, g, ctx, (0, 32 if g > 1 else bs, 1024, 2048),
                        seed=1000 * bs + d + 7 * g + (vc == "i4"))


def check_decode_append(bs, d, vc, g, ctx, parts, seed, hkv=2, repeat=False):
    """Sequences of the given contexts, their last token stored two ways
    (kv_quantize_store then paged_attn_decode, and paged_attn_decode_append)
    for each partition size: the pools bit-identical to each other and to the
    oracle's, both outputs within tolerance of the oracle's.  repeat: the
    fused call runs twice on identical pools and must give identical bits."""
    hq = g * hkv
    S = len(ctx)
    rng = np.random.default_rng(seed)
    hk = [rng.standard_normal((c, hkv, d)).astype(np.float16) for c in ctx]
    hv = [rng.standard_normal((c, hkv, d)).astype(np.float16) for c in ctx]
    q = rng.standard_normal((S, hq, d)).astype(np.float16)
    n_blocks = sum((c + bs - 1) // bs for c in ctx) + 2
    order = rng.permutation(n_blocks)
    max_blocks = max((c + bs - 1) // bs for c in ctx)
    sm = 1.0 / np.sqrt(d)
    dev = torch.device("cuda")

    def build():
        pool = make_pool(n_blocks, bs, hkv, d, vc, max_seqs=S, free_order=order)
        for s, c in enumerate(ctx):
            pool.alloc(s, c - 1)
        tables, _, slots = pool.batch_tables(list(range(S)), max_blocks)
        lens = [c - 1 for c in ctx]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        k = torch.from_numpy(np.concatenate([h[:c - 1] for h, c in zip(hk, ctx)])).to(dev)
        v = torch.from_numpy(np.concatenate([h[:c - 1] for h, c in zip(hv, ctx)])).to(dev)
        pool.quantize_store(k, v, cu, torch.zeros(S, dtype=torch.int32, device=dev),
                            tables.to(dev), slots.to(dev), max(max(lens), 1))
        for s in range(S):
            assert pool.append(s, 1) == []
        tables, ctx_h, slots = pool.batch_tables(list(range(S)), max_blocks)
        assert list(ctx_h.numpy()) == ctx
        for s in range(S):
            assert pool.table(s)[0] == model.table(s)[0], f"seq {s} table"
        return pool, tables.to(dev), ctx_h.to(dev), slots.to(dev)

    k_new = torch.from_numpy(np.stack([h[c - 1] for h, c in zip(hk, ctx)])).to(dev)
    v_new = torch.from_numpy(np.stack([h[c - 1] for h, c in zip(hv, ctx)])).to(dev)
    qd = torch.from_numpy(q).to(dev)
    # the oracle: every row stored, tables from the allocator model
    model = A.BlockPoolModel(n_blocks, bs, S, order)
    opool = opool_for(n_blocks, hkv, bs, d, vc)
    for s, c in enumerate(ctx):          # the same call order as build()
        model.alloc(s, c - 1)
    for s, c in enumerate(ctx):
        model.append(s, 1)
        paged.store_range(opool, model.table(s)[0], hk[s], hv[s], 0, c)
    ref = attention.paged_decode(opool, [model.table(s)[0] for s in range(S)], ctx, q, sm)

    for part in parts:
        pa, ta, ca, sa = build()
        pa.quantize_store(k_new, v_new, torch.arange(S + 1, dtype=torch.int32, device=dev),
                          ca - 1, ta, sa, 1)
        out_a = torch.empty_like(qd)
        pa.decode(qd, out_a, ta, ca, max(ctx), sm, part)
        pb, tb, cb, sb = build()
        out_b = torch.empty_like(qd)
        pb.decode_append(k_new, v_new, sb, qd, out_b, tb, cb, max(ctx), sm, part)
        torch.cuda.synchronize()
        for name in ("k_codes", "v_codes", "k_scale", "v_scale", "tail_k", "tail_v") + zp_arrays(vc):
            x, y = pa.arrays[name].cpu().numpy(), pb.arrays[name].cpu().numpy()
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{name} differs (part {part})"
        g_k = pb.k_codes.cpu().numpy()
        bad = [(s, j, b) for s in range(S) for j, b in enumerate(model.table(s)[0])
               if not np.array_equal(g_k[b], opool.k_codes[b])]
        assert not bad, f"K codes differ at (seq, block, phys) {bad[:6]}"
        assert_pool_equal(pb, opool)
        assert_close(out_a.cpu().numpy(), ref, f"store+decode part {part}")
        assert_close(out_b.cpu().numpy(), ref, f"decode_append part {part}")
        if repeat:
            pc, tc, cc, sc = build()
            out_c = torch.empty_like(qd)
            pc.decode_append(k_new, v_new, sc, qd, out_c, tc, cc, max(ctx), sm, part)
            torch.cuda.synchronize()
            assert np.array_equal(out_c.cpu().numpy().view(np.uint16), out_b.cpu().numpy().view(np.uint16)), \
                f"decode_append not reproducible (part {part})"


# Single-pass grouped-query calls run in paired work groups: two sequences
# (ranked by context length, longest with shortest; beyond 256 sequences in
# the call's order) share four waves that split their steps end to end.
PAIR_CONTEXTS = {
    "one": [40],
    "stored_only": [1, 2],                 # both sequences: the stored step alone
    "second_stored_only": [700, 20],       # the short one: its stored step alone
    "ties": [50, 50, 7, 50, 7, 96],
    "odd": [33, 1, 64, 500, 31],
    "ranked_256": [int(x) for x in np.random.default_rng(17).integers(1, 200, 256)],
    "unranked_300": [int(x) for x in np.random.default_rng(18).integers(1, 90, 300)],
}


@pytest.mark.parametrize("name", list(PAIR_CONTEXTS))
@pytest.mark.parametrize("vc", ["i4", "fp8", "k4i4", "k4i8"])
def test_paired_groups(name, vc):
    """Paired grouped-query groups against the oracle, plain decode and fused
    store + decode, in one pass; the fused call is reproducible bit for bit.
    INT4 K (k4i4, k4i8) stages its 64-byte rows through LDS like byte K."""
    announce("paired", name, vc)
    ctx = PAIR_CONTEXTS[name]
    check_decode_append(32, 128, vc, 8, ctx, (2048,), seed=len(ctx) + 3 * sum(ctx) % 1000, repeat=True)
    case = normal_case(ctx, 8 * 2, 2, 128, 32, vc, seed=sum(ctx) % 997)
    case.store_all()
    ref = case.reference()
    out = case.decode(2048)
    assert_close(out, ref, f"paired plain decode {name} {vc}")
    assert np.array_equal(case.decode(2048).view(np.uint16), out.view(np.uint16)), "plain decode not reproducible"


SHARED_SHAPES = [
    # (block_size, head_dim, v codec, query heads per KV head, KV heads, sequences, partition)
    (16, 64, "i8", 1, 2, 5, 64),
    (16, 128, "i4", 1, 2, 20, 128),
    (32, 64, "i4", 1, 3, 5, 64),
    (32, 128, "i8", 1, 2, 5, 128),
    (32, 128, "i4", 8, 2, 5, 64),
    (16, 64, "i8", 4, 1, 5, 96),
    (32, 128, "fp8", 8, 2, 5, 64),
    (16, 128, "fp8", 1, 2, 5, 128),
    (32, 64, "i8a", 1, 2, 5, 64),
    (32, 128, "k4i4", 8, 2, 5, 64),
    (16, 64, "k4i8", 1, 2, 5, 64),
]


@pytest.mark.parametrize("bs,d,vc,g,hkv,S,part", SHARED_SHAPES)
def test_shared_prefix_decode(bs, d, vc, g, hkv, S, part):
    """Sequences forked from one prefix of two partitions, then ragged
    continuations.  paged_attn_decode_shared_prefix (prefix tiles read once,
    on matrix cores, for all sequences' queries) with the current token's
    store: every sequence's blocks bit-exact and outputs within tolerance of
    the oracle; the per-sequence path leaves the same pool bit for bit; the
    plain (no store) form gives the oracle's outputs too.  Two 16-query tiles
    when sequences x group exceed 16."""
    import dataclasses
    from paged_block_quantized_amd import runner, workloads as W
    from gpu_util import check_sequence
    announce("shared-prefix", bs, d, vc, g, hkv, S, part)
    prefix = 2 * part
    ctx = tuple(prefix + x for x in [1, bs, bs + 1, 3 * bs + 5, 300, 2, 5 * bs, 77, 1, 33,
                                     bs - 1, 64, 129, 9, 40, 500, 3, 17, 250, 6][:S])
    w = dataclasses.replace(W.WORKLOADS["shared_prefix"], name="shared_small", num_seqs=S,
                            num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, block_size=bs,
                            v_codec=codecs(vc)[1], k_codec=codecs(vc)[0], ctx_kind="list", ctx=ctx,
                            prefix=prefix, partition=part,
                            seed=11 * bs + d + g + S)
    setup = runner.setup_decode(w)
    assert setup.shared == prefix
    setup.step()
    torch.cuda.synchronize()
    out_shared = setup.out.cpu().numpy()
    for s in range(S):
        check_sequence(setup, s, out_shared, "shared-prefix step")
    snap = {n: t.clone() for n, t in setup.pool.arrays.items()}
    setup.step_unshared()
    torch.cuda.synchronize()
    for n, t in snap.items():
        assert torch.equal(t, setup.pool.arrays[n]), f"{n} differs between the two step paths"
    for s in range(S):
        check_sequence(setup, s, setup.out.cpu().numpy(), "per-sequence step")
    # plain decode over the same (now stored) contexts
    out = torch.empty_like(setup.q)
    setup.pool.decode_shared_prefix(setup.q, out, setup.tables, setup.ctx_dev, setup.max_ctx,
                                    setup.sm_scale, part, prefix)
    torch.cuda.synchronize()
    for s in range(S):
        check_sequence(setup, s, out.cpu().numpy(), "shared-prefix decode")


P9_SHAPES = [
    # (block_size, head_dim, v codec, query heads per KV head, KV heads)
    (32, 128, "i4", 1, 2),
    (16, 64, "i8", 4, 1),
    (32, 128, "fp8", 8, 2),
    (16, 128, "i8a", 1, 2),
    (32, 128, "k4i4", 8, 2),
    (16, 64, "k4i8", 1, 2),
]


@pytest.mark.parametrize("bs,d,vc,g,hkv", P9_SHAPES)
def test_shared_prefix_equals_private_copies_bitwise(bs, d, vc, g, hkv):
    """Sequences forked from one prefix (yunthe.com "PagedAttention
    mechanism": prefix sharing maps every sequence's prefix to the same
    physical blocks) decode bitwise as they do when each holds a private
    copy of the prefix blocks (kv_copy_blocks into fresh blocks, tables
    rewritten), at several partition sizes; the shared blocks are the
    oracle's quantization of the prefix rows after every sequence's
    divergent tokens are stored."""
    import dataclasses
    from oracle import allocator as A
    from paged_block_quantized_amd import runner, workloads as W
    from gpu_util import check_sequence
    announce("P9 shared vs private prefix", bs, d, vc, g, hkv)
    S, part = 5, 64
    prefix = 2 * part
    ctx = tuple(prefix + x for x in [1, bs + 1, 3 * bs + 5, 300, 77])
    w = dataclasses.replace(W.WORKLOADS["shared_prefix"], name="p9_small", num_seqs=S,
                            num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, block_size=bs,
                            v_codec=codecs(vc)[1], k_codec=codecs(vc)[0], ctx_kind="list", ctx=ctx,
                            prefix=prefix, partition=part,
                            seed=3 * bs + d + g)
    P = prefix // bs
    n_blocks = runner.blocks_needed(w, W.context_lengths(w)) + S * P
    w = dataclasses.replace(w, pool_blocks=n_blocks)
    setup = runner.setup_decode(w)
    setup.step_unshared()          # the current tokens stored, decoded per sequence
    torch.cuda.synchronize()
    pool = setup.pool
    shared_ids = setup.tables[:, :P].cpu().numpy()
    assert (shared_ids == shared_ids[0]).all(), "every sequence maps the prefix to the same blocks"
    for s in range(S):
        check_sequence(setup, s, setup.out.cpu().numpy(), "P9 shared step")
    # private copies of the prefix blocks, one set per sequence
    dummy = S + 7
    pool.alloc(dummy, S * prefix)
    dtab = pool.table(dummy)[0]
    private = setup.tables.clone()
    copies = []
    for s in range(S):
        for j in range(P):
            copies.append((A.COPY_BLOCK, int(shared_ids[s, j]), int(dtab[s * P + j])))
            private[s, j] = int(dtab[s * P + j])
    keep = pool.copy_blocks(copies)
    torch.cuda.synchronize()
    del keep
    for p in (0, bs if g == 1 else 32, part, 4096):
        outs = []
        for tables in (setup.tables, private):
            out = torch.empty_like(setup.q)
            pool.decode(setup.q, out, tables, setup.ctx_dev, setup.max_ctx, setup.sm_scale, p)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16)), f"partition {p}"


@pytest.mark.parametrize("bs,vc", [(16, "i8"), (32, "i4"), (32, "k4i4")])
def test_prefix_cache_end_to_end(bs, vc):
    """kv_seq_alloc_prefix: requests whose token ids share prefixes map the
    cached blocks and store only their uncached positions; the pool equals
    the oracle's (model allocator + store of the same ranges) bit for bit,
    shared blocks are not rewritten, and decode over the full contexts
    matches the oracle.  K/V rows are a seeded function of (token id,
    position), as a model's would be, so equal prefixes have equal rows."""
    announce("prefix-cache", bs, vc)
    from paged_block_quantized_amd import KVPool
    h, d, hq = 2, 64, 4
    rng = np.random.default_rng(77 + bs)
    vocab = 5
    table_k = rng.standard_normal((vocab, 4096, h, d)).astype(np.float16)
    table_v = rng.standard_normal((vocab, 4096, h, d)).astype(np.float16)
    base = [int(t) for t in rng.integers(0, vocab, 8 * bs)]
    reqs = [base[:5 * bs + 3], base[:3 * bs] + [0] * (bs + 1), base[:5 * bs + 3],
            base[:2 * bs], [1] * (2 * bs + 7), base[:4 * bs] + [2] * (2 * bs)]
    N = 64
    order = rng.permutation(N)
    pool = make_pool(N, bs, h, d, vc, max_seqs=len(reqs), free_order=order)
    model = A.BlockPoolModel(N, bs, len(reqs), order)
    opool = opool_for(N, h, bs, d, vc)
    shared_before = {}
    for s, ids in enumerate(reqs):
        tab, cached = pool.alloc_prefix(s, ids)
        assert (tab, cached) == model.alloc_prefix(s, ids)
        assert cached % bs == 0 and cached <= len(ids)
        hk = np.stack([table_k[t, p] for p, t in enumerate(ids)])
        hv = np.stack([table_v[t, p] for p, t in enumerate(ids)])
        n = len(ids)
        if cached:
            assert np.array_equal(pool.k_codes[tab[0]].cpu().numpy(), opool.k_codes[tab[0]])
            shared_before[s] = pool.k_codes[torch.tensor(tab[:cached // bs])].clone()
        if n > cached:
            t, _, sl = pool.batch_tables([s], max(1, len(tab)))
            k = torch.from_numpy(hk[cached:]).cuda()
            v = torch.from_numpy(hv[cached:]).cuda()
            cu = torch.tensor([0, n - cached], dtype=torch.int32, device="cuda")
            st = torch.tensor([cached], dtype=torch.int32, device="cuda")
            pool.quantize_store(k, v, cu, st, t.cuda(), sl.cuda(), n - cached)
            paged.store_range(opool, tab, hk, hv, cached, n)
        torch.cuda.synchronize()
    assert_pool_equal(pool, opool)
    for s, codes in shared_before.items():   # shared blocks were not rewritten
        tab = model.table(s)[0]
        assert torch.equal(pool.k_codes[torch.tensor(tab[:codes.shape[0]])], codes)
    assert model.stats() == pool.stats()
    S = len(reqs)
    tables, ctx_h, _ = pool.batch_tables(list(range(S)), 8)
    q = rng.standard_normal((S, hq, d)).astype(np.float16)
    qd = torch.from_numpy(q).cuda()
    out = torch.empty_like(qd)
    pool.decode(qd, out, tables.cuda(), ctx_h.cuda(), int(ctx_h.max()), 1 / np.sqrt(d), 0)
    torch.cuda.synchronize()
    ref = attention.paged_decode(opool, [model.table(s)[0] for s in range(S)], ctx_h.numpy(), q,
                                 1 / np.sqrt(d))
    assert_close(out.cpu().numpy(), ref, "prefix-cache decode")


# ---- swap to host memory (deepinsea "Swap") --------------------------------

_POOL_ARRAYS = ("k_codes", "v_codes", "k_scale", "v_scale", "v_zp", "tail_k", "tail_v", "k_zp")


def _fill_random(rng, arrays, used):
    """Seeded random bytes in every array the codecs use (device or pinned
    host tensors); returns numpy uint8 copies shaped [rows, bytes per row]."""
    exp = {}
    for n in _POOL_ARRAYS:
        if n.endswith("_zp") and n not in used:
            continue
        t = arrays[n]
        b = rng.integers(0, 256, t.numel() * t.element_size(), dtype=np.uint8)
        t.view(torch.uint8).reshape(-1).copy_(torch.from_numpy(b))
        exp[n] = b.reshape(t.shape[0], -1)
    return exp


def _apply_plan(plan, dev, host, h, bs):
    """The plan's definition on numpy byte arrays: whole rows of the block
    arrays; the first `rows` token rows of each head of a tail slot."""
    block = ("k_codes", "v_codes", "k_scale", "v_scale", "v_zp", "k_zp")
    for kind, src, dst, rows in plan:
        out = kind in (A.SWAP_BLOCK_OUT, A.SWAP_SLOT_OUT)
        a, b = (dev, host) if out else (host, dev)
        if kind in (A.SWAP_BLOCK_OUT, A.SWAP_BLOCK_IN):
            for n in block:
                if n in a:
                    b[n][dst] = a[n][src]
        else:
            for n in ("tail_k", "tail_v"):
                b[n][dst].reshape(h, bs, -1)[:, :rows] = a[n][src].reshape(h, bs, -1)[:, :rows]


SWAP_SHAPES = [(16, 2, 64, "i8"), (32, 3, 128, "i4"), (16, 32, 128, "i8"), (32, 8, 64, "i4"),
               (16, 4, 128, "fp8"), (32, 2, 64, "i8a"), (32, 3, 128, "k4i4"), (16, 2, 64, "k4i8")]


@pytest.mark.parametrize("bs,h,d,vc", SWAP_SHAPES)
def test_swap_moves_bytes_exactly(bs, h, d, vc):
    """kv_seq_swap_out / kv_seq_swap_in plans equal the oracle model's, and
    kv_swap_blocks moves exactly the bytes they name: every device and host
    array equals seeded random contents with the plans applied by numpy,
    bit for bit, through forks, reuse of freed blocks, and partial groups."""
    announce("swap-bytes", bs, h, d, vc)
    from paged_block_quantized_amd import KVPool
    rng = np.random.default_rng(1000 + bs + h + d)
    N, S = 40, 8
    order = rng.permutation(N)
    pool = make_pool(N, bs, h, d, vc, max_seqs=S, free_order=order)
    model = A.BlockPoolModel(N, bs, S, order)
    pool.set_swap_space(24, 4)
    model.set_swap_space(24, 4)
    dev = _fill_random(rng, pool.arrays, zp_arrays(vc))
    host = _fill_random(rng, pool.host_arrays, zp_arrays(vc))
    for s, n in {0: 3 * bs + 5, 1: 2 * bs, 2: 1, 3: 4 * bs - 1, 4: bs + 2}.items():
        assert pool.alloc(s, n) == model.alloc(s, n)
    copies = model.fork(0, 5)
    assert pool.fork(0, 5) == copies
    pool.copy_blocks(copies)
    for _, src, dst in copies:                       # a slot copy: whole slot
        for n in ("tail_k", "tail_v"):
            dev[n][dst] = dev[n][src]

    def swap(direction, group):
        plan = getattr(pool, direction)(group)
        assert plan == getattr(model, direction)(group)
        _apply_plan(plan, dev, host, h, bs)
        return plan

    plan = swap("swap_out", [0, 5])                  # a fork pair: shared blocks once
    assert sum(1 for e in plan if e[0] == A.SWAP_SLOT_OUT) == 2
    # a new sequence takes freed blocks and a freed slot and writes them
    tab = pool.alloc(6, 3 * bs)
    assert tab == model.alloc(6, 3 * bs)
    slot6 = pool.table(6)[2]
    for n in ("k_codes", "v_codes", "k_scale", "v_scale"):
        fresh = rng.integers(0, 256, dev[n][tab].shape, dtype=np.uint8)
        dev[n][tab] = fresh
        pool.arrays[n].view(torch.uint8).reshape(N, -1)[torch.tensor(tab)] = \
            torch.from_numpy(fresh).cuda()
    fresh = rng.integers(0, 256, dev["tail_k"][slot6].shape, dtype=np.uint8)
    dev["tail_k"][slot6] = fresh
    pool.arrays["tail_k"].view(torch.uint8).reshape(S, -1)[slot6] = torch.from_numpy(fresh).cuda()
    swap("swap_out", [2])                            # one token: one block, one row
    swap("swap_in", [0, 5])
    pool.release(6)
    model.release(6)
    swap("swap_in", [2])
    swap("swap_out", [3, 1])
    swap("swap_in", [1])                             # 3 stays out
    torch.cuda.synchronize()
    for n in dev:
        got = pool.arrays[n].view(torch.uint8).reshape(dev[n].shape).cpu().numpy()
        assert np.array_equal(got, dev[n]), f"device {n}"
    for n in host:
        got = pool.host_arrays[n].view(torch.uint8).reshape(host[n].shape).numpy()
        assert np.array_equal(got, host[n]), f"host {n}"
    for s in model.seqs:
        assert pool.table(s) == model.table(s)
    assert pool.stats() == model.stats()


@pytest.mark.parametrize("bs,vc", [(16, "i8"), (32, "i4"), (16, "k4i4")])
def test_swap_then_decode_append_end_to_end(bs, vc):
    """Sequences swapped out (their freed blocks overwritten by another
    owner) and back in decode as before, bit for bit; their next token's
    fused store re-quantizes the partial block from the tail rows that came
    back, so the pool equals the oracle's quantization of each full history
    through the final tables, and the decode matches the oracle."""
    announce("swap-e2e", bs, vc)
    h, d, hq = 2, 64, 4
    ctx = [2 * bs + 3, 1, 5 * bs, 3 * bs + bs - 1, bs]
    case = normal_case(ctx, hq, h, d, bs, vc, seed=31 + bs, extra_blocks=12)
    case.store_all()
    out0 = case.decode()
    assert_close(out0, case.reference(), "swap-e2e before")
    pool, model = case.pool, case.model
    pool.set_swap_space(16, 3)
    model.set_swap_space(16, 3)
    rng = np.random.default_rng(5)
    assert pool.swap_out([1, 3]) == model.swap_out([1, 3])
    tab = pool.alloc(9, 4 * bs)
    assert tab == model.alloc(9, 4 * bs)
    idx = torch.tensor(tab)
    pool.k_codes.view(torch.uint8)[idx] = torch.randint(0, 256, pool.k_codes[idx].shape,
                                                       dtype=torch.uint8).cuda()
    pool.v_codes.view(torch.uint8)[idx] = torch.randint(0, 256, pool.v_codes[idx].shape,
                                                       dtype=torch.uint8).cuda()
    pool.tail_k[pool.table(9)[2]] = torch.randn(pool.tail_k.shape[1:]).half().cuda()
    pool.release(9)
    model.release(9)
    assert pool.swap_in([3, 1]) == model.swap_in([3, 1])
    S = len(ctx)
    tables, ctx_h, slots = pool.batch_tables(list(range(S)), case.max_blocks + 1)
    case.tables, case.slots = tables.cuda(), slots.cuda()
    out1 = case.decode()
    assert np.array_equal(out1.view(np.uint16), out0.view(np.uint16))
    # the next token of every sequence, stored by the fused decode
    for s in range(S):
        assert pool.append(s, 1) == model.append(s, 1)
    new_k = rng.standard_normal((S, h, d)).astype(np.float16)
    new_v = rng.standard_normal((S, h, d)).astype(np.float16)
    q = rng.standard_normal((S, hq, d)).astype(np.float16)
    tables, ctx_h, slots = pool.batch_tables(list(range(S)), case.max_blocks + 1)
    qd = torch.from_numpy(q).cuda()
    out = torch.empty_like(qd)
    pool.decode_append(torch.from_numpy(new_k).cuda(), torch.from_numpy(new_v).cuda(), slots.cuda(),
                       qd, out, tables.cuda(), ctx_h.cuda(), int(ctx_h.max()), 1 / np.sqrt(d))
    torch.cuda.synchronize()
    ref_pool = opool_for(pool.num_blocks, h, bs, d, vc)
    tabs = []
    for s in range(S):
        hk = np.concatenate([case.hist_k[s], new_k[s:s + 1]])
        hv = np.concatenate([case.hist_v[s], new_v[s:s + 1]])
        t = model.table(s)[0]
        paged.store_range(ref_pool, t, hk, hv, 0, ctx[s] + 1)
        tabs.append(t)
    used = sorted(b for t in tabs for b in t)
    assert_pool_equal(pool, ref_pool, used)
    ref = attention.paged_decode(ref_pool, tabs, [c + 1 for c in ctx], q, 1 / np.sqrt(d))
    assert_close(out.cpu().numpy(), ref, "swap-e2e after")


# ---- several query tokens per sequence (chunked prefill, candidates) --------

MULTI_SHAPES = [
    # (block_size, head_dim, v codec, query heads per KV head, KV heads)
    (16, 128, "i8", 1, 2),
    (32, 64, "i4", 1, 3),
    (32, 128, "i4", 8, 2),
    (16, 64, "i8", 4, 1),
    (16, 128, "fp8", 2, 2),
    (32, 128, "i8a", 8, 1),
    (32, 64, "i8", 16, 1),
    (16, 128, "i4", 7, 2),
    (32, 128, "k4i4", 8, 2),
    (16, 64, "k4i8", 1, 2),
    (16, 128, "k4i4", 4, 1),
]


@pytest.mark.parametrize("bs,d,vc,g,hkv", MULTI_SHAPES)
def test_multi_query_ragged(bs, d, vc, g, hkv):
    """paged_attn_multi_query: each sequence's last n stored tokens attend
    causally (full prefills, chunks after a prefix, single tokens, chunks
    across partitions and blocks), every partition size and a single pass,
    against the oracle;
    a one-token query equals the decode's output within tolerance."""
    announce("multi", bs, d, vc, g, hkv)
    seqs = [(1, 1), (17, 5), (100, 100), (700, 64), (33, 32), (2100, 17), (300, 1), (64, 40)]
    ctx = [c for c, _ in seqs]
    ns = [n for _, n in seqs]
    hq = g * hkv
    case = normal_case(ctx, hq, hkv, d, bs, vc, seed=11 * bs + d + g + hkv)
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    rng = np.random.default_rng(bs + d + g)
    T = sum(ns)
    q_rows = rng.standard_normal((T, hq, d)).astype(np.float16)
    # the last query of each sequence is the decode query
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    for s in range(len(seqs)):
        q_rows[cu[s + 1] - 1] = case.q[s]
    sm = 1 / np.sqrt(d)
    ref = attention.paged_multi_query(case.opool, [case.model.table(s)[0] for s in range(len(seqs))], ctx,
                                      q_rows, cu, sm)
    qd = torch.from_numpy(q_rows).cuda()
    cud = torch.from_numpy(cu).cuda()
    dec = case.decode()
    # 4096: one pass over every context (two-wave groups: the one-slot merge,
    # or with INT4 V the shared staging)
    for part in (0, 32, 96, 256, 2048, 4096):
        out = torch.full_like(qd, float("nan"))
        case.pool.multi_query(qd, out, cud, max(ns), case.tables, case.ctx_dev, max(ctx), sm, part)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert_close(got, ref, f"multi bs{bs} d{d} {vc} g{g} part{part}")
        assert_close(got[cu[1:] - 1], dec.astype(np.float64), f"multi vs decode part{part}")


@pytest.mark.parametrize("bs,d,vc,g,hkv,ns", [
    (16, 128, "i8", 1, 2, [1, 16, 9, 3]),
    (32, 128, "i4", 8, 2, [2, 1, 2]),
    (32, 64, "i8", 16, 1, [1, 1]),
    (16, 64, "fp8", 4, 2, [4, 3, 1, 4]),
    (32, 128, "k4i4", 8, 2, [2, 1, 2]),
])
def test_multi_query_single_tile(bs, d, vc, g, hkv, ns):
    """Calls whose queries of one (sequence, KV head) fit one 16-query tile
    (n G <= 16) take the one-tile work groups; against the oracle at every
    partition size."""
    announce("multi-one-tile", bs, d, vc, g, hkv, ns)
    ctx = [50, 700, 33, 2100][:len(ns)]
    hq = g * hkv
    case = normal_case(ctx, hq, hkv, d, bs, vc, seed=7 * bs + d + g)
    case.store_all()
    rng = np.random.default_rng(bs + d + g + 1)
    q_rows = rng.standard_normal((sum(ns), hq, d)).astype(np.float16)
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    sm = 1 / np.sqrt(d)
    ref = attention.paged_multi_query(case.opool, [case.model.table(s)[0] for s in range(len(ns))], ctx,
                                      q_rows, cu, sm)
    qd = torch.from_numpy(q_rows).cuda()
    cud = torch.from_numpy(cu).cuda()
    # 4096: a single pass (two-wave groups merging through one wave's slot)
    for part in (0, 32, 256, 4096):
        out = torch.full_like(qd, float("nan"))
        case.pool.multi_query(qd, out, cud, max(ns), case.tables, case.ctx_dev, max(ctx), sm, part)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, f"multi one tile bs{bs} d{d} {vc} g{g} part{part}")


@pytest.mark.parametrize("vc,vmul", [("i8", 12000.0), ("i4", 1000.0), ("fp8", 200.0), ("i8a", 12000.0)])
def test_multi_query_large_v_scales(vc, vmul):
    """V blocks whose scales are 2^8 or more, with scores that jump by just
    under 8 (base 2) after the first 32 tokens: the multi-query softmax,
    which rescales only when its maximum grows by more than 8, would weight
    those tokens by about 2^8 times their V scale, past the fp16 range.
    Outputs stay finite and match the oracle (compared relative to the V
    magnitude: attention is linear in V)."""
    announce("multi-large-v", vc, vmul)
    bs, d, hkv, g = 16, 128, 2, 1
    ctx = [700, 333, 64]
    ns = [64, 40, 17]
    rng = np.random.default_rng(23)
    hk, hv = [], []
    for c in ctx:
        k = rng.standard_normal((c, hkv, d)) * 0.1
        # score 0 for the first 32 tokens, then 7.95 (base 2) for the rest
        k[:, :, 0] = np.where(np.arange(c) >= 32, 7.95 / np.log2(np.e) * np.sqrt(d), 0.0)[:, None]
        v = np.clip(rng.standard_normal((c, hkv, d)) * vmul, -65000, 65000)
        hk.append(k.astype(np.float16))
        hv.append(v.astype(np.float16))
    q_dec = np.zeros((len(ctx), hkv * g, d), np.float16)
    q_dec[:, :, 0] = 1
    n_blocks = sum((c + bs - 1) // bs for c in ctx) + 2
    case = SmallCase(hk, hv, q_dec, hkv * g, hkv, d, bs, vc, n_blocks, rng.permutation(n_blocks))
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    assert float(np.max(case.opool.v_scale.astype(np.float64))) * (256 if vc == "fp8" else 1) >= 255
    q_rows = np.zeros((sum(ns), hkv * g, d), np.float16)
    q_rows[:, :, 0] = 1
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    sm = 1 / np.sqrt(d)
    ref = attention.paged_multi_query(case.opool, [case.model.table(s)[0] for s in range(len(ctx))], ctx,
                                      q_rows, cu, sm)
    qd = torch.from_numpy(q_rows).cuda()
    cud = torch.from_numpy(cu).cuda()
    for part in (0, 256, 4096):
        out = torch.full_like(qd, float("nan"))
        case.pool.multi_query(qd, out, cud, max(ns), case.tables, case.ctx_dev, max(ctx), sm, part)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got)), f"non-finite outputs, {vc} part{part}"
        assert_close(got / vmul, ref / vmul, f"multi large V {vc} part{part}")
    dec = case.decode()
    assert np.all(np.isfinite(dec))
    assert_close(dec / vmul, case.reference() / vmul, f"decode large V {vc}")


def test_multi_query_validates():
    from paged_block_quantized_amd import _lib as L
    from paged_block_quantized_amd import KVPool
    pool = KVPool(8, 16, 2, 64, "i8", max_seqs=1)
    q = torch.zeros((4, 2, 64), dtype=torch.float16, device="cuda")
    t = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    c = torch.tensor([40], dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    with pytest.raises(L.PBQError, match="max_q_len"):
        L.paged_attn_multi_query(pool.desc, pool.mem, q, q, 1, 2, cu, 4, 0, t, 4, c, 40, 0.1)
    with pytest.raises(L.PBQError, match="multiple of 32"):
        L.paged_attn_multi_query(pool.desc, pool.mem, q, q, 1, 2, cu, 4, 4, t, 4, c, 40, 0.1, 16)
    with pytest.raises(L.PBQError, match="workspace"):
        L.paged_attn_multi_query(pool.desc, pool.mem, q, q, 1, 2, cu, 4, 4, t, 4, c, 40, 0.1, 32)


# ---- V magnitudes far from 1: the fp16 weights of the matrix-core path ------

def _scaled_v_case(bs, d, vc, g, hkv, kind, seed):
    """Histories whose V values are tiny (kind "small3": N(0, 1e-3),
    "small4": N(0, 1e-4): fp16 V scales near or below fp16's normal range)
    or alternate by 32-token step between N(0, 1e-3) and N(0, 10) with K
    set so that the tiny-V tokens dominate the softmax ("mixed").  Returns
    (hk, hv, q, sigma), sigma the magnitude of the V values that dominate
    the output."""
    rng = np.random.default_rng(seed)
    ctx = [1, 40, 333, 700, 1100, 2047]
    hq = g * hkv
    hk, hv = [], []
    for c in ctx:
        k = rng.standard_normal((c, hkv, d))
        v = rng.standard_normal((c, hkv, d))
        if kind == "mixed":
            small = (np.arange(c) // 32) % 2 == 0
            v *= np.where(small, 1e-3, 10.0)[:, None, None]
            k *= 0.05
            k[:, :, 0] = np.where(small, 20.0 * np.sqrt(d), 0.0)[:, None]
        else:
            v *= 1e-3 if kind == "small3" else 1e-4
        hk.append(k.astype(np.float16))
        hv.append(v.astype(np.float16))
    if kind == "mixed":
        q = (rng.standard_normal((len(ctx), hq, d)) * 0.01).astype(np.float16)
        q[:, :, 0] = 1.0
    else:
        q = rng.standard_normal((len(ctx), hq, d)).astype(np.float16)
    sigma = 1e-4 if kind == "small4" else 1e-3
    return ctx, hk, hv, q, sigma


SCALED_V = [(bs, g, vc, kind) for bs, g in ((32, 8), (16, 4), (32, 1), (16, 1))
            for vc in ("i8", "i4", "i8a", "fp8") for kind in ("small3", "small4", "mixed")]


@pytest.mark.parametrize("bs,g,vc,kind", SCALED_V)
def test_decode_scaled_v(bs, g, vc, kind):
    """Decode with V far from unit magnitude, grouped-query (g > 1) and MHA
    (g = 1): outputs within tolerance relative to the V magnitude (attention
    is linear in V), for the plain decode at several partition sizes and for
    the fused store + decode (single pass).  Both kernels weight V with fp16
    values: the matrix cores take p * sv normalised by a power of two that
    follows the V scales, the MHA kernel takes p alone and applies the V
    scale per block in fp32, so tiny scales keep full fp16 precision."""
    announce("scaled-v", bs, g, vc, kind)
    from paged_block_quantized_amd import KVPool
    d, hkv = 128, 2
    ctx, hk, hv, q, sigma = _scaled_v_case(bs, d, vc, g, hkv, kind, seed=bs + g + len(kind))
    n_blocks = sum((c + bs - 1) // bs for c in ctx) + 2
    order = np.random.default_rng(5).permutation(n_blocks)
    case = SmallCase(hk, hv, q, g * hkv, hkv, d, bs, vc, n_blocks, order)
    case.store_all()
    assert_pool_equal(case.pool, case.opool)
    ref = case.reference()
    for part in (0, 32, 4096):
        got = case.decode(part)
        assert_close(got / sigma, ref / sigma, f"scaled V g{g} {kind} {vc} bs{bs} part{part}")
    # the fused store + decode: every token but the last stored first
    dev = "cuda"
    S = len(ctx)
    pool = make_pool(n_blocks, bs, hkv, d, vc, max_seqs=S, free_order=order)
    for s, c in enumerate(ctx):
        pool.alloc(s, c - 1)
    mb = max((c + bs - 1) // bs for c in ctx)
    tables, _, slots = pool.batch_tables(list(range(S)), mb)
    lens = [c - 1 for c in ctx]
    kk = torch.from_numpy(np.concatenate([h[:c - 1] for h, c in zip(hk, ctx)])).to(dev)
    vv = torch.from_numpy(np.concatenate([h[:c - 1] for h, c in zip(hv, ctx)])).to(dev)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    pool.quantize_store(kk, vv, cu, torch.zeros(S, dtype=torch.int32, device=dev), tables.to(dev),
                        slots.to(dev), max(max(lens), 1))
    for s in range(S):
        assert pool.append(s, 1) == []
    tables, ctx_h, slots = pool.batch_tables(list(range(S)), mb)
    k_new = torch.from_numpy(np.stack([h[c - 1] for h, c in zip(hk, ctx)])).to(dev)
    v_new = torch.from_numpy(np.stack([h[c - 1] for h, c in zip(hv, ctx)])).to(dev)
    qd = torch.from_numpy(q).to(dev)
    out = torch.empty_like(qd)
    pool.decode_append(k_new, v_new, slots.to(dev), qd, out, tables.to(dev), ctx_h.to(dev), max(ctx),
                       1 / np.sqrt(d), 4096)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy() / sigma, ref / sigma, f"fused scaled V g{g} {kind} {vc} bs{bs}")


@pytest.mark.parametrize("bs,g,vc,kind", [(32, 8, vc, k) for vc in ("i8", "i4", "i8a", "fp8")
                                          for k in ("small3", "small4", "mixed")] +
                         [(16, 1, vc, k) for vc in ("i8", "i4") for k in ("small4", "mixed")])
def test_multi_query_scaled_v(bs, g, vc, kind):
    """Multi-query attention with V far from unit magnitude, within
    tolerance relative to the V magnitude, one pass and split partitions."""
    announce("multi-scaled-v", bs, g, vc, kind)
    d, hkv = 128, 2
    ctx, hk, hv, q_dec, sigma = _scaled_v_case(bs, d, vc, g, hkv, kind, seed=3 * bs + g + len(kind))
    n_blocks = sum((c + bs - 1) // bs for c in ctx) + 2
    case = SmallCase(hk, hv, q_dec, g * hkv, hkv, d, bs, vc, n_blocks,
                     np.random.default_rng(6).permutation(n_blocks))
    case.store_all()
    ns = [1, 17, 64, 40, 100, 33]
    rng = np.random.default_rng(bs + g)
    T = sum(ns)
    if kind == "mixed":
        q_rows = (rng.standard_normal((T, g * hkv, d)) * 0.01).astype(np.float16)
        q_rows[:, :, 0] = 1.0
    else:
        q_rows = rng.standard_normal((T, g * hkv, d)).astype(np.float16)
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    sm = 1 / np.sqrt(d)
    ref = attention.paged_multi_query(case.opool, [case.model.table(s)[0] for s in range(len(ctx))],
                                      case.ctx, q_rows, cu, sm)
    qd = torch.from_numpy(q_rows).cuda()
    cud = torch.from_numpy(cu).cuda()
    for part in (0, 256, 4096):
        out = torch.full_like(qd, float("nan"))
        case.pool.multi_query(qd, out, cud, max(ns), case.tables, case.ctx_dev, max(case.ctx), sm, part)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy() / sigma, ref / sigma, f"multi scaled V {kind} {vc} part{part}")


# ---- the plain-read ceiling kernel -------------------------------------------

@pytest.mark.parametrize("tile_bytes,n_src,n,ordered", [(2048, 3000, 3000, True), (4096, 700, 313, True),
                                                      (1024, 5000, 4999, False), (2048, 64, 1, True)])
def test_stream_read_reads_every_listed_tile(tile_bytes, n_src, n, ordered):
    """kv_stream_read_tiles reads exactly the listed tiles: the xor of its
    sink words equals the xor of every 32-bit word of those tiles."""
    announce("stream-read", tile_bytes, n_src, n, ordered)
    from paged_block_quantized_amd import _lib as L
    rng = np.random.default_rng(tile_bytes + n)
    src = rng.integers(0, 2 ** 32, n_src * tile_bytes // 4, dtype=np.uint32)
    ids = rng.permutation(n_src)[:n].astype(np.int32) if ordered else np.arange(n, dtype=np.int32)
    expect = np.bitwise_xor.reduce(src.reshape(n_src, -1)[ids].ravel())
    src_d = torch.from_numpy(src.view(np.int32)).cuda()
    order_d = torch.from_numpy(ids).cuda() if ordered else None
    sink = torch.full((L.kv_stream_read_sink_words(n),), 0x55, dtype=torch.int32, device="cuda")
    L.kv_stream_read_tiles(src_d, n_src, tile_bytes, order_d, n, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == expect


def test_debug_checks_catch_contract_violations():
    """With the library's debug checks on, a store or a decode with the
    current token's store that would write one physical block for two
    sequences fails before launching, and so does a shared-prefix decode whose
    tables do not hold the same prefix blocks; valid calls go through (and
    with the checks off the same calls are not inspected)."""
    announce("debug-checks")
    from paged_block_quantized_amd import PBQError, _lib as L
    bs, hkv, d, hq = 16, 2, 64, 4
    n = 3 * bs
    dev = torch.device("cuda")
    prev = L.kv_set_debug_checks(True)
    try:
        pool = make_pool(32, bs, hkv, d, "i8", max_seqs=4)
        pool.alloc(0, n)                 # three full blocks
        assert pool.fork(0, 1) == []     # sequence 1 shares them (aligned: no copy)
        pool.alloc(2, bs + 4)            # a sequence of its own
        rows = torch.zeros((3, hkv, d), dtype=torch.float16, device=dev)
        # one token at position n - 1 of sequences 0 and 1: both in their shared block 2
        tables, _, slots = pool.batch_tables([0, 1, 2], 4)
        cu = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device=dev)
        start = torch.tensor([n - 1, n - 1, bs + 3], dtype=torch.int32, device=dev)
        with pytest.raises(PBQError, match="written for sequences 0 and 1"):
            pool.quantize_store(rows, rows, cu, start, tables.to(dev), slots.to(dev), 1)
        # the same token of sequences 0 and 2 only: disjoint blocks, accepted
        t02, _, s02 = pool.batch_tables([0, 2], 4)
        pool.quantize_store(rows[:2], rows[:2], cu[:3], start[[0, 2]].contiguous(), t02.to(dev), s02.to(dev), 1)
        torch.cuda.synchronize()
        # the fused store of the current token (position n - 1) of sequences 0 and 1
        q = torch.zeros((2, hq, d), dtype=torch.float16, device=dev)
        out = torch.empty_like(q)
        ctx01 = torch.tensor([n, n], dtype=torch.int32, device=dev)
        t01, _, s01 = pool.batch_tables([0, 1], 4)
        with pytest.raises(PBQError, match="paged_attn_decode_append: block"):
            pool.decode_append(rows[:2], rows[:2], s01.to(dev), q, out, t01.to(dev), ctx01, n, 0.125, 2048)
        # a shared prefix of two blocks, which sequence 1's table does not hold
        bad = t01.clone()
        bad[1, 0] = int(t02[1, 0])
        with pytest.raises(PBQError, match="differs from sequence 0's"):
            pool.decode_shared_prefix(q, out, bad.to(dev), ctx01, n, 0.125, 32, 32)
        pool.decode_shared_prefix(q, out, t01.to(dev), ctx01, n, 0.125, 32, 32)   # the real tables
        torch.cuda.synchronize()
        assert L.kv_set_debug_checks(False) == 1
        pool.decode_shared_prefix(q, out, t01.to(dev), ctx01, n, 0.125, 32, 32)
        torch.cuda.synchronize()
    finally:
        L.kv_set_debug_checks(prev)

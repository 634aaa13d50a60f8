"""paged_attn_decode_append_noalloc (the fused store + decode with the
library's own scratch instead of a workspace argument) against
paged_attn_decode_append, through the C ABI: outputs and every pool array
bit for bit, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), with split partitions (the
scratch holds the partial results) and in a single pass (no scratch)."""

import numpy as np
import pytest
import torch

from gpu_util import announce, make_pool, zp_arrays

pytestmark = pytest.mark.gpu


def _pools(bs, d, vc, hkv, ctx, seed):
    """Two pools holding the same ctx - 1 stored tokens per sequence with the
    current token reserved, plus the step's inputs."""
    S = len(ctx)
    rng = np.random.default_rng(seed)
    hk = [rng.standard_normal((c, hkv, d)).astype(np.float16) for c in ctx]
    hv = [rng.standard_normal((c, hkv, d)).astype(np.float16) for c in ctx]
    n_blocks = sum((c + bs - 1) // bs for c in ctx) + 2
    order = rng.permutation(n_blocks)
    max_blocks = max((c + bs - 1) // bs for c in ctx)
    dev = torch.device("cuda")
    out = []
    for _ in range(2):
        pool = make_pool(n_blocks, bs, hkv, d, vc, max_seqs=S, free_order=order)
        for s, c in enumerate(ctx):
            pool.alloc(s, c - 1)
        tables, _, slots = pool.batch_tables(list(range(S)), max_blocks)
        lens = [c - 1 for c in ctx]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        k = torch.from_numpy(np.concatenate([h[:c - 1] for h, c in zip(hk, ctx)])).to(dev)
        v = torch.from_numpy(np.concatenate([h[:c - 1] for h, c in zip(hv, ctx)])).to(dev)
        pool.quantize_store(k, v, cu, torch.zeros(S, dtype=torch.int32, device=dev), tables.to(dev),
                            slots.to(dev), max(max(lens), 1))
        for s in range(S):
            assert pool.append(s, 1) == []
        tables, ctx_h, slots = pool.batch_tables(list(range(S)), max_blocks)
        out.append((pool, tables.to(dev), ctx_h.to(dev), slots.to(dev)))
    k_new = torch.from_numpy(np.stack([h[c - 1] for h, c in zip(hk, ctx)])).to(dev)
    v_new = torch.from_numpy(np.stack([h[c - 1] for h, c in zip(hv, ctx)])).to(dev)
    return out, k_new, v_new, max_blocks


CASES = [
    # (block size, head dim, V codec, query heads per KV head)
    (16, 128, "i8", 1),
    (32, 128, "i4", 8),
    (32, 64, "fp8", 4),
    (16, 64, "i8a", 1),
    (32, 128, "k4i4", 8),
    (16, 64, "k4i8", 1),
]


@pytest.mark.parametrize("bs,d,vc,g", CASES)
def test_noalloc_matches_decode_append(bs, d, vc, g):
    from paged_block_quantized_amd import _lib as L
    hkv = 2
    hq = g * hkv
    # call 1: larger; call 2: fewer, shorter sequences (the scratch still
    # holds call 1's partial results); then a single pass
    calls = [([1, bs + 1, 700, 2100, 3 * bs + 5, 1500, 64], 256),
             ([bs - 1, 300, 901], 128),
             ([5, 2 * bs, 260], 4096)]
    for i, (ctx, part) in enumerate(calls):
        announce("noalloc", bs, d, vc, g, "call", i, ctx, part)
        pools, k_new, v_new, max_blocks = _pools(bs, d, vc, hkv, ctx, seed=100 * i + bs + d + g)
        (pa, ta, ca, sa), (pb, tb, cb, sb) = pools
        S = len(ctx)
        rng = np.random.default_rng(7 + i)
        q = torch.from_numpy(rng.standard_normal((S, hq, d)).astype(np.float16)).cuda()
        sm = 1.0 / np.sqrt(d)
        out_a = torch.empty_like(q)
        pa.decode_append(k_new, v_new, sa, q, out_a, ta, ca, max(ctx), sm, part)
        out_b = torch.full_like(q, float("nan"))
        L.paged_attn_decode_append_noalloc(pb.desc, pb.mem, k_new, v_new, sb, q, out_b, S, hq, tb, max_blocks,
                                           cb, max(ctx), sm, part)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"call {i}: outputs differ"
        for name in ("k_codes", "v_codes", "k_scale", "v_scale", "tail_k", "tail_v") + zp_arrays(vc):
            assert torch.equal(pa.arrays[name], pb.arrays[name]), f"call {i}: {name} differs"


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    """A call whose split-K workspace exceeds the scratch fails before any
    device work, with the sizes in the message."""
    from paged_block_quantized_amd import KVPool
    from paged_block_quantized_amd import _lib as L
    pool = KVPool(8, 16, 2, 128, "i8", max_seqs=1)
    S, hq, ctx = 4096, 2, 65536   # 4096 x 2 x 256 partitions x 520 bytes > 64 MiB
    assert L.paged_attn_workspace_bytes(pool.desc, S, hq, ctx, 256) > 64 << 20
    t = torch.zeros((S, ctx // 16), dtype=torch.int32, device="cuda")
    c = torch.zeros(S, dtype=torch.int32, device="cuda")
    q = torch.zeros((S, hq, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(L.PBQError, match="scratch"):
        L.paged_attn_decode_append_noalloc(pool.desc, pool.mem, q, q, c, q, q, S, hq, t, ctx // 16, c, ctx,
                                           0.1, 256)

"""Helpers for the GPU parity tests: run a small case through the HIP path
(libpbq via the binding) and through the oracle on the same inputs."""

import sys

import numpy as np
import torch

from oracle import allocator as A
from oracle import attention, paged

ATOL, RTOL = 2e-3, 1e-2   # |gpu - ref| <= ATOL + RTOL * |ref|, fp32 accumulate


def codecs(spec):
    """(K codec, V codec) of a test's codec name: "k4i4" and "k4i8" are INT4 K
    with INT4 or INT8 V, "fp8" is FP8 K and V, any other name is INT8 K with
    that V codec."""
    if spec.startswith("k4"):
        return "i4", spec[2:]
    return ("fp8" if spec == "fp8" else "i8"), spec


def zp_arrays(spec):
    """Names of the zero-point arrays a codec pair uses."""
    kc, vc = codecs(spec)
    return (("v_zp",) if vc in ("i4", "i8a") else ()) + (("k_zp",) if kc == "i4" else ())


def make_pool(n_blocks, bs, hkv, d, spec, **kw):
    from paged_block_quantized_amd import KVPool
    kc, vc = codecs(spec)
    return KVPool(n_blocks, bs, hkv, d, vc, k_codec=kc, **kw)


def announce(*what):
    print("CASE", *what, flush=True)
    sys.stdout.flush()


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"max abs err {err.max():.3e}")
    return float(err.max())


def pool_numpy(pool):
    out = {n: pool.arrays[n].cpu().numpy() for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    out["v_zp"] = pool.arrays["v_zp"].cpu().numpy() if pool.v_zp_used else None
    out["k_zp"] = pool.arrays["k_zp"].cpu().numpy() if pool.k_zp_used else None
    return out


def assert_pool_equal(gpu_pool, opool, blocks=None):
    """Bit-exact comparison of codes, fp16 scale bits and zero points."""
    g = pool_numpy(gpu_pool)
    sel = slice(None) if blocks is None else np.asarray(blocks)
    assert np.array_equal(g["k_codes"][sel].view(np.uint8), opool.k_codes[sel].view(np.uint8)), "K codes differ"
    assert np.array_equal(g["v_codes"][sel].view(np.uint8), opool.v_codes[sel].view(np.uint8)), "V codes differ"
    assert np.array_equal(g["k_scale"][sel].view(np.uint16), opool.k_scale[sel].view(np.uint16)), "K scales differ"
    assert np.array_equal(g["v_scale"][sel].view(np.uint16), opool.v_scale[sel].view(np.uint16)), "V scales differ"
    if gpu_pool.v_zp_used:
        assert np.array_equal(g["v_zp"][sel], opool.v_zp[sel]), "V zero points differ"
    if gpu_pool.k_zp_used:
        assert np.array_equal(g["k_zp"][sel], opool.k_zp[sel]), "K zero points differ"


class SmallCase:
    """A batch of sequences with explicit fp16 histories, stored by one
    prefill call and decoded, on the GPU and in the oracle."""

    def __init__(self, hist_k, hist_v, q, hq, hkv, d, bs, v_codec, n_blocks, free_order,
                 device="cuda"):
        self.S = len(hist_k)
        self.ctx = [int(k.shape[0]) for k in hist_k]
        self.hist_k, self.hist_v, self.q = hist_k, hist_v, q
        self.hq, self.hkv, self.d, self.bs = hq, hkv, d, bs
        self.v_int4 = codecs(v_codec)[1] == "i4"
        self.device = device
        self.pool = make_pool(n_blocks, bs, hkv, d, v_codec, max_seqs=self.S, free_order=free_order,
                              device=device)
        self.model = A.BlockPoolModel(n_blocks, bs, self.S, free_order)
        self.opool = opool_for(n_blocks, hkv, bs, d, v_codec)
        for s, c in enumerate(self.ctx):
            t_gpu = self.pool.alloc(s, c)
            t_ref = self.model.alloc(s, c)
            assert t_gpu == t_ref
        self.max_blocks = max(1, max((c + bs - 1) // bs for c in self.ctx))
        tables, ctx_h, slots = self.pool.batch_tables(list(range(self.S)), self.max_blocks)
        self.tables = tables.to(device)
        self.ctx_dev = ctx_h.to(device)
        self.slots = slots.to(device)

    def store_all(self):
        lens = self.ctx
        k = torch.from_numpy(np.concatenate(self.hist_k)).to(self.device)
        v = torch.from_numpy(np.concatenate(self.hist_v)).to(self.device)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=self.device)
        st = torch.zeros(self.S, dtype=torch.int32, device=self.device)
        self.pool.quantize_store(k, v, cu, st, self.tables, self.slots, max(max(lens), 1))
        for s, c in enumerate(lens):
            paged.store_range(self.opool, self.model.table(s)[0], self.hist_k[s], self.hist_v[s], 0, c)

    def decode(self, partition=0, sm_scale=None):
        sm = 1.0 / np.sqrt(self.d) if sm_scale is None else sm_scale
        qd = torch.from_numpy(self.q).to(self.device)
        out = torch.empty_like(qd)
        self.pool.decode(qd, out, self.tables, self.ctx_dev, max(max(self.ctx), 0), sm, partition)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def reference(self, sm_scale=None):
        sm = 1.0 / np.sqrt(self.d) if sm_scale is None else sm_scale
        tables = [self.model.table(s)[0] for s in range(self.S)]
        return attention.paged_decode(self.opool, tables, self.ctx, self.q, sm)


def opool_for(n_blocks, hkv, bs, d, spec):
    """The oracle's pool for a test's codec name (see codecs)."""
    kc, vc = codecs(spec)
    return paged.PoolArrays(n_blocks, hkv, bs, d, k_codec=kc, v_codec=vc)


def normal_case(ctx, hq, hkv, d, bs, v_codec, seed, extra_blocks=3, perm=True):
    rng = np.random.default_rng(seed)
    hk = [rng.standard_normal((c, hkv, d)).astype(np.float16) for c in ctx]
    hv = [rng.standard_normal((c, hkv, d)).astype(np.float16) for c in ctx]
    q = rng.standard_normal((len(ctx), hq, d)).astype(np.float16)
    n_blocks = sum((c + bs - 1) // bs for c in ctx) + extra_blocks
    order = rng.permutation(n_blocks) if perm else None
    return SmallCase(hk, hv, q, hq, hkv, d, bs, v_codec, n_blocks, order)


def gathered_pool(setup, s):
    """This sequence's blocks as stored on the GPU, in logical order (a
    runner.DecodeSetup)."""
    pool = setup.pool
    nb = (int(setup.ctx[s]) + pool.block_size - 1) // pool.block_size
    table = setup.tables[s, :nb].long()
    g = paged.PoolArrays(nb, pool.num_kv_heads, pool.block_size, pool.head_dim, k_codec=pool.k_codec,
                         v_codec=pool.v_codec)
    g.k_codes = pool.k_codes[table].cpu().numpy()
    g.v_codes = pool.v_codes[table].cpu().numpy()
    g.k_scale = pool.k_scale[table].cpu().numpy()
    g.v_scale = pool.v_scale[table].cpu().numpy()
    if pool.v_zp_used:
        g.v_zp = pool.v_zp[table].cpu().numpy()
    if pool.k_zp_used:
        g.k_zp = pool.k_zp[table].cpu().numpy()
    return g


def check_sequence(setup, s, out, what=None):
    """Sequence s of a runner.DecodeSetup against the oracle: its blocks bit
    for bit (re-quantized from the seeded history), out[s] within tolerance."""
    from paged_block_quantized_amd import runner
    w = setup.w
    ctx = int(setup.ctx[s])
    hk, hv = runner.sequence_history(setup, s)
    nb = (ctx + w.block_size - 1) // w.block_size
    from paged_block_quantized_amd import workloads as W
    ref_pool = paged.PoolArrays(nb, w.num_kv_heads, w.block_size, w.head_dim, k_codec=W.k_codec_of(w),
                                v_codec=w.v_codec)
    paged.store_range(ref_pool, list(range(nb)), hk, hv, 0, ctx)
    g = gathered_pool(setup, s)
    assert np.array_equal(g.k_codes.view(np.uint8), ref_pool.k_codes.view(np.uint8)), f"seq {s}: K codes"
    assert np.array_equal(g.v_codes.view(np.uint8), ref_pool.v_codes.view(np.uint8)), f"seq {s}: V codes"
    assert np.array_equal(g.k_scale.view(np.uint16), ref_pool.k_scale.view(np.uint16)), f"seq {s}: K scales"
    assert np.array_equal(g.v_scale.view(np.uint16), ref_pool.v_scale.view(np.uint16)), f"seq {s}: V scales"
    if ref_pool.v_codec in ("i4", "i8a"):
        assert np.array_equal(g.v_zp, ref_pool.v_zp), f"seq {s}: zero points"
    if ref_pool.k_codec == "i4":
        assert np.array_equal(g.k_zp, ref_pool.k_zp), f"seq {s}: K zero points"
    khat, vhat = paged.gather_dequant(ref_pool, list(range(nb)), ctx)
    q = setup.q[s].cpu().numpy()
    ref = attention.decode_attention(q, khat, vhat, setup.sm_scale)
    return assert_close(out[s], ref, f"{what or w.name} seq {s}")

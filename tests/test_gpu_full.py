"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: sampled sequences are checked against the oracle (codes and
scales bit-exact through the block tables, attention within tolerance), and
the rest through properties that hold at any size."""

import numpy as np
import pytest
import torch

from oracle import paged

from gpu_util import announce, check_sequence

pytestmark = pytest.mark.gpu


def _run(name, samples):
    from paged_block_quantized_amd import runner, workloads as W
    w = W.WORKLOADS[name]
    announce("full", name, "setup")
    setup = runner.setup_decode(w)
    announce("full", name, "step")
    setup.step()
    torch.cuda.synchronize()
    out = setup.out.cpu().numpy()
    assert np.all(np.isfinite(out))
    for s in samples:
        announce("full", name, "oracle seq", s)
        check_sequence(setup, s, out)
    # the step is idempotent: a second step gives bitwise the same output
    setup.step()
    torch.cuda.synchronize()
    assert np.array_equal(setup.out.cpu().numpy().view(np.uint16), out.view(np.uint16))
    return setup


def test_llama7b_full():
    _run("llama7b", samples=[0, 9, 13, 22, 31])


@pytest.mark.parametrize("name", ["llama7b_fp8", "llama7b_i8a", "gqa70b_fp8", "llama7b_k4v4", "llama7b_k4v8",
                                  "gqa70b_k4"])
def test_codec_variants_full(name):
    """The FP8, INT8-asymmetric and INT4-K workloads at full size, sampled
    sequences against the oracle."""
    _run(name, samples=[0, 11, 17, 31] if name.startswith("llama") else [0, 40, 77, 127])


def test_shared_prefix_full():
    """The step reads the 4096-token prefix once (paged_attn_decode_shared_prefix);
    the per-sequence path (paged_attn_decode_append) gives the same pool bit
    for bit and outputs within tolerance of it."""
    setup = _run("shared_prefix", samples=[0, 10, 21, 31])
    assert setup.shared == 4096
    st = setup.pool.stats()
    assert st["used"] == 28800 and st["shared"] == 128 and st["free"] == 0
    shared_out = setup.out.clone()
    codes = (setup.pool.k_codes.clone(), setup.pool.v_codes.clone())
    announce("full shared_prefix per-sequence path")
    setup.step_unshared()
    torch.cuda.synchronize()
    assert torch.equal(codes[0], setup.pool.k_codes) and torch.equal(codes[1], setup.pool.v_codes)
    for s in (0, 17, 31):
        check_sequence(setup, s, setup.out.cpu().numpy(), "shared_prefix per-sequence")
    diff = (setup.out.float() - shared_out.float()).abs().max().item()
    assert diff <= 4e-3, diff


def test_prefill_store_full():
    """64 prompts x 2048 tokens stored in one call into a 16384-block pool in
    random order; sampled sequences bit-exact; then 64 partially filled
    blocks grow by one token per step through their fill point."""
    from paged_block_quantized_amd import KVPool, workloads as W
    w = W.WORKLOADS["prefill_store"]
    announce("full prefill_store")
    S, T, H, D, bs = w.num_seqs, w.ctx[0], w.num_kv_heads, w.head_dim, w.block_size
    pool = KVPool(w.pool_blocks, bs, H, D, "i8", max_seqs=S,
                  free_order=W.free_order(w, w.pool_blocks))
    for s in range(S):
        pool.alloc(s, T)
    tables, _, slots = pool.batch_tables(list(range(S)), T // bs)
    tables, slots = tables.cuda(), slots.cuda()
    ks, vs = zip(*[W.kv_tokens(w, s, T, "cuda") for s in range(S)])
    k, v = torch.cat(ks), torch.cat(vs)
    cu = torch.arange(0, (S + 1) * T, T, dtype=torch.int32, device="cuda")
    st = torch.zeros(S, dtype=torch.int32, device="cuda")
    pool.quantize_store(k, v, cu, st, tables, slots, T)
    torch.cuda.synchronize()
    for s in (0, 37, 63):
        announce("full prefill_store oracle seq", s)
        hk, hv = ks[s].cpu().numpy(), vs[s].cpu().numpy()
        nb = T // bs
        ref = paged.PoolArrays(nb, H, bs, D, False)
        paged.store_range(ref, list(range(nb)), hk, hv, 0, T)
        t = tables[s].long()
        assert np.array_equal(pool.k_codes[t].cpu().numpy(), ref.k_codes)
        assert np.array_equal(pool.v_codes[t].cpu().numpy(), ref.v_codes)
        assert np.array_equal(pool.k_scale[t].cpu().numpy().view(np.uint16), ref.k_scale.view(np.uint16))
        assert np.array_equal(pool.v_scale[t].cpu().numpy().view(np.uint16), ref.v_scale.view(np.uint16))
    # decode appends: 64 fresh sequences with partial last blocks (1..15 rows)
    announce("full prefill_store appends")
    rng = np.random.default_rng([w.seed, 7])
    fill = rng.integers(1, bs, S)
    for s in range(S):
        pool.release(s)
    for s in range(S):
        pool.alloc(s, int(fill[s]))
    hist = [W.kv_tokens(w, 100 + s, int(fill[s]) + 16, "cuda") for s in range(S)]
    tables, _, slots = pool.batch_tables(list(range(S)), 2)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(fill)]), dtype=torch.int32, device="cuda")
    pool.quantize_store(torch.cat([h[0][:f] for h, f in zip(hist, fill)]),
                        torch.cat([h[1][:f] for h, f in zip(hist, fill)]),
                        cu, torch.zeros(S, dtype=torch.int32, device="cuda"),
                        tables.cuda(), slots.cuda(), int(fill.max()))
    for step in range(16):
        for s in range(S):
            assert pool.append(s, 1) == []
        tables, _, slots = pool.batch_tables(list(range(S)), 2)
        kn = torch.cat([h[0][f + step:f + step + 1] for h, f in zip(hist, fill)])
        vn = torch.cat([h[1][f + step:f + step + 1] for h, f in zip(hist, fill)])
        pool.quantize_store(kn, vn, torch.arange(S + 1, dtype=torch.int32, device="cuda"),
                            torch.tensor(fill + step, dtype=torch.int32, device="cuda"),
                            tables.cuda(), slots.cuda(), 1)
    torch.cuda.synchronize()
    tables, ctx_h, _ = pool.batch_tables(list(range(S)), 2)
    for s in range(S):
        n = int(ctx_h[s])
        hk, hv = hist[s][0].cpu().numpy(), hist[s][1].cpu().numpy()
        ref = paged.PoolArrays(2, H, bs, D, False)
        paged.store_range(ref, [0, 1], hk, hv, 0, n)
        t = tables[s].long()
        assert np.array_equal(pool.k_codes[t].cpu().numpy(), ref.k_codes), s
        assert np.array_equal(pool.v_codes[t].cpu().numpy(), ref.v_codes), s
        assert np.array_equal(pool.k_scale[t].cpu().numpy().view(np.uint16), ref.k_scale.view(np.uint16)), s
        assert np.array_equal(pool.v_scale[t].cpu().numpy().view(np.uint16), ref.v_scale.view(np.uint16)), s


def test_gqa70b_full():
    setup = _run("gqa70b", samples=[0, 33, 64, 127])
    assert setup.w.num_q_heads // setup.w.num_kv_heads == 8


def test_llama7b_swap_round_trip_full():
    """A quarter of the llama7b batch (8 sequences x 4096 tokens: 2048
    blocks of 128 KiB) swapped out to pinned host memory, its device blocks
    overwritten by another owner, and swapped back into other blocks: the
    decode over the stored tokens is bitwise unchanged and the swapped
    sequences still match the oracle."""
    from oracle import allocator as A
    from paged_block_quantized_amd import runner, workloads as W
    w = W.WORKLOADS["llama7b"]
    announce("full swap llama7b", "setup")
    setup = runner.setup_decode(w)
    setup.step()
    setup.attend()
    torch.cuda.synchronize()
    out0 = setup.out.clone()
    pool = setup.pool
    group = list(range(0, w.num_seqs, 4))
    nb = 4096 // w.block_size
    pool.set_swap_space(len(group) * nb, len(group))
    announce("full swap llama7b", "out")
    plan = pool.swap_out(group)
    srcs = [e[1] for e in plan if e[0] == A.SWAP_BLOCK_OUT]
    assert len(srcs) == len(group) * nb and len(plan) == len(srcs)   # full blocks: no slot rows
    idx = torch.tensor(srcs, device="cuda")
    pool.k_codes[idx] = 0
    pool.v_codes[idx] = 0
    pool.k_scale[idx] = 0
    announce("full swap llama7b", "in")
    pool.swap_in(group)
    tables, _, slots = pool.batch_tables(list(range(w.num_seqs)), setup.tables.shape[1])
    assert not torch.equal(tables[group].cuda(), setup.tables[group])
    setup.tables, setup.slots = tables.cuda(), slots.cuda()
    setup.attend()
    torch.cuda.synchronize()
    assert torch.equal(setup.out.view(torch.int16), out0.view(torch.int16))
    out = setup.out.cpu().numpy()
    for s in (group[1], group[-1]):
        announce("full swap llama7b", "oracle seq", s)
        check_sequence(setup, s, out, "llama7b after swap")


@pytest.mark.parametrize("name", ["prefill_chunk", "prefill_chunk_gqa"])
def test_multi_query_full(name):
    """Chunked prefill at full size in the benchmark's launch configuration:
    sampled query rows (first, middle and last of sampled sequences) against
    the oracle; a second call gives bitwise the same output."""
    from oracle import attention
    from paged_block_quantized_amd import runner, workloads as W
    w = W.WORKLOADS[name]
    announce("full multi", name, "setup")
    setup = runner.setup_multi(w)
    setup.run()
    torch.cuda.synchronize()
    out = setup.out.clone()
    assert torch.isfinite(out.float()).all()
    setup.run()
    torch.cuda.synchronize()
    assert torch.equal(setup.out.view(torch.int16), out.view(torch.int16))
    out = out.cpu().numpy()
    n = w.q_len
    for s in (0, w.num_seqs - 1):
        announce("full multi", name, "oracle seq", s)
        ctx = int(setup.ctx[s])
        k, v = W.kv_tokens(w, s, ctx, "cuda")
        nb = (ctx + w.block_size - 1) // w.block_size
        ref_pool = paged.PoolArrays(nb, w.num_kv_heads, w.block_size, w.head_dim, k_codec=W.k_codec_of(w),
                                    v_codec=w.v_codec)
        paged.store_range(ref_pool, list(range(nb)), k.cpu().numpy(), v.cpu().numpy(), 0, ctx)
        khat, vhat = paged.gather_dequant(ref_pool, list(range(nb)), ctx)
        for i in (0, n // 2, n - 1):
            row = s * n + i
            pos = ctx - n + i
            ref = attention.decode_attention(setup.q[row].cpu().numpy(), khat[:, :pos + 1], vhat[:, :pos + 1],
                                             setup.sm_scale)
            from gpu_util import assert_close
            assert_close(out[row], ref, f"{name} seq {s} query {i}")

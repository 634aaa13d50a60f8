"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay gives the eager call's outputs and pool bit for bit.

The captured calls cover the launch forms a serving loop would capture: a
single pass with the fused store (MHA and the paired grouped-query groups),
a split-partition MHA step (store fused into the last partition), and the
shared-prefix step, whose prefix partitions run on the library's side stream
(forked from the captured stream and joined back before the reduce, so the
graph holds both streams' kernels).  Between replays the test runs eager
work of its own (clearing the outputs, a synchronization) and checks each
replay separately."""

import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import announce, codecs

pytestmark = pytest.mark.gpu

CASES = [
    # (name, block_size, head_dim, v codec, query heads per KV head, KV heads, seqs, partition, shared prefix)
    ("single-pass MHA", 16, 128, "i8", 1, 2, 5, 0, 0),
    ("single-pass grouped (paired)", 32, 128, "i4", 8, 2, 7, 0, 0),
    ("split MHA", 32, 64, "i4", 1, 2, 4, 64, 0),
    ("shared prefix MHA", 32, 128, "i4", 1, 2, 6, 64, 128),
    ("shared prefix grouped", 16, 128, "fp8", 4, 2, 5, 64, 128),
]


@pytest.mark.parametrize("name,bs,d,vc,g,hkv,S,part,prefix", CASES)
def test_step_replays_from_a_graph(name, bs, d, vc, g, hkv, S, part, prefix):
    from paged_block_quantized_amd import runner, workloads as W
    announce("graph replay", name, bs, d, vc, g, hkv, S, part, prefix)
    base = W.WORKLOADS["shared_prefix" if prefix else "gqa70b"]
    ctx = tuple(prefix + x for x in [1, bs + 1, 3 * bs + 5, 300, 77, 2 * bs, 130][:S])
    w = dataclasses.replace(base, name="graph_small", num_seqs=S, num_q_heads=g * hkv, num_kv_heads=hkv,
                            head_dim=d, block_size=bs, v_codec=codecs(vc)[1], k_codec=codecs(vc)[0],
                            ctx_kind="list", ctx=ctx, prefix=prefix, partition=part,
                            outlier_frac=0.0, seed=5 * bs + d + g + S)
    setup = runner.setup_decode(w, partition=part or None)
    assert setup.shared == prefix
    # eager: the current tokens stored, then the step again (the same token
    # stored again leaves the pool as it is), its outputs the reference
    setup.step()
    setup.step()
    torch.cuda.synchronize()
    ref = setup.out.clone()
    pool = {n: t.clone() for n, t in setup.pool.arrays.items()}
    assert torch.isfinite(ref.float()).all()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        setup.step()
    torch.cuda.synchronize()
    for i in range(4):
        setup.out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(setup.out, ref), f"{name}: replay {i} differs from the eager step"
        for n, t in pool.items():
            assert torch.equal(setup.pool.arrays[n], t), f"{name}: replay {i} changed {n}"
    # eager again after the replays
    setup.out.fill_(float("nan"))
    setup.step()
    torch.cuda.synchronize()
    assert torch.equal(setup.out, ref), f"{name}: eager step after the replays differs"
    del graph
    np.testing.assert_array_equal(setup.out.cpu().numpy(), ref.cpu().numpy())

"""Pins for the oracle's block-pool model (oracle/allocator.py): a hand-traced
golden sequence, the page's demo, the workloads' block counts, and invariants
under random operation sequences."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as hst

from oracle import allocator as A
from oracle import kv_size

from alloc_harness import GOLDEN, ContentSim, apply_op, random_ops, run_golden_trace


class ModelAdapter:
    def __init__(self, n, bs, max_seqs, free_order):
        self.m = A.BlockPoolModel(n, bs, max_seqs, free_order)

    def alloc(self, s, n):
        return self.m.alloc(s, n)

    def alloc_prefix(self, s, toks):
        return self.m.alloc_prefix(s, toks)

    def fork(self, p, c):
        return self.m.fork(p, c)

    def append(self, s, n):
        return self.m.append(s, n)

    def release(self, s):
        return self.m.release(s)

    def swap_out(self, seqs):
        return self.m.swap_out(seqs)

    def swap_in(self, seqs):
        return self.m.swap_in(seqs)

    def table(self, s):
        return self.m.table(s)

    def stats(self):
        return self.m.stats()

    def free_list(self):
        return list(self.m.free)


def test_golden_trace():
    run_golden_trace(ModelAdapter, A.AllocError)


def test_page_demo_counts():
    g = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["demo_allocation"]
    m = A.BlockPoolModel(g["num_blocks"], g["block_size"], 4)
    t = m.alloc(0, g["request_tokens"])
    assert len(t) == g["blocks_taken"]
    assert m.stats()["free"] == g["free_after"]


def test_workload_block_counts():
    g = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["workload_block_counts"]
    tiny = g["tiny"]
    perm = np.random.default_rng(0).permutation(tiny["pool"])
    m = A.BlockPoolModel(tiny["pool"], tiny["block_size"], 8, perm)
    for s, c in enumerate(tiny["ctx"]):
        assert len(m.alloc(s, c)) == tiny["blocks"][s]
    st = m.stats()
    assert st["used"] == tiny["used"] and st["free"] == tiny["free"]
    # LIFO over the permutation: sequence 0 takes the permutation's last id
    assert m.table(0)[0] == [int(perm[-1])]
    assert m.table(1)[0] == [int(perm[-2]), int(perm[-3])]

    g7 = g["llama7b_layer"]
    assert g7["seqs"] * kv_size.num_blocks_for(g7["ctx"], g7["block_size"]) == g7["blocks_total"]
    gp = g["prefill_store"]
    assert gp["seqs"] * kv_size.num_blocks_for(gp["tokens"], gp["block_size"]) == gp["blocks_total"]

    sp = g["shared_prefix"]
    m = A.BlockPoolModel(sp["physical"], sp["block_size"], sp["seqs"] + 1)
    m.alloc(-1, sp["prefix"])
    for s in range(sp["seqs"]):
        assert m.fork(-1, s) == []            # block-aligned prefix: no slot copy
    m.release(-1)
    for s in range(sp["seqs"]):
        assert m.append(s, sp["ctx"] - sp["prefix"]) == []   # no COW at an aligned boundary
    m.check_invariants()
    st = m.stats()
    assert st["used"] == sp["physical"] and st["free"] == 0
    assert st["shared"] == sp["prefix_blocks"]
    t0 = m.table(0)[0]
    assert len(t0) == sp["logical_per_seq"]
    assert all(m.refcount[b] == sp["prefix_refcount"] for b in t0[:sp["prefix_blocks"]])
    with pytest.raises(A.NoBlocks):
        m.append(0, 1)


def test_unaligned_prefix_copy_path():
    """A prefix ending mid-block: the fork copies the tail slot and the first
    append of each child copies only the shared partial block."""
    bs = 32
    m = A.BlockPoolModel(64, bs, 4)
    m.alloc(100, 4080 % 1024)          # 1008 tokens = 31.5 blocks
    last = m.table(100)[0][-1]
    assert m.fork(100, 0) == [(A.COPY_SLOT, 0, 1)]
    cp = m.append(0, 1)
    assert len(cp) == 1 and cp[0][0] == A.COPY_BLOCK and cp[0][1] == last
    assert m.table(0)[0][:-1] == m.table(100)[0][:-1]
    assert m.table(0)[0][-1] != last
    assert m.append(100, 1) == []      # the parent now owns `last` alone
    m.check_invariants()


def test_failed_ops_leave_state_unchanged():
    m = A.BlockPoolModel(4, 4, 2)
    m.alloc(0, 9)
    snap = (list(m.free), list(m.refcount), {k: (list(v.table), v.num_tokens) for k, v in m.seqs.items()})
    with pytest.raises(A.NoBlocks):
        m.alloc(1, 8)
    with pytest.raises(A.NoBlocks):
        m.append(0, 8)
    with pytest.raises(A.UnknownSeq):
        m.append(5, 1)
    with pytest.raises(A.BadState):
        m.alloc(0, 1)
    m.alloc(1, 0)
    with pytest.raises(A.NoSlots):
        m.alloc(2, 0)
    m.release(1)
    assert snap == (list(m.free), list(m.refcount), {k: (list(v.table), v.num_tokens) for k, v in m.seqs.items()})


@settings(max_examples=60, deadline=None)
@given(seed=hst.integers(0, 2 ** 31 - 1), n_blocks=hst.integers(1, 24),
       bs=hst.sampled_from([1, 2, 4, 16]))
def test_random_ops_keep_invariants(seed, n_blocks, bs):
    rng = np.random.default_rng(seed)
    m = A.BlockPoolModel(n_blocks, bs, 6, rng.permutation(n_blocks))
    for op in random_ops(rng, 80):
        apply_op(m, op, A.AllocError)
        m.check_invariants()


def test_prefix_cache_hand_worked():
    """yunthe "prefix caching", as read: full blocks matched from the first,
    keyed by (parent block, token ids); hits shared; fresh full blocks
    indexed; the partial block private; index entries leave with the block."""
    m = A.BlockPoolModel(16, 4, 8)          # free stack 0..15, popped from 15
    a = [1, 1, 1, 1, 2, 2, 2, 2, 3, 3]
    assert m.alloc_prefix(0, a) == ([15, 14, 13], 0)
    assert m.stats()["cached"] == 2         # blocks 15 and 14; 13 is partial
    b = [1, 1, 1, 1, 2, 2, 2, 2, 4, 4, 4, 4, 5]
    assert m.alloc_prefix(1, b) == ([15, 14, 12, 11], 8)
    assert m.refcount[15] == 2 and m.refcount[14] == 2
    assert m.alloc_prefix(2, [1, 1, 1, 1, 9, 9, 9, 9]) == ([15, 10], 4)
    # the same ids without the same parent are no hit
    assert m.alloc_prefix(3, [2, 2, 2, 2]) == ([9], 0)
    # the same prompt again: both full blocks hit, the partial one is fresh
    assert m.alloc_prefix(4, a) == ([15, 14, 8], 8)
    assert m.stats()["cached"] == 5         # 15, 14, 12, 10, 9
    m.release(1)                            # 12 and 11 reach zero; 12 leaves the index
    assert m.stats()["cached"] == 4
    # its third block left the index with block 12: recomputed into a fresh
    # block (11, pushed last), the partial one takes 12
    assert m.alloc_prefix(5, b) == ([15, 14, 11, 12], 8)
    # an empty request and a request shorter than a block: nothing to match
    assert m.alloc_prefix(6, []) == ([], 0)
    m.check_invariants()
    for s in list(m.seqs):
        m.release(s)
    assert m.stats()["cached"] == 0 and m.index == {} and m.stats()["free"] == 16
    m.check_invariants()


def test_prefix_cache_failure_leaves_state_unchanged():
    m = A.BlockPoolModel(3, 2, 4)
    m.alloc_prefix(0, [7, 7, 8, 8])
    snap = (list(m.free), list(m.refcount), dict(m.index))
    with pytest.raises(A.NoBlocks):
        m.alloc_prefix(1, [7, 7, 9, 9, 9, 9])   # one hit, two fresh, one free
    with pytest.raises(A.BadState):
        m.alloc_prefix(0, [7, 7])
    assert snap == (list(m.free), list(m.refcount), dict(m.index))


@settings(max_examples=60, deadline=None)
@given(seed=hst.integers(0, 2 ** 31 - 1), n_blocks=hst.integers(1, 24),
       bs=hst.sampled_from([1, 2, 4, 8]))
def test_prefix_cache_hits_are_equal_prefixes(seed, n_blocks, bs):
    """Brute force: after any op sequence, every cached block's parent chain
    spells a token prefix, and every sequence allocated through the cache
    holds, at each indexed position, the block that spells its own prefix."""
    rng = np.random.default_rng(seed)
    m = A.BlockPoolModel(n_blocks, bs, 6, rng.permutation(n_blocks))
    toks = {}
    for op in random_ops(rng, 80, prefix=True):
        rec = apply_op(m, op, A.AllocError)
        if rec[0] == "ok" and op[0] == "prefix":
            toks[op[1]] = op[2]
        elif rec[0] == "ok" and op[0] in ("alloc", "free"):
            toks.pop(op[1], None)
        m.check_invariants()

        def spelled(b):
            parent, ids = m.key_of[b]
            return (spelled(parent) if parent != -1 else []) + list(ids)

        for s, ids in toks.items():
            if s not in m.seqs:
                continue
            table = m.seqs[s].table
            for j, blk in enumerate(table[:len(ids) // bs]):
                if blk in m.key_of:
                    assert spelled(blk) == ids[:(j + 1) * bs]


def test_swap_hand_worked():
    """deepinsea "Swap", as read: a group moves the blocks only it holds (a
    block shared with a sequence outside the group stays on the device), its
    slots move with the rows of a partial last block; swap-in takes fresh
    device blocks and the lowest free slot; both are all-or-nothing."""
    O, I, SO, SI = A.SWAP_BLOCK_OUT, A.SWAP_BLOCK_IN, A.SWAP_SLOT_OUT, A.SWAP_SLOT_IN
    m = A.BlockPoolModel(8, 4, 3)             # free stack 0..7, popped from 7
    m.set_swap_space(4, 2)                    # host stack 0..3, popped from 3
    assert m.alloc(1, 10) == [7, 6, 5]        # two rows in the partial block
    assert m.fork(1, 2) == [(A.COPY_SLOT, 0, 1)]
    assert m.append(2, 1) == [(A.COPY_BLOCK, 5, 4)]
    assert m.alloc(3, 4) == [3]
    # 7 and 6 are also held by sequence 2: only 5 moves
    assert m.swap_out([1]) == [(O, 5, 3, 0), (SO, 0, 0, 2)]
    assert m.table(1) == ([7, 6, -4], 10, -1)
    assert m.free == [0, 1, 2, 5]
    assert {k: m.stats()[k] for k in ("free", "host_free", "swapped")} == \
        dict(free=4, host_free=3, swapped=1)
    with pytest.raises(A.BadState):
        m.append(1, 1)
    with pytest.raises(A.BadState):
        m.fork(1, 9)
    with pytest.raises(A.BadState):
        m.swap_out([1])
    assert m.alloc(4, 8) == [5, 2]            # slot 0, freed by the swap
    with pytest.raises(A.NoSlots):            # slots 0, 1, 2 all held
        m.swap_in([1])
    m.release(3)
    assert m.swap_in([1]) == [(I, 3, 3, 0), (SI, 0, 2, 2)]
    assert m.table(1) == ([7, 6, 3], 10, 2)
    # both forks together: every block is the group's own, shared ones once
    assert m.swap_out([1, 2]) == [(O, 7, 3, 0), (O, 6, 2, 0), (O, 3, 1, 0), (O, 4, 0, 0),
                                  (SO, 2, 0, 2), (SO, 1, 1, 3)]
    assert m.table(1) == ([-4, -3, -2], 10, -1)
    assert m.table(2) == ([-4, -3, -1], 11, -2)
    assert m.free == [0, 1, 7, 6, 3, 4]
    # one of them back: the host blocks it shares stay for the other
    assert m.swap_in([2]) == [(I, 3, 4, 0), (I, 2, 3, 0), (I, 0, 6, 0), (SI, 1, 1, 3)]
    assert m.table(2) == ([4, 3, 6], 11, 1)
    assert m.host_free == [0] and m.host_refcount == [0, 1, 1, 1]
    m.release(1)
    assert m.host_free == [0, 3, 2, 1]
    st = m.stats()
    assert (st["free"], st["used"], st["host_free"], st["swapped"], st["seqs"]) == (3, 5, 4, 0, 2)
    m.check_invariants()


def test_swap_failure_leaves_state_unchanged():
    m = A.BlockPoolModel(6, 2, 3)
    m.set_swap_space(2, 1)
    m.alloc(0, 6)
    m.alloc(1, 1)

    def snap():
        return (list(m.free), list(m.refcount), list(m.host_free), list(m.host_refcount),
                {k: (list(v.table), v.num_tokens, v.slot, v.swapped) for k, v in m.seqs.items()})

    before = snap()
    with pytest.raises(A.NoBlocks):           # three blocks, two host blocks
        m.swap_out([0])
    with pytest.raises(A.NoSlots):            # two sequences, one host slot
        m.swap_out([1, 0])
    with pytest.raises(A.BadArg):
        m.swap_out([1, 1])
    with pytest.raises(A.UnknownSeq):
        m.swap_out([1, 5])
    with pytest.raises(A.BadState):
        m.swap_in([1])
    assert snap() == before
    m.swap_out([1])
    with pytest.raises(A.BadState):           # resize while a sequence is out
        m.set_swap_space(4, 4)
    m.check_invariants()


@settings(max_examples=80, deadline=None)
@given(seed=hst.integers(0, 2 ** 31 - 1), n_blocks=hst.integers(1, 24),
       bs=hst.sampled_from([1, 2, 4, 8]), host_blocks=hst.integers(0, 16))
def test_tables_and_plans_keep_every_sequence_data(seed, n_blocks, bs, host_blocks):
    """Brute force over random op sequences (prefix-cached allocations and
    swaps included): running each op's copies and swap plans on stamped
    blocks leaves every sequence's data where its table and slot point, and
    a prefix hit always finds the block holding that very token prefix."""
    rng = np.random.default_rng(seed)
    m = A.BlockPoolModel(n_blocks, bs, 6, rng.permutation(n_blocks))
    m.set_swap_space(host_blocks, 3)
    sim = ContentSim(bs)
    for op in random_ops(rng, 160, max_seq_id=6, prefix=True, swap=True):
        rec = apply_op(m, op, A.AllocError)
        sim.apply(m, op, rec)
        m.check_invariants()

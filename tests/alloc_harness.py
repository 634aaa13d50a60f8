"""Drives a block-pool implementation through a trace or a random operation
sequence.  Used with the oracle model and with the C library's allocator, so
both are held to the same hand-traced expectations and to each other."""

import json
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def status_of(exc):
    return getattr(exc, "kind", "invalid")


def run_golden_trace(make_pool, errors):
    """``make_pool(num_blocks, block_size, max_seqs, free_order)`` returns an
    object with alloc/fork/append/release/table/stats/free_list; ``errors`` is
    the exception base class it raises."""
    g = json.load(open(os.path.join(GOLDEN, "allocator_trace.json")))
    pool = make_pool(g["num_blocks"], g["block_size"], g["max_seqs"], g["free_order"])
    for st in g["steps"]:
        op = st["op"]
        try:
            if op == "alloc":
                res = pool.alloc(st["seq"], st["n"])
                seq = st["seq"]
            elif op == "fork":
                res = pool.fork(st["parent"], st["child"])
                seq = st["child"]
            elif op == "append":
                res = pool.append(st["seq"], st["n"])
                seq = st["seq"]
            elif op == "free":
                res = pool.release(st["seq"])
                seq = None
            status = "ok"
        except errors as e:  # noqa: PERF203
            status = status_of(e)
        assert status == st.get("expect_status", "ok"), st
        if status != "ok":
            if "expect_free" in st:
                assert pool.free_list() == st["expect_free"], st
            continue
        if "expect_table" in st:
            assert pool.table(seq)[0] == st["expect_table"], st
        if "expect_slot" in st:
            assert pool.table(seq)[2] == st["expect_slot"], st
        if "expect_copies" in st:
            assert [list(c) for c in res] == st["expect_copies"], st
        if "expect_free" in st:
            assert pool.free_list() == st["expect_free"], st
    stats = pool.stats()
    assert {k: stats[k] for k in g["final_stats"]} == g["final_stats"]


def random_ops(rng, n_ops, max_seq_id=12, max_tokens=40, prefix=False):
    """A seeded list of (op, args) tuples mixing every operation, including
    ones that must fail (unknown sequences, over-allocation).  With prefix,
    a quarter of the allocations go through the prefix cache with token ids
    that share prefixes of three seeded prompts (vocabulary of 3, so that
    different prompts also share blocks)."""
    prompts = [list(rng.integers(0, 3, max_tokens)) for _ in range(3)]
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        a = int(rng.integers(0, max_seq_id))
        if prefix and r < 0.12:
            n = int(rng.integers(0, max_tokens))
            k = int(rng.integers(0, n + 1))
            toks = prompts[int(rng.integers(0, 3))][:k] + list(rng.integers(0, 3, n - k))
            ops.append(("prefix", a, [int(t) for t in toks]))
        elif r < 0.3:
            ops.append(("alloc", a, int(rng.integers(0, max_tokens))))
        elif r < 0.45:
            ops.append(("fork", a, int(rng.integers(0, max_seq_id))))
        elif r < 0.75:
            ops.append(("append", a, int(rng.integers(0, 9))))
        else:
            ops.append(("free", a))
    return ops


def apply_op(pool, op, errors):
    """Apply one op; return a comparable record of its outcome."""
    try:
        if op[0] == "alloc":
            res = pool.alloc(op[1], op[2])
        elif op[0] == "prefix":
            res = pool.alloc_prefix(op[1], op[2])
        elif op[0] == "fork":
            res = [tuple(c) for c in pool.fork(op[1], op[2])]
        elif op[0] == "append":
            res = [tuple(c) for c in pool.append(op[1], op[2])]
        else:
            res = pool.release(op[1])
        return ("ok", res)
    except errors as e:
        return (status_of(e), None)

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


def random_ops(rng, n_ops, max_seq_id=12, max_tokens=40, prefix=False, swap=False):
    """A seeded list of (op, args) tuples mixing every operation, including
    ones that must fail (unknown sequences, over-allocation).  With prefix,
    a quarter of the allocations go through the prefix cache with token ids
    that share prefixes of three seeded prompts (vocabulary of 3, so that
    different prompts also share blocks).  With swap, about one op in nine
    swaps a group of one to three sequence ids out or in (a repeated id, an
    unknown or a wrongly placed sequence must fail)."""
    prompts = [list(rng.integers(0, 3, max_tokens)) for _ in range(3)]
    ops, outs = [], []
    for _ in range(n_ops):
        r = rng.random()
        a = int(rng.integers(0, max_seq_id))
        if swap and r >= 0.89:
            if rng.random() < 0.5:
                extra = rng.integers(0, max_seq_id, int(rng.choice(3, p=[0.6, 0.3, 0.1])))
                group = [a] + [int(x) for x in extra]
                outs.append(group)
                ops.append(("swap_out", group))
            else:   # mostly a group swapped out before, or its first member
                group = [a]
                if outs and rng.random() < 0.8:
                    group = list(outs[int(rng.integers(0, len(outs)))])
                    if rng.random() < 0.3:
                        group = group[:1]
                ops.append(("swap_in", group))
        elif prefix and r < 0.12:
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
        elif op[0] == "swap_out":
            res = [tuple(c) for c in pool.swap_out(op[1])]
        elif op[0] == "swap_in":
            res = [tuple(c) for c in pool.swap_in(op[1])]
        else:
            res = pool.release(op[1])
        return ("ok", res)
    except errors as e:
        return (status_of(e), None)


class ContentSim:
    """Brute-force check that a pool's tables and copy lists keep every
    sequence's data where its table points.  Each freshly written block gets
    a unique stamp (or, for a full block allocated through the prefix cache,
    the token prefix it holds); copies and swap plans move stamps between
    device blocks, host blocks and tail slots; blocks back on a free stack
    are poisoned.  After every op each sequence must find, through its table
    (host blocks as -1 - h) and its slot, the stamps it was given."""

    POISON = ("free",)

    def __init__(self, block_size):
        self.bs = block_size
        self.dev, self.host, self.slot, self.hslot = {}, {}, {}, {}
        self.exp = {}
        self.n = 0

    def _new(self):
        self.n += 1
        return ("w", self.n)

    def _copy(self, kinds, plan):
        # entries of one call run concurrently: distinct destinations, and
        # no destination is another entry's source
        for space in ("dev", "host", "slot", "hslot"):
            dsts = [d for k, s, d, *_ in plan if kinds[k][1] == space]
            srcs = {s for k, s, d, *_ in plan if kinds[k][0] == space}
            assert len(dsts) == len(set(dsts)) and not (set(dsts) & srcs), plan
        moved = [(kinds[k], s, d) for k, s, d, *_ in plan]
        vals = [getattr(self, a)[s] for (a, _), s, _ in moved]
        for ((_, b), _, d), v in zip(moved, vals):
            getattr(self, b)[d] = v

    def apply(self, model, op, rec):
        """``model`` is the oracle's BlockPoolModel after ``op`` returned
        ``rec`` (apply_op's record)."""
        if rec[0] != "ok":
            self.check(model)
            return
        bs, kind, res = self.bs, op[0], rec[1]
        copy_kinds = {0: ("dev", "dev"), 1: ("slot", "slot")}
        swap_kinds = {0: ("dev", "host"), 1: ("host", "dev"), 2: ("slot", "hslot"), 3: ("hslot", "slot")}
        if kind in ("alloc", "prefix"):
            seq = op[1]
            table, n, _ = model.table(seq)
            hits = res[1] // bs if kind == "prefix" else 0
            toks = op[2] if kind == "prefix" else None
            exp = []
            for j, b in enumerate(table):
                full = toks is not None and (j + 1) * bs <= n
                want = ("p", tuple(toks[:(j + 1) * bs])) if full else None
                if j < hits:
                    assert self.dev[b] == want, (op, j)
                else:
                    self.dev[b] = want if full else self._new()
                exp.append(self.dev[b])
            self.exp[seq] = exp
        elif kind == "fork":
            self._copy(copy_kinds, res)
            self.exp[op[2]] = list(self.exp[op[1]])
        elif kind == "append":
            seq, add = op[1], op[2]
            self._copy(copy_kinds, res)
            table, n, _ = model.table(seq)
            exp = self.exp[seq]
            old = n - add
            if add > 0 and old % bs:
                j = len(exp) - 1
                self.dev[table[j]] = exp[j] = self._new()
            for j in range(len(exp), len(table)):
                self.dev[table[j]] = self._new()
                exp.append(self.dev[table[j]])
        elif kind in ("swap_out", "swap_in"):
            self._copy(swap_kinds, res)
        else:
            self.exp.pop(op[1])
        if kind in ("alloc", "prefix") or (kind == "append" and op[2] > 0):
            # the store writes the exact rows of a partial last block
            table, n, slot = model.table(op[1])
            if n % bs:
                self.slot[slot] = self.exp[op[1]][-1]
        for b in model.free:
            self.dev[b] = self.POISON
        for h in model.host_free:
            self.host[h] = self.POISON
        held = {st.slot for st in model.seqs.values()}
        for k in range(model.max_seqs):
            if k not in held:
                self.slot[k] = self.POISON
        for k in range(model.host_slots):
            if -1 - k not in held:
                self.hslot[k] = self.POISON
        self.check(model)

    def check(self, model):
        assert set(self.exp) == set(model.seqs)
        for seq, exp in self.exp.items():
            table, n, slot = model.table(seq)
            got = [self.dev[b] if b >= 0 else self.host[-1 - b] for b in table]
            assert got == exp, seq
            if n % self.bs:
                have = self.slot[slot] if slot >= 0 else self.hslot[-1 - slot]
                assert have == exp[-1], seq

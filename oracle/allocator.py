"""List/dict model of the physical block pool and its block tables
(test infrastructure only).

What the pages fix
------------------
* The pool is a fixed set of physical block ids handed out from a free list;
  a request of n tokens takes ceil(n / block_size) blocks, and its block table
  lists them in logical order (tbr8.org §4 ``allocate_for_request``;
  deepinsea.top "paging mechanism design" ``allocate``; yunthe.com
  "PagedAttention mechanism", block_table maps a sequence to physical ids).
* An allocation that does not fit fails as a whole (deepinsea.top
  ``allocate`` checks the free count first and returns False).
* Freeing a request gives every one of its blocks back (deepinsea.top
  ``free``); blocks carry reference counts so that clearing a conversation
  only releases blocks nobody else holds (tbr8.org §5, point 3).
* Sequences may share prefix blocks; a sequence about to modify a shared
  block gets its own copy of only that block, and tokens generated after a
  fork go to new blocks (deepinsea.top "Copy-on-Write"; yunthe.com
  "PagedAttention mechanism", third benefit).

Readings where the pages are silent or disagree
-----------------------------------------------
* Free-list order: tbr8.org pops from the front, deepinsea.top from the back.
  This model follows deepinsea.top (the page that also checks capacity): the
  free list is a stack popped from its end and pushed on release.  The initial
  stack is ``free_order`` (default 0..N-1, as both pages start from
  ``list(range(num_blocks))``); the workloads pass a seeded permutation.
* Release order: blocks are decremented in table order, and each block whose
  count reaches zero is pushed at once (deepinsea.top ``free`` appends in
  table order).
* Append: for every new token at position p, a block boundary (p % bs == 0)
  takes a fresh block; a partial last block that is shared (count > 1) is
  first replaced by a fresh private block and a (src -> dst) copy is
  recorded.  The copy is taken before any boundary block.  The whole append
  is checked against the free count first and fails as a whole.
* Tail slots: every live sequence owns one fp16 "tail" slot that holds the
  unquantized rows of its last, partially filled block, so that the block can
  be re-quantized from exact values when tokens are appended.  The pages are
  silent on how a partial block grows; this is the reading that keeps every
  block equal to a fresh quantization of its rows.  A sequence takes the
  lowest free slot; a fork whose parent has a partial last block records a
  slot copy (parent slot -> child slot).
* Error kinds: unknown sequence, sequence already present, no free blocks,
  no free slot, bad argument.  A failed call leaves the state unchanged.

Prefix caching (yunthe.com "prefix caching": a new request first looks for
blocks of the pool that already hold its prefix and, on a hit, maps them
instead of recomputing; the page gives no matching rule or lifetime):
* Only full blocks are matched, in order from the first; the lookup stops at
  the first block that is not found.  A block's identity is its parent block
  (the physical block before it, or none) and its own bs token ids, so a hit
  means the whole prefix up to and including the block is equal.
* Hits are shared (refcount + 1); the other blocks come from the free stack
  as in ``alloc``, and each fresh full block is entered in the index at
  once (its codes are the caller's to store before anything reads them).
  The partial last block is private and never entered.
* A block leaves the index when its count reaches zero (a freed block's
  codes may be overwritten by its next owner): hits are blocks some live
  sequence holds.
"""

from dataclasses import dataclass, field

COPY_BLOCK = 0  # copy codes, scales and zero points of one physical block
COPY_SLOT = 1   # copy one fp16 tail slot


class AllocError(Exception):
    kind = "invalid"


class NoBlocks(AllocError):
    kind = "no_blocks"


class NoSlots(AllocError):
    kind = "no_slots"


class UnknownSeq(AllocError):
    kind = "unknown_seq"


class BadState(AllocError):
    kind = "state"


class BadArg(AllocError):
    kind = "invalid"


@dataclass
class SeqState:
    table: list
    num_tokens: int
    slot: int


@dataclass
class BlockPoolModel:
    num_blocks: int
    block_size: int
    max_seqs: int
    free_order: list = None
    free: list = field(init=False)
    refcount: list = field(init=False)
    seqs: dict = field(init=False)
    index: dict = field(init=False)     # (parent block or -1, token ids) -> block
    key_of: dict = field(init=False)    # block -> its index key

    def __post_init__(self):
        if self.num_blocks <= 0 or self.block_size <= 0 or self.max_seqs <= 0:
            raise BadArg("sizes must be positive")
        order = list(range(self.num_blocks)) if self.free_order is None \
            else [int(b) for b in self.free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise BadArg("free_order must be a permutation of 0..N-1")
        self.free = order
        self.refcount = [0] * self.num_blocks
        self.seqs = {}
        self.index = {}
        self.key_of = {}

    # -- helpers ---------------------------------------------------------
    def _lowest_free_slot(self):
        used = {s.slot for s in self.seqs.values()}
        for k in range(self.max_seqs):
            if k not in used:
                return k
        raise NoSlots("no free tail slot")

    def _blocks_for(self, n):
        return (n + self.block_size - 1) // self.block_size

    # -- operations ------------------------------------------------------
    def alloc(self, seq: int, num_tokens: int):
        if num_tokens < 0:
            raise BadArg("num_tokens < 0")
        if seq in self.seqs:
            raise BadState("sequence already present")
        slot = self._lowest_free_slot()
        need = self._blocks_for(num_tokens)
        if need > len(self.free):
            raise NoBlocks("not enough free blocks")
        table = []
        for _ in range(need):
            b = self.free.pop()
            self.refcount[b] = 1
            table.append(b)
        self.seqs[seq] = SeqState(table, num_tokens, slot)
        return list(table)

    def alloc_prefix(self, seq: int, tokens):
        """alloc for len(tokens) tokens that reuses the indexed blocks of the
        longest matching full-block prefix; returns (table, cached tokens)."""
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if seq in self.seqs:
            raise BadState("sequence already present")
        slot = self._lowest_free_slot()
        bs = self.block_size
        need = self._blocks_for(n)
        hits = []
        parent = -1
        for j in range(n // bs):
            b = self.index.get((parent, tuple(tokens[j * bs:(j + 1) * bs])))
            if b is None:
                break
            hits.append(b)
            parent = b
        if need - len(hits) > len(self.free):
            raise NoBlocks("not enough free blocks")
        table = list(hits)
        for b in hits:
            self.refcount[b] += 1
        for j in range(len(hits), need):
            b = self.free.pop()
            self.refcount[b] = 1
            table.append(b)
            if (j + 1) * bs <= n:
                key = (table[j - 1] if j > 0 else -1, tuple(tokens[j * bs:(j + 1) * bs]))
                self.index[key] = b
                self.key_of[b] = key
        self.seqs[seq] = SeqState(table, n, slot)
        return list(table), len(hits) * bs

    def fork(self, parent: int, child: int):
        if parent not in self.seqs:
            raise UnknownSeq("unknown parent")
        if child in self.seqs:
            raise BadState("child already present")
        slot = self._lowest_free_slot()
        p = self.seqs[parent]
        for b in p.table:
            self.refcount[b] += 1
        self.seqs[child] = SeqState(list(p.table), p.num_tokens, slot)
        copies = []
        if p.num_tokens % self.block_size:
            copies.append((COPY_SLOT, p.slot, slot))
        return copies

    def append(self, seq: int, n: int):
        if n < 0:
            raise BadArg("n < 0")
        if seq not in self.seqs:
            raise UnknownSeq("unknown sequence")
        st = self.seqs[seq]
        bs = self.block_size
        cow = (n > 0 and st.num_tokens % bs != 0
               and self.refcount[st.table[-1]] > 1)
        boundaries = sum(1 for p in range(st.num_tokens, st.num_tokens + n)
                         if p % bs == 0)
        if int(cow) + boundaries > len(self.free):
            raise NoBlocks("not enough free blocks")
        copies = []
        if cow:
            src = st.table[-1]
            dst = self.free.pop()
            self.refcount[src] -= 1
            self.refcount[dst] = 1
            st.table[-1] = dst
            copies.append((COPY_BLOCK, src, dst))
        for p in range(st.num_tokens, st.num_tokens + n):
            if p % bs == 0:
                b = self.free.pop()
                self.refcount[b] = 1
                st.table.append(b)
        st.num_tokens += n
        return copies

    def release(self, seq: int):
        if seq not in self.seqs:
            raise UnknownSeq("unknown sequence")
        st = self.seqs.pop(seq)
        for b in st.table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
                if b in self.key_of:
                    del self.index[self.key_of.pop(b)]

    def table(self, seq: int):
        if seq not in self.seqs:
            raise UnknownSeq("unknown sequence")
        st = self.seqs[seq]
        return list(st.table), st.num_tokens, st.slot

    def stats(self):
        used = sum(1 for r in self.refcount if r > 0)
        shared = sum(1 for r in self.refcount if r > 1)
        return dict(total=self.num_blocks, free=len(self.free), used=used,
                    shared=shared, seqs=len(self.seqs), cached=len(self.index))

    def check_invariants(self):
        """Each block is either on the free stack or referenced; counts equal
        the number of table references; the stack has no duplicates; every
        table has ceil(tokens / bs) entries; slots are distinct."""
        refs = [0] * self.num_blocks
        for st in self.seqs.values():
            assert len(st.table) == self._blocks_for(st.num_tokens)
            for b in st.table:
                refs[b] += 1
        assert refs == self.refcount
        assert len(set(self.free)) == len(self.free)
        free = set(self.free)
        for b in range(self.num_blocks):
            assert (b in free) != (self.refcount[b] > 0)
        assert len(self.free) + sum(1 for r in refs if r > 0) == self.num_blocks
        slots = [st.slot for st in self.seqs.values()]
        assert len(set(slots)) == len(slots)
        assert all(0 <= s < self.max_seqs for s in slots)
        # indexed blocks are held, their parents too, and the maps agree
        assert len(self.index) == len(self.key_of)
        for key, b in self.index.items():
            assert self.key_of[b] == key and self.refcount[b] > 0
            assert key[0] == -1 or self.refcount[key[0]] > 0
            assert len(key[1]) == self.block_size

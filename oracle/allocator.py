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

Swap (deepinsea.top "Swap": when GPU memory runs short, KV-cache blocks are
moved to a CPU swap space sized in GB, at the price of host-device transfer
time; the page gives no policy):
* The swap space is a second pool of ``host_blocks`` blocks with the device
  blocks' layout, plus ``host_slots`` tail slots, with its own free stack
  (popped from its end, starting 0..H-1) and reference counts.
* A group of live, resident sequences is swapped out together (forked
  sequences share blocks; a shared block moves once).  A block moves only
  if every reference to it comes from the group: only then does moving it
  free device memory, so blocks also held outside the group stay where they
  are and the group keeps its references to them.  Moved blocks take host
  blocks in first-seen order (sequences in the given order, each table in
  order), keep the group's count on the host side, and go back on the device
  free stack in that order (leaving the prefix index).  Each sequence then
  gives up its device slot for the lowest free host slot; the rows of a
  partial last block are copied with it.
* Swapping a group in takes a fresh device block for every host block its
  tables name (first-seen order) with the group's count; host blocks whose
  count reaches zero go back on the host free stack.  A host block that
  sequences outside the group still hold stays for them (they get their own
  device copy when they come back).  Blocks that come back are not
  re-entered in the prefix index.  Each sequence takes the lowest free
  device slot.
* Both calls are all-or-nothing: slots are checked first, then blocks.  A
  swapped sequence may only be freed or swapped in: fork, append and the
  decode's batch tables refuse it.
* Tables of swapped sequences name host block h as -1 - h, and their slot
  is -1 - (host slot).
* Each call returns its copy plan: (kind, src, dst, rows) with kinds
  SWAP_BLOCK_OUT / SWAP_BLOCK_IN (one whole block: codes, scales, zero
  points) and SWAP_SLOT_OUT / SWAP_SLOT_IN (the first ``rows`` fp16 rows of
  each head of a tail slot, K and V; only for a partial last block).  Block
  entries come first, then slot entries, each in the order above.
"""

from dataclasses import dataclass, field

COPY_BLOCK = 0  # copy codes, scales and zero points of one physical block
COPY_SLOT = 1   # copy one fp16 tail slot

SWAP_BLOCK_OUT = 0  # device block -> host block
SWAP_BLOCK_IN = 1   # host block -> device block
SWAP_SLOT_OUT = 2   # device tail slot -> host slot (first `rows` rows)
SWAP_SLOT_IN = 3    # host slot -> device tail slot


def host_id(h):
    """Table entry (or slot) naming host block (or host slot) h."""
    return -1 - h


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
    swapped: bool = False


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
    host_blocks: int = field(init=False, default=0)
    host_slots: int = field(init=False, default=0)
    host_free: list = field(init=False)
    host_refcount: list = field(init=False)

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
        self.host_free = []
        self.host_refcount = []

    # -- helpers ---------------------------------------------------------
    def _lowest_free_slot(self):
        used = {s.slot for s in self.seqs.values() if not s.swapped}
        for k in range(self.max_seqs):
            if k not in used:
                return k
        raise NoSlots("no free tail slot")

    def _free_host_slots(self):
        used = {host_id(s.slot) for s in self.seqs.values() if s.swapped}
        return [k for k in range(self.host_slots) if k not in used]

    def _resident(self, seq):
        if self.seqs[seq].swapped:
            raise BadState("sequence is swapped out")
        return self.seqs[seq]

    def _group(self, seqs):
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise BadArg("a sequence is named twice")
        for s in seqs:
            if s not in self.seqs:
                raise UnknownSeq("unknown sequence")
        return seqs

    def _release_block(self, b, n=1):
        """Drop n references to device block b; at zero it goes back on the
        free stack and leaves the prefix index."""
        self.refcount[b] -= n
        if self.refcount[b] == 0:
            self.free.append(b)
            if b in self.key_of:
                del self.index[self.key_of.pop(b)]

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
        p = self._resident(parent)
        slot = self._lowest_free_slot()
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
        st = self._resident(seq)
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
            if b >= 0:
                self._release_block(b)
            else:
                h = host_id(b)
                self.host_refcount[h] -= 1
                if self.host_refcount[h] == 0:
                    self.host_free.append(h)

    # -- swap ------------------------------------------------------------
    def set_swap_space(self, host_blocks: int, host_slots: int):
        if host_blocks < 0 or host_slots < 0:
            raise BadArg("swap space sizes must be >= 0")
        if any(s.swapped for s in self.seqs.values()):
            raise BadState("sequences are swapped out")
        self.host_blocks, self.host_slots = host_blocks, host_slots
        self.host_free = list(range(host_blocks))
        self.host_refcount = [0] * host_blocks

    def swap_out(self, seqs):
        """Move the blocks only this group holds, and the group's tail slots,
        to the swap space; returns the copy plan."""
        seqs = self._group(seqs)
        for s in seqs:
            self._resident(s)
        count, order = {}, []
        for s in seqs:
            for b in self.seqs[s].table:
                if b not in count:
                    order.append(b)
                count[b] = count.get(b, 0) + 1
        moving = [b for b in order if count[b] == self.refcount[b]]
        if len(self._free_host_slots()) < len(seqs):
            raise NoSlots("no free host slot")
        if len(moving) > len(self.host_free):
            raise NoBlocks("not enough free host blocks")
        plan, where = [], {}
        for b in moving:
            h = self.host_free.pop()
            self.host_refcount[h] = count[b]
            self._release_block(b, count[b])
            where[b] = h
            plan.append((SWAP_BLOCK_OUT, b, h, 0))
        for s in seqs:
            st = self.seqs[s]
            hs = self._free_host_slots()[0]
            rows = st.num_tokens % self.block_size
            if rows:
                plan.append((SWAP_SLOT_OUT, st.slot, hs, rows))
            st.table = [host_id(where[b]) if b in where else b for b in st.table]
            st.slot = host_id(hs)
            st.swapped = True
        return plan

    def swap_in(self, seqs):
        """Bring a swapped group back into fresh device blocks and slots;
        returns the copy plan."""
        seqs = self._group(seqs)
        for s in seqs:
            if not self.seqs[s].swapped:
                raise BadState("sequence is not swapped out")
        count, order = {}, []
        for s in seqs:
            for b in self.seqs[s].table:
                if b < 0:
                    if b not in count:
                        order.append(b)
                    count[b] = count.get(b, 0) + 1
        used = {s.slot for s in self.seqs.values() if not s.swapped}
        if self.max_seqs - len(used) < len(seqs):
            raise NoSlots("no free tail slot")
        if len(order) > len(self.free):
            raise NoBlocks("not enough free blocks")
        plan, where = [], {}
        for e in order:
            h = host_id(e)
            d = self.free.pop()
            self.refcount[d] = count[e]
            self.host_refcount[h] -= count[e]
            if self.host_refcount[h] == 0:
                self.host_free.append(h)
            where[e] = d
            plan.append((SWAP_BLOCK_IN, h, d, 0))
        for s in seqs:
            st = self.seqs[s]
            hs = host_id(st.slot)
            slot = self._lowest_free_slot()
            st.swapped = False
            rows = st.num_tokens % self.block_size
            if rows:
                plan.append((SWAP_SLOT_IN, hs, slot, rows))
            st.table = [where[b] if b < 0 else b for b in st.table]
            st.slot = slot
        return plan

    def table(self, seq: int):
        if seq not in self.seqs:
            raise UnknownSeq("unknown sequence")
        st = self.seqs[seq]
        return list(st.table), st.num_tokens, st.slot

    def stats(self):
        used = sum(1 for r in self.refcount if r > 0)
        shared = sum(1 for r in self.refcount if r > 1)
        return dict(total=self.num_blocks, free=len(self.free), used=used,
                    shared=shared, seqs=len(self.seqs), cached=len(self.index),
                    host_total=self.host_blocks, host_free=len(self.host_free),
                    swapped=sum(1 for s in self.seqs.values() if s.swapped))

    def check_invariants(self):
        """Each block is either on the free stack or referenced; counts equal
        the number of table references; the stack has no duplicates; every
        table has ceil(tokens / bs) entries; slots are distinct."""
        refs = [0] * self.num_blocks
        host_refs = [0] * self.host_blocks
        for st in self.seqs.values():
            assert len(st.table) == self._blocks_for(st.num_tokens)
            for b in st.table:
                assert b >= 0 or st.swapped
                if b >= 0:
                    refs[b] += 1
                else:
                    host_refs[host_id(b)] += 1
        assert refs == self.refcount
        assert host_refs == self.host_refcount
        assert len(set(self.host_free)) == len(self.host_free)
        hfree = set(self.host_free)
        for h in range(self.host_blocks):
            assert (h in hfree) != (self.host_refcount[h] > 0)
        assert len(set(self.free)) == len(self.free)
        free = set(self.free)
        for b in range(self.num_blocks):
            assert (b in free) != (self.refcount[b] > 0)
        assert len(self.free) + sum(1 for r in refs if r > 0) == self.num_blocks
        slots = [st.slot for st in self.seqs.values() if not st.swapped]
        assert len(set(slots)) == len(slots)
        assert all(0 <= s < self.max_seqs for s in slots)
        hslots = [host_id(st.slot) for st in self.seqs.values() if st.swapped]
        assert len(set(hslots)) == len(hslots)
        assert all(0 <= s < self.host_slots for s in hslots)
        # indexed blocks are held, their parents too, and the maps agree
        assert len(self.index) == len(self.key_of)
        for key, b in self.index.items():
            assert self.key_of[b] == key and self.refcount[b] > 0
            assert key[0] == -1 or self.refcount[key[0]] > 0
            assert len(key[1]) == self.block_size

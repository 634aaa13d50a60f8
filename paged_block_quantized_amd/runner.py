"""Sets up a decode workload through libpbq and runs decode steps.

Orchestration of library calls only (allocate, fork, store, build tables,
decode); every step of the computation happens in the HIP kernels.

A decode step for one layer stores the current token of every sequence
(re-quantizing its block from the tail slot) and runs the fused dequantizing
attention over the whole context, current token included: one call of
paged_attn_decode_append, or (step_separate) kv_quantize_store followed by
paged_attn_decode.  Sequences forked from one prefix use
paged_attn_decode_shared_prefix, which reads the shared blocks once.
"""

from dataclasses import dataclass

import numpy as np
import torch

from . import workloads as W
from .pool import KVPool


def code_bits(w: W.Workload):
    """(K bits, V bits, metadata bytes per (block, head)) of the workload's
    codecs: two fp16 scales, plus a u8 zero point for each asymmetric codec."""
    kc = W.k_codec_of(w)
    kbits = 4 if kc == "i4" else 8
    vbits = 4 if w.v_codec == "i4" else 8
    meta = 2 + 2 + (1 if w.v_codec in ("i4", "i8a") else 0) + (1 if kc == "i4" else 0)
    return kbits, vbits, meta


def blocks_needed(w: W.Workload, ctx: np.ndarray) -> int:
    bs = w.block_size
    per_seq = (ctx + bs - 1) // bs
    if w.prefix:
        assert w.prefix % bs == 0, "shared prefix must end on a block boundary"
        return int(w.prefix // bs + np.sum(per_seq - w.prefix // bs))
    return int(np.sum(per_seq))


@dataclass
class DecodeSetup:
    w: W.Workload
    pool: KVPool
    ctx: np.ndarray
    tables: torch.Tensor        # int32 [S, max_blocks] on the device
    ctx_dev: torch.Tensor       # int32 [S]
    slots: torch.Tensor         # int32 [S]
    start_pos: torch.Tensor     # int32 [S] = ctx - 1
    cu_step: torch.Tensor       # int32 [S+1] = 0..S
    k_new: torch.Tensor         # fp16 [S, Hkv, D]: the current token
    v_new: torch.Tensor
    q: torch.Tensor             # fp16 [S, Hq, D]
    out: torch.Tensor           # fp16 [S, Hq, D]
    workspace: torch.Tensor
    max_ctx: int
    sm_scale: float
    partition: int
    replicas: list = None       # [(kv_pool_mem, arrays)] copies of the pool
    shared: int = 0             # tokens of the prefix all sequences share (read once), 0: none
    order: np.ndarray = None    # batch index b holds the workload's sequence order[b]

    def add_replicas(self, n):
        """n more copies of the pool arrays at other addresses (each the same
        cache contents), so that consecutive steps can read memory that no
        earlier step has left in a cache, as the layers of a model would."""
        self.replicas = (self.replicas or []) + [self.pool.replica() for _ in range(n)]

    def _mem(self, r):
        return None if not r else self.replicas[r - 1][0]

    def store_current(self, stream=None, r=0):
        self.pool.quantize_store(self.k_new, self.v_new, self.cu_step, self.start_pos,
                                 self.tables, self.slots, 1, stream, mem=self._mem(r))

    def attend(self, stream=None, r=0):
        self.pool.decode(self.q, self.out, self.tables, self.ctx_dev, self.max_ctx,
                         self.sm_scale, self.partition, self.workspace, stream, mem=self._mem(r))

    def step_separate(self, stream=None, r=0):
        """The step as two calls: kv_quantize_store, then paged_attn_decode."""
        self.store_current(stream, r)
        self.attend(stream, r)

    def step(self, stream=None, r=0):
        """The step as one call: paged_attn_decode_append (store fused in), or
        paged_attn_decode_shared_prefix when the sequences share a prefix."""
        if self.shared:
            self.pool.decode_shared_prefix(self.q, self.out, self.tables, self.ctx_dev, self.max_ctx,
                                           self.sm_scale, self.partition, self.shared, self.k_new,
                                           self.v_new, self.slots, self.workspace, stream,
                                           mem=self._mem(r))
        else:
            self.step_unshared(stream, r)

    def step_unshared(self, stream=None, r=0):
        """paged_attn_decode_append, which reads a shared prefix per sequence."""
        self.pool.decode_append(self.k_new, self.v_new, self.slots, self.q, self.out, self.tables,
                                self.ctx_dev, self.max_ctx, self.sm_scale, self.partition,
                                self.workspace, stream, mem=self._mem(r))


def _store(pool, k, v, seq_ids, starts, device):
    """Store rows k/v [T, Hkv, D] (device fp16) for several sequences:
    sequence seq_ids[i] receives the i-th run of rows at position starts[i]."""
    lens = [int(x.shape[0]) for x in k]
    kk = torch.cat(k).contiguous()
    vv = torch.cat(v).contiguous()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=device)
    st = torch.tensor(starts, dtype=torch.int32, device=device)
    max_blocks = max(len(pool.table(s)[0]) for s in seq_ids)
    tables, _, slots = pool.batch_tables(seq_ids, max_blocks)
    pool.quantize_store(kk, vv, cu, st, tables.to(device), slots.to(device), max(lens))


def setup_decode(w: W.Workload, device="cuda", chunk_seqs=8, partition=None, order=None) -> DecodeSetup:
    """Build the pool for workload ``w`` holding ctx-1 tokens per sequence,
    reserve the current token's position, and allocate the step's tensors.
    The batch is laid out in ``order`` (workload sequence ids; by default
    the workload's own order -- the library balances ragged batches over the
    GPU itself): batch index b is sequence order[b]."""
    ctx_w = W.context_lengths(w)
    order = np.arange(len(ctx_w)) if order is None else np.asarray(order)
    ctx = ctx_w[order]
    S, bs = w.num_seqs, w.block_size
    N = w.pool_blocks or blocks_needed(w, ctx)
    pool = KVPool(N, bs, w.num_kv_heads, w.head_dim, w.v_codec, k_codec=W.k_codec_of(w), max_seqs=S + 1,
                  free_order=W.free_order(w, N), device=device)
    if w.prefix:
        parent = S
        pool.alloc(parent, w.prefix)
        kp, vp = W.kv_tokens(w, "prefix", w.prefix, device)
        _store(pool, [kp], [vp], [parent], [0], device)
        for s in range(S):
            copies = pool.fork(parent, s)
            assert copies == [], "aligned prefix: no tail copy"
        pool.release(parent)
    for c0 in range(0, S, chunk_seqs):
        ids = list(range(c0, min(S, c0 + chunk_seqs)))
        ks, vs, starts = [], [], []
        for s in ids:
            n_hist = int(ctx[s]) - 1 - w.prefix
            if w.prefix:
                copies = pool.append(s, n_hist)
                assert copies == []
            else:
                pool.alloc(s, n_hist)
            k, v = W.kv_tokens(w, int(order[s]), int(ctx[s]) - w.prefix, device)
            ks.append(k[:n_hist])
            vs.append(v[:n_hist])
            starts.append(w.prefix)
        if any(x.shape[0] for x in ks):
            _store(pool, ks, vs, ids, starts, device)
    # reserve the current token; copies (COW) would precede its store
    k_new, v_new = [], []
    for s in range(S):
        copies = pool.append(s, 1)
        if copies:
            pool.copy_blocks(copies)
        k, v = W.kv_tokens(w, int(order[s]), int(ctx[s]) - w.prefix, device)
        k_new.append(k[-1:])
        v_new.append(v[-1:])
    max_blocks = int(np.max((ctx + bs - 1) // bs))
    tables, ctx_h, slots = pool.batch_tables(list(range(S)), max_blocks)
    assert np.array_equal(ctx_h.numpy(), ctx)
    part = w.partition if partition is None else partition
    max_ctx = int(ctx.max())
    if not part:
        part = pool.default_partition(S, w.num_q_heads, max_ctx)
    q = W.queries(w, device)[torch.as_tensor(order, device=device)].contiguous()
    out = torch.empty_like(q)
    ws_bytes = pool.workspace_bytes(S, w.num_q_heads, max_ctx, part)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    return DecodeSetup(
        w=w, pool=pool, ctx=ctx, tables=tables.to(device), ctx_dev=ctx_h.to(device),
        slots=slots.to(device),
        start_pos=torch.tensor(ctx - 1, dtype=torch.int32, device=device),
        cu_step=torch.arange(S + 1, dtype=torch.int32, device=device),
        k_new=torch.cat(k_new).contiguous(), v_new=torch.cat(v_new).contiguous(),
        q=q, out=out, workspace=workspace, max_ctx=max_ctx,
        sm_scale=1.0 / float(np.sqrt(w.head_dim)), partition=part,
        shared=shared_prefix_tokens(w, part), order=order)


def shared_prefix_tokens(w: W.Workload, partition: int) -> int:
    """Tokens of the workload's shared prefix that the shared-prefix decode
    reads once: whole partitions of it (0 when it has none)."""
    if not w.prefix or partition % 32:
        return 0
    return (w.prefix // partition) * partition


def sequence_history(setup: DecodeSetup, s: int, device="cuda"):
    """fp16 K/V of every token of sequence s (host numpy [ctx, Hkv, D]),
    regenerated from the seeded streams."""
    w = setup.w
    k, v = W.kv_tokens(w, int(setup.order[s]), int(setup.ctx[s]) - w.prefix, device)
    if w.prefix:
        kp, vp = W.kv_tokens(w, "prefix", w.prefix, device)
        k, v = torch.cat([kp, k]), torch.cat([vp, v])
    return k.cpu().numpy(), v.cpu().numpy()


def decode_bytes(w: W.Workload, ctx: np.ndarray) -> int:
    """Algorithmic HBM bytes of one decode attention pass: the codes of every
    valid token, the metadata of every block read, Q, O, the block tables and
    the context lengths; a shared prefix counted once."""
    S, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    kbits, vbits, meta = code_bits(w)
    tokens = int(np.sum(ctx))
    blocks = int(np.sum((ctx + bs - 1) // bs))
    if w.prefix:
        tokens -= (S - 1) * w.prefix
        blocks -= (S - 1) * (w.prefix // bs)
    codes = tokens * Hkv * D * (kbits + vbits) // 8
    meta_b = blocks * Hkv * meta
    qo = 2 * S * Hq * D * 2
    tables = int(np.sum((ctx + bs - 1) // bs)) * 4 + S * 4
    return codes + meta_b + qo + tables


def store_step_bytes(w: W.Workload, ctx: np.ndarray, rewrite_tiles: bool = True) -> int:
    """Algorithmic bytes of storing the current token: the block's exact rows
    read (tail slot + new row, fp16 K and V), its codes and metadata written,
    and the per-sequence index arrays.

    rewrite_tiles False: the block's scale (and zero point) is already what
    the store computes -- as when the same token is stored again -- so the
    earlier rows' codes are unchanged and only the token's own codes are
    written (its K row and its entry of every V dim row), with the block's
    metadata read instead of written."""
    Hkv, D, bs = w.num_kv_heads, w.head_dim, w.block_size
    kbits, vbits, meta = code_bits(w)
    rows = (ctx - 1) % bs + 1                    # rows the block holds after the store
    read = int(np.sum(rows)) * Hkv * D * 2 * 2
    if rewrite_tiles:
        write = len(ctx) * Hkv * (bs * D * (kbits + vbits) // 8 + meta)
    else:
        write = len(ctx) * Hkv * (D * (kbits + vbits) // 8 + meta)   # metadata read, not written
    tail_write = int(np.sum(rows < bs)) * Hkv * D * 2 * 2
    return read + write + tail_write + len(ctx) * 4 * 4


@dataclass
class MultiSetup:
    """A multi-query workload: every token stored, the last q_len of each
    sequence as queries."""
    w: W.Workload
    pool: KVPool
    ctx: np.ndarray
    tables: torch.Tensor
    ctx_dev: torch.Tensor
    cu: torch.Tensor            # int32 [S+1]
    q: torch.Tensor             # fp16 [S * q_len, Hq, D]
    out: torch.Tensor
    workspace: torch.Tensor
    max_ctx: int
    sm_scale: float
    partition: int

    def run(self, stream=None):
        self.pool.multi_query(self.q, self.out, self.cu, self.w.q_len, self.tables, self.ctx_dev,
                              self.max_ctx, self.sm_scale, self.partition, self.workspace, stream)


def setup_multi(w: W.Workload, device="cuda", chunk_seqs=8, partition=0) -> MultiSetup:
    """Build the pool for multi-query workload ``w`` with all its tokens
    stored (the queries' own K/V included) and allocate the call's tensors."""
    from . import _lib as L
    ctx = W.context_lengths(w)
    S, bs = w.num_seqs, w.block_size
    N = blocks_needed(w, ctx)
    pool = KVPool(N, bs, w.num_kv_heads, w.head_dim, w.v_codec, k_codec=W.k_codec_of(w), max_seqs=S,
                  free_order=W.free_order(w, N), device=device)
    for c0 in range(0, S, chunk_seqs):
        ids = list(range(c0, min(S, c0 + chunk_seqs)))
        ks, vs = [], []
        for s in ids:
            pool.alloc(s, int(ctx[s]))
            k, v = W.kv_tokens(w, s, int(ctx[s]), device)
            ks.append(k)
            vs.append(v)
        _store(pool, ks, vs, ids, [0] * len(ids), device)
    max_blocks = int(np.max((ctx + bs - 1) // bs))
    tables, ctx_h, _ = pool.batch_tables(list(range(S)), max_blocks)
    q = W.multi_queries(w, device)
    cu = torch.arange(0, S + 1, dtype=torch.int32, device=device) * w.q_len
    max_ctx = int(ctx.max())
    ws = L.paged_attn_multi_query_workspace_bytes(pool.desc, S, S * w.q_len, w.num_q_heads, w.q_len,
                                                  max_ctx, partition)
    torch.cuda.synchronize()
    return MultiSetup(w=w, pool=pool, ctx=ctx, tables=tables.to(device), ctx_dev=ctx_h.to(device), cu=cu,
                      q=q, out=torch.empty_like(q), workspace=torch.empty(max(ws, 16), dtype=torch.uint8,
                                                                          device=device),
                      max_ctx=max_ctx, sm_scale=1.0 / float(np.sqrt(w.head_dim)), partition=partition)


def multi_flops(w: W.Workload, ctx: np.ndarray) -> int:
    """Algorithmic flops of one multi-query pass: per query token, query head
    and visible token, a D-long dot product and a D-long weighted sum (2 D
    multiply-adds)."""
    n = w.q_len
    vis = int(np.sum(ctx - n)) * n + len(ctx) * n * (n + 1) // 2   # sum over queries of pos + 1
    return 4 * w.head_dim * w.num_q_heads * vis


def multi_bytes(w: W.Workload, ctx: np.ndarray) -> int:
    """Algorithmic HBM bytes of one multi-query pass: every stored token's
    codes and block metadata once, the query and output rows, the tables."""
    S, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    kbits, vbits, meta = code_bits(w)
    blocks = int(np.sum((ctx + bs - 1) // bs))
    return (int(np.sum(ctx)) * Hkv * D * (kbits + vbits) // 8 + blocks * Hkv * meta
            + 2 * S * w.q_len * Hq * D * 2 + blocks * 4 + (2 * S + 1) * 4)


@dataclass
class StoreSetup:
    """A quantize-and-store workload: every sequence's prompt (fp16 K/V in
    HBM) stored in one call into blocks the allocator took from a pool in
    seeded random order."""
    w: W.Workload
    pool: KVPool
    k: torch.Tensor             # fp16 [S * T, Hkv, D]
    v: torch.Tensor
    cu: torch.Tensor            # int32 [S+1]
    start: torch.Tensor         # int32 [S] (zeros)
    tables: torch.Tensor
    slots: torch.Tensor
    tokens: int                 # tokens per prompt

    def run(self, stream=None):
        self.pool.quantize_store(self.k, self.v, self.cu, self.start, self.tables, self.slots, self.tokens,
                                 stream)


def setup_prefill_store(w: W.Workload, device="cuda") -> StoreSetup:
    """The pool and inputs of a store-only workload (all prompts allocated,
    nothing stored yet)."""
    S, T, bs = w.num_seqs, w.ctx[0], w.block_size
    N = w.pool_blocks or S * ((T + bs - 1) // bs)
    pool = KVPool(N, bs, w.num_kv_heads, w.head_dim, w.v_codec, k_codec=W.k_codec_of(w), max_seqs=S,
                  free_order=W.free_order(w, N), device=device)
    for s in range(S):
        pool.alloc(s, T)
    tables, _, slots = pool.batch_tables(list(range(S)), (T + bs - 1) // bs)
    ks, vs = zip(*[W.kv_tokens(w, s, T, device) for s in range(S)])
    k, v = torch.cat(ks), torch.cat(vs)
    del ks, vs
    cu = torch.arange(0, (S + 1) * T, T, dtype=torch.int32, device=device)
    torch.cuda.synchronize()
    return StoreSetup(w=w, pool=pool, k=k, v=v, cu=cu, start=torch.zeros(S, dtype=torch.int32, device=device),
                      tables=tables.to(device), slots=slots.to(device), tokens=T)


def prefill_store_bytes(w: W.Workload) -> int:
    """Algorithmic HBM bytes of storing every prompt of a store-only
    workload: the fp16 K and V rows read, the codes and per-(block, head)
    metadata written, the block tables read."""
    S, T, Hkv, D, bs = w.num_seqs, w.ctx[0], w.num_kv_heads, w.head_dim, w.block_size
    kbits, vbits, meta = code_bits(w)
    tok = S * T
    blocks = S * ((T + bs - 1) // bs)
    return tok * Hkv * D * 2 * 2 + tok * Hkv * D * (kbits + vbits) // 8 + blocks * Hkv * meta + blocks * 4


@dataclass
class AppendSetup:
    """One-token appends to sequences whose last block is partly filled: each
    step reserves a position per sequence on the host and stores the new
    token, re-quantizing its block from the tail slot's exact rows."""
    pool: KVPool
    hist: list                  # per sequence (K, V) fp16 [fill + steps, Hkv, D] on the device
    fill: np.ndarray            # rows stored before the first step

    def inputs(self, step, device="cuda"):
        """Reserve step `step`'s positions and return the call's arguments."""
        S = len(self.fill)
        for s in range(S):
            assert self.pool.append(s, 1) == []
        tables, _, slots = self.pool.batch_tables(list(range(S)), 2)
        kn = torch.cat([h[0][f + step:f + step + 1] for h, f in zip(self.hist, self.fill)])
        vn = torch.cat([h[1][f + step:f + step + 1] for h, f in zip(self.hist, self.fill)])
        cu = torch.arange(S + 1, dtype=torch.int32, device=device)
        st = torch.tensor(self.fill + step, dtype=torch.int32, device=device)
        return kn, vn, cu, st, tables.to(device), slots.to(device)


def setup_append(w: W.Workload, steps: int = 16, device="cuda") -> AppendSetup:
    """The store workload's sequences restarted with 1..bs-1 stored rows each
    (seeded), ready for `steps` one-token appends that carry every block
    through its fill point."""
    S, bs = w.num_seqs, w.block_size
    rng = np.random.default_rng([w.seed, 7])
    fill = rng.integers(1, bs, S)
    pool = KVPool(w.pool_blocks or S * 2, bs, w.num_kv_heads, w.head_dim, w.v_codec, k_codec=W.k_codec_of(w), max_seqs=S,
                  free_order=W.free_order(w, w.pool_blocks or S * 2), device=device)
    for s in range(S):
        pool.alloc(s, int(fill[s]))
    hist = [W.kv_tokens(w, 100 + s, int(fill[s]) + steps, device) for s in range(S)]
    tables, _, slots = pool.batch_tables(list(range(S)), 2)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(fill)]), dtype=torch.int32, device=device)
    pool.quantize_store(torch.cat([h[0][:f] for h, f in zip(hist, fill)]),
                        torch.cat([h[1][:f] for h, f in zip(hist, fill)]),
                        cu, torch.zeros(S, dtype=torch.int32, device=device),
                        tables.to(device), slots.to(device), int(fill.max()))
    torch.cuda.synchronize()
    return AppendSetup(pool=pool, hist=hist, fill=fill)

"""ctypes binding of libpbq.so (include/pbq.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
computation of its own.  Device arguments are torch CUDA tensors (their
data_ptr() is passed); the stream is torch's current stream unless one is
given.  A failing call raises ``PBQError`` with the library's message.
"""

import ctypes
import os

import torch  # loads the HIP runtime the library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
# PBQ_LIB_PATH selects another build of the library (the sanitizer test's)
LIB_PATH = os.environ.get("PBQ_LIB_PATH") or os.path.join(_HERE, "libpbq.so")

KV_OK, KV_ERR_INVALID, KV_ERR_NO_BLOCKS, KV_ERR_UNKNOWN_SEQ, KV_ERR_STATE, \
    KV_ERR_NO_SLOTS, KV_ERR_HIP = range(7)
STATUS_NAMES = {KV_OK: "ok", KV_ERR_INVALID: "invalid", KV_ERR_NO_BLOCKS: "no_blocks",
                KV_ERR_UNKNOWN_SEQ: "unknown_seq", KV_ERR_STATE: "state",
                KV_ERR_NO_SLOTS: "no_slots", KV_ERR_HIP: "hip"}
KV_CODEC_I8_SYM, KV_CODEC_I4_ASYM, KV_CODEC_FP8_E4M3, KV_CODEC_I8_ASYM = 0, 1, 2, 3
KV_COPY_BLOCK, KV_COPY_SLOT = 0, 1
KV_SWAP_BLOCK_OUT, KV_SWAP_BLOCK_IN, KV_SWAP_SLOT_OUT, KV_SWAP_SLOT_IN = range(4)


class PBQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status
        self.kind = STATUS_NAMES.get(status, "invalid")


class kv_pool_desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_codec", ctypes.c_int32), ("v_codec", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32)]


POOL_ARRAYS = ("k_codes", "v_codes", "k_scale", "v_scale", "v_zp", "tail_k", "tail_v", "k_zp")


class kv_pool_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in POOL_ARRAYS]


class kv_pool_mem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in POOL_ARRAYS]


class kv_copy(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("src", ctypes.c_int32), ("dst", ctypes.c_int32)]


class kv_swap(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("src", ctypes.c_int32), ("dst", ctypes.c_int32),
                ("rows", ctypes.c_int32)]


class kv_pool_stats_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("total", "free", "used", "shared", "seqs", "cached",
                                              "host_total", "host_free", "swapped")]


EXPORTS = [
    "kv_pool_bytes", "kv_pool_create", "kv_pool_destroy", "kv_seq_alloc", "kv_seq_alloc_prefix",
    "kv_seq_fork", "kv_seq_append", "kv_seq_free", "kv_seq_table",
    "kv_batch_tables", "kv_pool_stats", "kv_pool_free_list", "kv_pool_set_swap_space",
    "kv_seq_swap_out", "kv_seq_swap_in", "kv_swap_blocks", "kv_copy_blocks",
    "kv_quantize_store", "paged_attn_workspace_bytes", "paged_attn_decode",
    "paged_attn_decode_append", "paged_attn_decode_append_noalloc", "paged_attn_decode_shared_prefix", "paged_attn_multi_query",
    "paged_attn_multi_query_workspace_bytes",
    "paged_attn_default_partition", "kv_stream_read_sink_words", "kv_stream_read_tiles", "kv_last_error",
    "kv_set_debug_checks",
]

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_block_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, VP = (ctypes.POINTER, ctypes.c_int32, ctypes.c_int64,
                               ctypes.c_size_t, ctypes.c_void_p)
        st = ctypes.c_int
        sig = {
            "kv_pool_bytes": (st, [P(kv_pool_desc), P(kv_pool_sizes)]),
            "kv_pool_create": (st, [P(kv_pool_desc), P(I32), P(VP)]),
            "kv_pool_destroy": (None, [VP]),
            "kv_seq_alloc": (st, [VP, I64, I32]),
            "kv_seq_alloc_prefix": (st, [VP, I64, P(I32), I32, P(I32)]),
            "kv_seq_fork": (st, [VP, I64, I64, P(kv_copy), I32, P(I32)]),
            "kv_seq_append": (st, [VP, I64, I32, P(kv_copy), I32, P(I32)]),
            "kv_seq_free": (st, [VP, I64]),
            "kv_seq_table": (st, [VP, I64, P(I32), I32, P(I32), P(I32), P(I32)]),
            "kv_batch_tables": (st, [VP, P(I64), I32, P(I32), I32, P(I32), P(I32)]),
            "kv_pool_stats": (st, [VP, P(kv_pool_stats_t)]),
            "kv_pool_free_list": (st, [VP, P(I32), I32, P(I32)]),
            "kv_pool_set_swap_space": (st, [VP, I32, I32]),
            "kv_seq_swap_out": (st, [VP, P(I64), I32, P(kv_swap), I32, P(I32)]),
            "kv_seq_swap_in": (st, [VP, P(I64), I32, P(kv_swap), I32, P(I32)]),
            "kv_swap_blocks": (st, [P(kv_pool_desc), P(kv_pool_mem), P(kv_pool_desc),
                                    P(kv_pool_mem), VP, I32, VP]),
            "kv_copy_blocks": (st, [P(kv_pool_desc), P(kv_pool_mem), VP, I32, VP]),
            "kv_quantize_store": (st, [P(kv_pool_desc), P(kv_pool_mem), VP, VP, I32, VP, VP,
                                       VP, I32, VP, I32, VP]),
            "paged_attn_workspace_bytes": (SZ, [P(kv_pool_desc), I32, I32, I32, I32]),
            "paged_attn_decode": (st, [P(kv_pool_desc), P(kv_pool_mem), VP, VP, I32, I32, VP,
                                       I32, VP, I32, ctypes.c_float, I32, VP, SZ, VP]),
            "paged_attn_decode_append": (st, [P(kv_pool_desc), P(kv_pool_mem), VP, VP, VP, VP, VP,
                                              I32, I32, VP, I32, VP, I32, ctypes.c_float, I32, VP,
                                              SZ, VP]),
            "paged_attn_decode_append_noalloc": (st, [P(kv_pool_desc), P(kv_pool_mem), VP, VP, VP, VP, VP,
                                                      I32, I32, VP, I32, VP, I32, ctypes.c_float, I32, VP]),
            "paged_attn_decode_shared_prefix": (st, [P(kv_pool_desc), P(kv_pool_mem), VP, VP, VP, VP,
                                                     VP, I32, I32, VP, I32, VP, I32, ctypes.c_float,
                                                     I32, I32, VP, SZ, VP]),
            "paged_attn_multi_query": (st, [P(kv_pool_desc), P(kv_pool_mem), VP, VP, I32, I32, VP, I32, I32,
                                            VP, I32, VP, I32, ctypes.c_float, I32, VP, SZ, VP]),
            "paged_attn_multi_query_workspace_bytes": (SZ, [P(kv_pool_desc), I32, I32, I32, I32, I32, I32]),
            "paged_attn_default_partition": (I32, [P(kv_pool_desc), I32, I32, I32]),
            "kv_stream_read_sink_words": (SZ, [I64]),
            "kv_stream_read_tiles": (st, [VP, I64, I32, VP, I64, VP, SZ, VP]),
            "kv_last_error": (ctypes.c_char_p, []),
            "kv_set_debug_checks": (I32, [I32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != KV_OK:
        raise PBQError(status, lib().kv_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _i32_array(values):
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr


# ---- entry points ---------------------------------------------------------

def make_desc(num_blocks, block_size, num_kv_heads, head_dim, v_codec=KV_CODEC_I8_SYM,
              max_seqs=1, k_codec=KV_CODEC_I8_SYM):
    return kv_pool_desc(num_blocks, block_size, num_kv_heads, head_dim, k_codec, v_codec,
                        max_seqs)


def kv_pool_bytes(desc):
    out = kv_pool_sizes()
    _check(lib().kv_pool_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in kv_pool_sizes._fields_}


def kv_pool_create(desc, free_order=None):
    handle = ctypes.c_void_p()
    fo = None if free_order is None else _i32_array(list(free_order))
    _check(lib().kv_pool_create(ctypes.byref(desc), fo, ctypes.byref(handle)))
    return handle


def kv_pool_destroy(handle):
    lib().kv_pool_destroy(handle)


def kv_seq_alloc(handle, seq, num_tokens):
    _check(lib().kv_seq_alloc(handle, int(seq), int(num_tokens)))


def kv_seq_alloc_prefix(handle, seq, token_ids):
    """Returns the number of leading tokens already held by shared blocks."""
    import numpy as np
    ids = np.ascontiguousarray(token_ids, dtype=np.int32)
    cached = ctypes.c_int32()
    ptr = ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if ids.size else None
    _check(lib().kv_seq_alloc_prefix(handle, int(seq), ptr, int(ids.size), ctypes.byref(cached)))
    return cached.value


def _copies_out(fn, *args):
    buf = (kv_copy * 4)()
    n = ctypes.c_int32()
    _check(fn(*args, buf, 4, ctypes.byref(n)))
    return [(buf[i].kind, buf[i].src, buf[i].dst) for i in range(n.value)]


def kv_seq_fork(handle, parent, child):
    return _copies_out(lib().kv_seq_fork, handle, int(parent), int(child))


def kv_seq_append(handle, seq, n_tokens):
    return _copies_out(lib().kv_seq_append, handle, int(seq), int(n_tokens))


def kv_seq_free(handle, seq):
    _check(lib().kv_seq_free(handle, int(seq)))


def kv_seq_table(handle, seq):
    nb, nt, slot = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().kv_seq_table(handle, int(seq), None, 0, ctypes.byref(nb), ctypes.byref(nt),
                              ctypes.byref(slot)))
    out = (ctypes.c_int32 * max(1, nb.value))()
    _check(lib().kv_seq_table(handle, int(seq), out, nb.value, None, None, None))
    return list(out)[:nb.value], nt.value, slot.value


def kv_batch_tables(handle, seqs, max_blocks):
    """Returns (tables int32 [n, max_blocks], ctx_lens [n], slots [n]) as
    CPU torch tensors."""
    n = len(seqs)
    sq = (ctypes.c_int64 * max(1, n))(*[int(s) for s in seqs])
    tables = torch.zeros((n, max_blocks), dtype=torch.int32)
    ctx = torch.zeros(n, dtype=torch.int32)
    slots = torch.zeros(n, dtype=torch.int32)
    I32P = ctypes.POINTER(ctypes.c_int32)
    _check(lib().kv_batch_tables(handle, sq, n,
                                 ctypes.cast(tables.data_ptr(), I32P), int(max_blocks),
                                 ctypes.cast(ctx.data_ptr(), I32P),
                                 ctypes.cast(slots.data_ptr(), I32P)))
    return tables, ctx, slots


def kv_pool_stats(handle):
    out = kv_pool_stats_t()
    _check(lib().kv_pool_stats(handle, ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in kv_pool_stats_t._fields_}


def kv_pool_free_list(handle):
    n = ctypes.c_int32()
    _check(lib().kv_pool_free_list(handle, None, 0, ctypes.byref(n)))
    out = (ctypes.c_int32 * max(1, n.value))()
    _check(lib().kv_pool_free_list(handle, out, n.value, None))
    return list(out)[:n.value]


def kv_pool_set_swap_space(handle, host_blocks, host_slots):
    _check(lib().kv_pool_set_swap_space(handle, int(host_blocks), int(host_slots)))


def swap_plan_cap(handle, seqs):
    """Plan entries a swap of these sequences can need: their table lengths
    plus one slot entry each (unknown sequences count 0; the call reports them)."""
    cap = len(seqs)
    for s in seqs:
        try:
            cap += len(kv_seq_table(handle, s)[0])
        except PBQError:
            pass
    return cap


def _swap(fn, handle, seqs, plan):
    n = len(seqs)
    sq = (ctypes.c_int64 * max(1, n))(*[int(s) for s in seqs])
    cnt = ctypes.c_int32()
    if plan is None:
        cap = swap_plan_cap(handle, seqs)
        buf = (kv_swap * max(1, cap))()
        _check(fn(handle, sq, n, buf, cap, ctypes.byref(cnt)))
        return [(buf[i].kind, buf[i].src, buf[i].dst, buf[i].rows) for i in range(cnt.value)]
    assert plan.dtype == torch.int32 and plan.dim() == 2 and plan.shape[1] == 4 and plan.is_contiguous()
    _check(fn(handle, sq, n, ctypes.cast(plan.data_ptr(), ctypes.POINTER(kv_swap)), plan.shape[0],
              ctypes.byref(cnt)))
    return cnt.value


def kv_seq_swap_out(handle, seqs, plan=None):
    """Without ``plan``: returns the plan as (kind, src, dst, rows) tuples.
    With ``plan`` (int32 [cap, 4] CPU tensor, e.g. pinned): writes it there
    and returns the number of entries."""
    return _swap(lib().kv_seq_swap_out, handle, seqs, plan)


def kv_seq_swap_in(handle, seqs, plan=None):
    return _swap(lib().kv_seq_swap_in, handle, seqs, plan)


def kv_swap_blocks(desc, mem, host_desc, host_mem, plan, n, stream=None):
    _check(lib().kv_swap_blocks(ctypes.byref(desc), ctypes.byref(mem), ctypes.byref(host_desc),
                                ctypes.byref(host_mem), _ptr(plan), int(n), _stream(stream)))


def kv_copy_blocks(desc, mem, copies_dev, n, stream=None):
    _check(lib().kv_copy_blocks(ctypes.byref(desc), ctypes.byref(mem), _ptr(copies_dev), int(n),
                                _stream(stream)))


def kv_quantize_store(desc, mem, k, v, num_seqs, cu_seqlens, start_pos, block_tables,
                      max_blocks_per_seq, tail_slots, max_new_tokens, stream=None):
    _check(lib().kv_quantize_store(ctypes.byref(desc), ctypes.byref(mem), _ptr(k), _ptr(v),
                                   int(num_seqs), _ptr(cu_seqlens), _ptr(start_pos),
                                   _ptr(block_tables), int(max_blocks_per_seq), _ptr(tail_slots),
                                   int(max_new_tokens), _stream(stream)))


def paged_attn_workspace_bytes(desc, num_seqs, num_q_heads, max_context_len, partition_size=0):
    return lib().paged_attn_workspace_bytes(ctypes.byref(desc), int(num_seqs), int(num_q_heads),
                                            int(max_context_len), int(partition_size))


def paged_attn_default_partition(desc, num_seqs, num_q_heads, max_context_len):
    return lib().paged_attn_default_partition(ctypes.byref(desc), int(num_seqs),
                                              int(num_q_heads), int(max_context_len))


def paged_attn_decode(desc, mem, q, out, num_seqs, num_q_heads, block_tables,
                      max_blocks_per_seq, context_lens, max_context_len, sm_scale,
                      partition_size=0, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().paged_attn_decode(ctypes.byref(desc), ctypes.byref(mem), _ptr(q), _ptr(out),
                                   int(num_seqs), int(num_q_heads), _ptr(block_tables),
                                   int(max_blocks_per_seq), _ptr(context_lens),
                                   int(max_context_len), float(sm_scale), int(partition_size),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream)))


def paged_attn_decode_append(desc, mem, k_new, v_new, tail_slots, q, out, num_seqs, num_q_heads,
                             block_tables, max_blocks_per_seq, context_lens, max_context_len,
                             sm_scale, partition_size=0, workspace=None, workspace_bytes=0,
                             stream=None):
    _check(lib().paged_attn_decode_append(ctypes.byref(desc), ctypes.byref(mem), _ptr(k_new),
                                          _ptr(v_new), _ptr(tail_slots), _ptr(q), _ptr(out),
                                          int(num_seqs), int(num_q_heads), _ptr(block_tables),
                                          int(max_blocks_per_seq), _ptr(context_lens),
                                          int(max_context_len), float(sm_scale),
                                          int(partition_size), _ptr(workspace),
                                          int(workspace_bytes), _stream(stream)))


def paged_attn_decode_append_noalloc(desc, mem, k_new, v_new, tail_slots, q, out, num_seqs, num_q_heads,
                                     block_tables, max_blocks_per_seq, context_lens, max_context_len,
                                     sm_scale, partition_size=0, stream=None):
    _check(lib().paged_attn_decode_append_noalloc(ctypes.byref(desc), ctypes.byref(mem), _ptr(k_new),
                                                  _ptr(v_new), _ptr(tail_slots), _ptr(q), _ptr(out),
                                                  int(num_seqs), int(num_q_heads), _ptr(block_tables),
                                                  int(max_blocks_per_seq), _ptr(context_lens),
                                                  int(max_context_len), float(sm_scale),
                                                  int(partition_size), _stream(stream)))


def paged_attn_decode_shared_prefix(desc, mem, k_new, v_new, tail_slots, q, out, num_seqs,
                                    num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                                    max_context_len, sm_scale, partition_size, shared_tokens,
                                    workspace=None, workspace_bytes=0, stream=None):
    _check(lib().paged_attn_decode_shared_prefix(
        ctypes.byref(desc), ctypes.byref(mem), _ptr(k_new), _ptr(v_new), _ptr(tail_slots), _ptr(q),
        _ptr(out), int(num_seqs), int(num_q_heads), _ptr(block_tables), int(max_blocks_per_seq),
        _ptr(context_lens), int(max_context_len), float(sm_scale), int(partition_size),
        int(shared_tokens), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def paged_attn_multi_query_workspace_bytes(desc, num_seqs, num_tokens, num_q_heads, max_q_len,
                                           max_context_len, partition_size=0):
    return lib().paged_attn_multi_query_workspace_bytes(ctypes.byref(desc), int(num_seqs), int(num_tokens),
                                                        int(num_q_heads), int(max_q_len),
                                                        int(max_context_len), int(partition_size))


def paged_attn_multi_query(desc, mem, q, out, num_seqs, num_q_heads, cu_seqlens, num_tokens, max_q_len,
                           block_tables, max_blocks_per_seq, context_lens, max_context_len, sm_scale,
                           partition_size=0, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().paged_attn_multi_query(
        ctypes.byref(desc), ctypes.byref(mem), _ptr(q), _ptr(out), int(num_seqs), int(num_q_heads),
        _ptr(cu_seqlens), int(num_tokens), int(max_q_len), _ptr(block_tables), int(max_blocks_per_seq),
        _ptr(context_lens), int(max_context_len), float(sm_scale), int(partition_size), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def kv_stream_read_sink_words(n_tiles):
    return lib().kv_stream_read_sink_words(int(n_tiles))


def kv_stream_read_tiles(src, n_src_tiles, tile_bytes, order, n_tiles, sink, stream=None):
    _check(lib().kv_stream_read_tiles(_ptr(src), int(n_src_tiles), int(tile_bytes), _ptr(order), int(n_tiles),
                                      _ptr(sink), int(sink.numel()), _stream(stream)))


def kv_set_debug_checks(on):
    """Turns the library's debug checks of caller contracts on or off;
    returns the previous setting."""
    return int(lib().kv_set_debug_checks(1 if on else 0))

"""KVPool: one layer's block pool -- the host allocator handle plus the device
arrays it indexes, allocated as torch CUDA tensors.  Marshalling only: every
operation is a call into libpbq (include/pbq.h)."""

import torch

from . import _lib as L


class KVPool:
    """Host allocator (``kv_pool_create``) + device arrays sized by
    ``kv_pool_bytes``.

    v_codec: "i8" (INT8 symmetric), "i4" (INT4 asymmetric), "i8a" (INT8
    asymmetric) or "fp8" (FP8 E4M3) V; k_codec: "i8", "fp8" or "i4" (INT4
    asymmetric, with V "i4" or "i8"), by default "fp8" exactly when V is FP8.
    free_order: initial free stack (a permutation of 0..N-1) or None.
    """

    CODECS = {"i8": L.KV_CODEC_I8_SYM, "i4": L.KV_CODEC_I4_ASYM, "fp8": L.KV_CODEC_FP8_E4M3,
              "i8a": L.KV_CODEC_I8_ASYM}

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, v_codec="i8",
                 max_seqs=1, free_order=None, device="cuda", k_codec=None):
        k_codec = k_codec or ("fp8" if v_codec == "fp8" else "i8")
        self.desc = L.make_desc(num_blocks, block_size, num_kv_heads, head_dim, self.CODECS[v_codec],
                                max_seqs, k_codec=self.CODECS[k_codec])
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.k_codec, self.v_codec = k_codec, v_codec
        self.v_int4 = v_codec == "i4"
        self.v_zp_used = v_codec in ("i4", "i8a")
        self.k_int4 = k_codec == "i4"
        self.k_zp_used = k_codec == "i4"
        self.max_seqs = max_seqs
        self.handle = L.kv_pool_create(self.desc, free_order)
        self.sizes = L.kv_pool_bytes(self.desc)
        self.device = device
        self.arrays = {}
        if device is not None:
            N, H, bs, D = num_blocks, num_kv_heads, block_size, head_dim
            dev = torch.device(device)
            self.arrays = self._arrays(N, max_seqs, lambda shape, dtype: torch.zeros(shape, dtype=dtype, device=dev))
            for name, t in self.arrays.items():
                if not self._used(name):
                    continue
                assert t.numel() * t.element_size() == self.sizes[name], name
            self.mem = self._mem(self.arrays)

    def _used(self, name):
        """False for a zero-point array the codecs do not use."""
        return not ((name == "v_zp" and not self.v_zp_used) or (name == "k_zp" and not self.k_zp_used))

    def _arrays(self, nb, ns, make):
        """The pool's arrays for nb blocks and ns tail slots (layout as
        kv_pool_bytes gives it), each from make(shape, dtype)."""
        H, bs, D = self.num_kv_heads, self.block_size, self.head_dim
        return {
            # K tiles are token-major: [bs, D] codes per (block, head); INT4
            # packs two consecutive head dims per byte
            "k_codes": make((nb, H, bs, D // 2 if self.k_int4 else D),
                            torch.int8 if self.k_codec == "i8" else torch.uint8),
            # V tiles are dim-major: [D, bs] codes per (block, head)
            "v_codes": make((nb, H, D, bs // 2 if self.v_int4 else bs),
                            torch.int8 if self.v_codec == "i8" else torch.uint8),
            "k_scale": make((nb, H), torch.float16),
            "v_scale": make((nb, H), torch.float16),
            "v_zp": make((nb, H) if self.v_zp_used else (1,), torch.uint8),
            "tail_k": make((ns, H, bs, D), torch.float16),
            "tail_v": make((ns, H, bs, D), torch.float16),
            "k_zp": make((nb, H) if self.k_zp_used else (1,), torch.uint8),
        }

    def _mem(self, arrays):
        return L.kv_pool_mem(*[arrays[n].data_ptr() if self._used(n) else None for n in L.POOL_ARRAYS])

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays", {})
        if name in arrays:
            return arrays[name]
        raise AttributeError(name)

    def close(self):
        if getattr(self, "handle", None) is not None:
            L.kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- host allocator ----------------------------------------------------
    def alloc(self, seq, num_tokens):
        L.kv_seq_alloc(self.handle, seq, num_tokens)
        return self.table(seq)[0]

    def alloc_prefix(self, seq, token_ids):
        """alloc through the prefix cache; returns (block table, cached tokens)."""
        cached = L.kv_seq_alloc_prefix(self.handle, seq, token_ids)
        return self.table(seq)[0], cached

    def fork(self, parent, child):
        return L.kv_seq_fork(self.handle, parent, child)

    def append(self, seq, n_tokens):
        return L.kv_seq_append(self.handle, seq, n_tokens)

    def release(self, seq):
        L.kv_seq_free(self.handle, seq)

    def table(self, seq):
        return L.kv_seq_table(self.handle, seq)

    def batch_tables(self, seqs, max_blocks):
        return L.kv_batch_tables(self.handle, seqs, max_blocks)

    def stats(self):
        return L.kv_pool_stats(self.handle)

    def free_list(self):
        return L.kv_pool_free_list(self.handle)

    # ---- swap space (deepinsea.top "Swap") ----------------------------------
    def set_swap_space(self, host_blocks, host_slots):
        """Size the swap space and allocate its arrays, the device arrays'
        layout for host_blocks blocks and host_slots slots, in pinned host
        memory."""
        L.kv_pool_set_swap_space(self.handle, host_blocks, host_slots)
        nb, ns = max(1, host_blocks), max(1, host_slots)
        self.host_desc = L.make_desc(nb, self.block_size, self.num_kv_heads, self.head_dim,
                                     self.desc.v_codec, ns, k_codec=self.desc.k_codec)
        self.host_arrays = {}
        self.host_mem = None
        if self.device is None:
            return
        self.host_arrays = self._arrays(nb, ns, lambda shape, dtype: torch.zeros(shape, dtype=dtype,
                                                                                pin_memory=True))
        self.host_mem = self._mem(self.host_arrays)

    def _run_plan(self, fn, seqs, stream, mem):
        cap = L.swap_plan_cap(self.handle, seqs)
        plan = torch.zeros((max(1, cap), 4), dtype=torch.int32, pin_memory=True)
        n = fn(self.handle, seqs, plan)
        if n:
            L.kv_swap_blocks(self.desc, self.mem if mem is None else mem, self.host_desc,
                             self.host_mem, plan, n, stream)
        # the kernel reads the plan from host memory: keep it until the stream
        # has passed the copy
        ev = torch.cuda.Event()
        ev.record(stream if stream is not None else torch.cuda.current_stream())
        self._plans = [(e, p) for e, p in getattr(self, "_plans", []) if not e.query()]
        self._plans.append((ev, plan))
        return [tuple(r) for r in plan[:n].tolist()]

    def swap_out(self, seqs, stream=None, mem=None):
        """Swap a group of sequences out and enqueue the copies on stream;
        returns the plan as (kind, src, dst, rows) tuples."""
        return self._run_plan(L.kv_seq_swap_out, seqs, stream, mem)

    def swap_in(self, seqs, stream=None, mem=None):
        return self._run_plan(L.kv_seq_swap_in, seqs, stream, mem)

    # ---- device calls ------------------------------------------------------
    def copy_blocks(self, copies, stream=None):
        """Perform (kind, src, dst) copies returned by fork/append."""
        if not copies:
            return
        t = torch.tensor([list(c) for c in copies], dtype=torch.int32).to(self.device)
        L.kv_copy_blocks(self.desc, self.mem, t, len(copies), stream)
        return t  # keep alive until the stream has consumed it

    def replica(self):
        """A copy of the pool's code, scale and zero-point arrays in fresh
        device memory (tail slots shared), as a kv_pool_mem: the same cache
        contents at other addresses, e.g. to stand for another layer's pool."""
        keep = {n: (t if n.startswith("tail") or not self._used(n) else t.clone())
                for n, t in self.arrays.items()}
        return self._mem(keep), keep

    def quantize_store(self, k, v, cu_seqlens, start_pos, block_tables, tail_slots,
                       max_new_tokens, stream=None, mem=None):
        L.kv_quantize_store(self.desc, self.mem if mem is None else mem, k, v,
                            cu_seqlens.numel() - 1, cu_seqlens, start_pos, block_tables,
                            block_tables.shape[1], tail_slots, max_new_tokens, stream)

    def workspace_bytes(self, num_seqs, num_q_heads, max_context_len, partition_size=0):
        return L.paged_attn_workspace_bytes(self.desc, num_seqs, num_q_heads, max_context_len,
                                            partition_size)

    def default_partition(self, num_seqs, num_q_heads, max_context_len):
        return L.paged_attn_default_partition(self.desc, num_seqs, num_q_heads, max_context_len)

    def decode(self, q, out, block_tables, context_lens, max_context_len, sm_scale,
               partition_size=0, workspace=None, stream=None, mem=None):
        S, Hq, _ = q.shape
        need = self.workspace_bytes(S, Hq, max_context_len, partition_size)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        L.paged_attn_decode(self.desc, self.mem if mem is None else mem, q, out, S, Hq,
                            block_tables, block_tables.shape[1], context_lens, max_context_len,
                            sm_scale, partition_size, workspace, nbytes, stream)
        return workspace

    def decode_append(self, k_new, v_new, tail_slots, q, out, block_tables, context_lens,
                      max_context_len, sm_scale, partition_size=0, workspace=None, stream=None,
                      mem=None):
        """Store each sequence's current token (k_new / v_new [S, Hkv, D] fp16,
        at position context_lens - 1) and decode, in one library call."""
        S, Hq, _ = q.shape
        need = self.workspace_bytes(S, Hq, max_context_len, partition_size)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        L.paged_attn_decode_append(self.desc, self.mem if mem is None else mem, k_new, v_new,
                                   tail_slots, q, out, S, Hq, block_tables, block_tables.shape[1],
                                   context_lens, max_context_len, sm_scale, partition_size,
                                   workspace, nbytes, stream)
        return workspace

    def multi_query(self, q, out, cu_seqlens, max_q_len, block_tables, context_lens, max_context_len,
                    sm_scale, partition_size=0, workspace=None, stream=None, mem=None):
        """Several query tokens per sequence (q, out [T, Hq, D]; sequence s's
        rows cu_seqlens[s] .. cu_seqlens[s+1]-1 are its last stored tokens),
        each attending causally."""
        T, Hq, _ = q.shape
        S = cu_seqlens.numel() - 1
        need = L.paged_attn_multi_query_workspace_bytes(self.desc, S, T, Hq, max_q_len, max_context_len,
                                                        partition_size)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        L.paged_attn_multi_query(self.desc, self.mem if mem is None else mem, q, out, S, Hq, cu_seqlens, T,
                                 max_q_len, block_tables, block_tables.shape[1], context_lens, max_context_len,
                                 sm_scale, partition_size, workspace, nbytes, stream)
        return workspace

    def decode_shared_prefix(self, q, out, block_tables, context_lens, max_context_len, sm_scale,
                             partition_size, shared_tokens, k_new=None, v_new=None,
                             tail_slots=None, workspace=None, stream=None, mem=None):
        """decode (k_new None) or decode_append for sequences whose first
        shared_tokens tokens sit in the same physical blocks."""
        S, Hq, _ = q.shape
        need = self.workspace_bytes(S, Hq, max_context_len, partition_size)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        L.paged_attn_decode_shared_prefix(self.desc, self.mem if mem is None else mem, k_new, v_new,
                                          tail_slots, q, out, S, Hq, block_tables,
                                          block_tables.shape[1], context_lens, max_context_len,
                                          sm_scale, partition_size, shared_tokens, workspace,
                                          nbytes, stream)
        return workspace

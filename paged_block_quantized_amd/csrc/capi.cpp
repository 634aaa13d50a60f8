// C-ABI layer: argument validation, sizing, and dispatch of the device calls
// declared in include/pbq.h.  No exception crosses the boundary; every
// failure sets a thread-local message.

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>
#include <algorithm>

#include "pbq_internal.h"

namespace pbq {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

kv_status check_device_desc(const kv_pool_desc* d) {
    if (!d) return fail(KV_ERR_INVALID, "desc is NULL");
    if (d->num_blocks < 1) return fail(KV_ERR_INVALID, "num_blocks must be >= 1");
    if (d->block_size != 16 && d->block_size != 32)
        return fail(KV_ERR_INVALID, "block_size must be 16 or 32");
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(KV_ERR_INVALID, "head_dim must be 64 or 128");
    if (d->num_kv_heads < 1 || d->num_kv_heads > 65535)
        return fail(KV_ERR_INVALID, "num_kv_heads must be in [1, 65535]");
    if (d->max_seqs < 1) return fail(KV_ERR_INVALID, "max_seqs must be >= 1");
    if (!codec_pair_supported(d->k_codec, d->v_codec))
        return fail(KV_ERR_INVALID, "unsupported (k_codec, v_codec): use (I8_SYM, I8_SYM | I4_ASYM | I8_ASYM), "
                                    "(FP8_E4M3, FP8_E4M3) or (I4_ASYM, I4_ASYM | I8_SYM)");
    return KV_OK;
}

kv_status check_mem(const kv_pool_desc* d, const kv_pool_mem* m, bool need_tail) {
    if (!m) return fail(KV_ERR_INVALID, "mem is NULL");
    const void* req[] = {m->k_codes, m->v_codes, m->k_scale, m->v_scale};
    for (const void* p : req)
        if (!p || !aligned16(p)) return fail(KV_ERR_INVALID, "pool arrays must be non-NULL and 16-byte aligned");
    if (codec_has_zp(d->v_codec) && (!m->v_zp || !aligned16(m->v_zp)))
        return fail(KV_ERR_INVALID, "v_zp must be non-NULL and 16-byte aligned for an asymmetric V codec");
    if (codec_has_zp(d->k_codec) && (!m->k_zp || !aligned16(m->k_zp)))
        return fail(KV_ERR_INVALID, "k_zp must be non-NULL and 16-byte aligned for an asymmetric K codec");
    if (need_tail && (!m->tail_k || !m->tail_v || !aligned16(m->tail_k) || !aligned16(m->tail_v)))
        return fail(KV_ERR_INVALID, "tail slots must be non-NULL and 16-byte aligned");
    return KV_OK;
}

kv_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return KV_OK;
    return fail(KV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Device address of pinned host memory [p, p + bytes): KV_ERR_INVALID unless
// HIP knows both ends as host memory mapped contiguously for the device.
kv_status pinned_device_ptr(const void* p, size_t bytes, const char* what, char** dev) {
    hipPointerAttribute_t at{}, end{};
    if (!p || hipPointerGetAttributes(&at, p) != hipSuccess || at.type != hipMemoryTypeHost ||
        !at.devicePointer ||
        hipPointerGetAttributes(&end, (const char*)p + bytes - 1) != hipSuccess ||
        end.type != hipMemoryTypeHost ||
        (const char*)end.devicePointer != (const char*)at.devicePointer + bytes - 1) {
        (void)hipGetLastError();
        return fail(KV_ERR_INVALID, std::string(what) + " must be pinned host memory (hipHostMalloc)");
    }
    *dev = (char*)at.devicePointer;
    return KV_OK;
}

// Checks a swap plan on the host: kinds, index ranges, rows, and that no
// destination is written twice or also read within the call (the entries
// run concurrently).  Returns the largest entry's byte count in *max_bytes.
kv_status check_swap_plan(const kv_pool_desc* d, const kv_pool_desc* h, const kv_swap* plan,
                          int32_t n, bool* has_slots, int64_t* max_bytes) {
    const int64_t tile = (int64_t)d->block_size * d->head_dim;
    const int64_t kb = tile * d->num_kv_heads;
    const int64_t block_bytes = (codec_packed4(d->k_codec) ? kb / 2 : kb) + (codec_packed4(d->v_codec) ? kb / 2 : kb);
    // spaces: device blocks, host blocks, device slots, host slots
    const int32_t size[4] = {d->num_blocks, h->num_blocks, d->max_seqs, h->max_seqs};
    std::vector<uint8_t> mark[4];
    for (int i = 0; i < 4; ++i) mark[i].assign(size[i], 0);
    *has_slots = false;
    *max_bytes = 0;
    for (int pass = 0; pass < 2; ++pass)
        for (int32_t i = 0; i < n; ++i) {
            const kv_swap& c = plan[i];
            int from, to;
            switch (c.kind) {
                case KV_SWAP_BLOCK_OUT: from = 0, to = 1; break;
                case KV_SWAP_BLOCK_IN: from = 1, to = 0; break;
                case KV_SWAP_SLOT_OUT: from = 2, to = 3; break;
                case KV_SWAP_SLOT_IN: from = 3, to = 2; break;
                default: return fail(KV_ERR_INVALID, "swap plan: unknown kind");
            }
            if (c.src < 0 || c.src >= size[from] || c.dst < 0 || c.dst >= size[to])
                return fail(KV_ERR_INVALID, "swap plan: index out of range");
            const bool slot = from >= 2;
            if (slot ? (c.rows < 1 || c.rows > d->block_size) : c.rows != 0)
                return fail(KV_ERR_INVALID, "swap plan: rows must be 1..block_size for slots, 0 for blocks");
            if (pass == 0) {
                mark[from][c.src] |= 1;
                *has_slots |= slot;
                *max_bytes = std::max(*max_bytes, slot ? 4 * tile / d->block_size * c.rows * d->num_kv_heads
                                                       : block_bytes);
            } else {
                if (mark[to][c.dst]) return fail(KV_ERR_INVALID, "swap plan: a destination is written twice or also read");
                mark[to][c.dst] = 2;
            }
        }
    return KV_OK;
}

// Compute units of the current device, cached per device; 256 (MI355X) when
// no device can be queried.
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// ---- debug checks of caller contracts ------------------------------------
// On when kv_set_debug_checks(1) was called, or (until then) when the
// environment variable PBQ_DEBUG_CHECKS is set to anything but "0".  They
// copy the calls' index arrays to the host (after synchronizing the stream),
// so they are for debugging, not for timed runs.
std::atomic<int> g_debug_checks{-1};

bool debug_checks() {
    int v = g_debug_checks.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = std::getenv("PBQ_DEBUG_CHECKS");
        v = e && *e && std::strcmp(e, "0") != 0 ? 1 : 0;
        int expected = -1;
        g_debug_checks.compare_exchange_strong(expected, v);
        v = g_debug_checks.load(std::memory_order_relaxed);
    }
    return v > 0;
}

template <class T>
kv_status fetch(const T* dev, size_t n, std::vector<T>& out, hipStream_t stream) {
    out.assign(n, T{});
    if (n == 0) return KV_OK;
    kv_status st = hip_status(hipStreamSynchronize(stream), "debug check: stream synchronize");
    if (st != KV_OK) return st;
    return hip_status(hipMemcpy(out.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost), "debug check: copy");
}

// The tiles one store call writes run concurrently: no physical block may be
// written for two sequences, and no tail slot may be written twice (rows are
// kept in a sequence's slot while its last block stays partial).  Sequence
// s writes positions first[s] .. end[s] - 1 through its table row.
kv_status check_disjoint_writes(const kv_pool_desc* d, const char* call, const std::vector<int32_t>& tables,
                                int32_t max_blocks, const std::vector<int32_t>& first,
                                const std::vector<int32_t>& end, const std::vector<int32_t>& slots) {
    const int32_t bs = d->block_size;
    std::vector<int32_t> owner_block(d->num_blocks, -1), owner_slot(d->max_seqs, -1);
    for (size_t s = 0; s < first.size(); ++s) {
        if (end[s] <= first[s]) continue;
        for (int32_t j = first[s] / bs; j <= (end[s] - 1) / bs; ++j) {
            if (j >= max_blocks) return fail(KV_ERR_INVALID, std::string(call) + ": a store runs past its table row");
            const int32_t b = tables[s * (size_t)max_blocks + j];
            if (b < 0 || b >= d->num_blocks) return fail(KV_ERR_INVALID, std::string(call) + ": block id out of range");
            if (owner_block[b] >= 0 && owner_block[b] != (int32_t)s)
                return fail(KV_ERR_INVALID, std::string(call) + ": block " + std::to_string(b) + " is written for sequences " +
                                                std::to_string(owner_block[b]) + " and " + std::to_string(s) +
                                                " in one call (copy-on-write first)");
            owner_block[b] = (int32_t)s;
        }
        if (end[s] % bs != 0) {   // the last block stays partial: its rows go to the slot
            const int32_t sl = slots[s];
            if (sl < 0 || sl >= d->max_seqs) return fail(KV_ERR_INVALID, std::string(call) + ": tail slot out of range");
            if (owner_slot[sl] >= 0)
                return fail(KV_ERR_INVALID, std::string(call) + ": tail slot " + std::to_string(sl) +
                                                " is written for two sequences in one call");
            owner_slot[sl] = (int32_t)s;
        }
    }
    return KV_OK;
}

}  // namespace

kv_status fail(kv_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

}  // namespace pbq

using pbq::fail;

namespace {

// New-token arguments of the fused store + decode (NULL for plain decode).
struct AppendArgs {
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int32_t* tail_slots;
};

// use_scratch: the workspace is the library's own scratch (workspace and
// workspace_bytes are ignored), looked up only after every argument check.
kv_status decode_impl(const kv_pool_desc* d, const kv_pool_mem* m, const AppendArgs* app,
                            const uint16_t* q, uint16_t* out, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float sm_scale,
                            int32_t partition_size, int32_t shared_tokens, void* workspace,
                            size_t workspace_bytes, void* stream, bool use_scratch = false) {
    kv_status st = pbq::check_device_desc(d);
    if (st != KV_OK) return st;
    if ((st = pbq::check_mem(d, m, app != nullptr)) != KV_OK) return st;
    if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0)
        return fail(KV_ERR_INVALID, "negative size argument");
    if (num_q_heads < 1 || num_q_heads % d->num_kv_heads != 0)
        return fail(KV_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
    if (num_q_heads / d->num_kv_heads > 16 && (num_q_heads / d->num_kv_heads) % 16 != 0)
        return fail(KV_ERR_INVALID, "query-group sizes above 16 must be multiples of 16");
    if (num_seqs == 0) return KV_OK;
    if (num_seqs > 65535 || num_q_heads > 65535)
        return fail(KV_ERR_INVALID, "num_seqs and num_q_heads must stay below 65536");
    if (!q || !out || !pbq::aligned16(q) || !pbq::aligned16(out))
        return fail(KV_ERR_INVALID, "q and out must be non-NULL and 16-byte aligned");
    if (!block_tables || !context_lens) return fail(KV_ERR_INVALID, "index arrays must be non-NULL");
    if (app && (!app->k_new || !app->v_new || !pbq::aligned16(app->k_new) || !pbq::aligned16(app->v_new)))
        return fail(KV_ERR_INVALID, "k_new and v_new must be non-NULL and 16-byte aligned");
    if (app && !app->tail_slots) return fail(KV_ERR_INVALID, "tail_slots must be non-NULL");
    if (app && max_blocks_per_seq < 1) return fail(KV_ERR_INVALID, "max_blocks_per_seq must be >= 1");
    if ((int64_t)max_blocks_per_seq * d->block_size < max_context_len)
        return fail(KV_ERR_INVALID, "max_blocks_per_seq * block_size < max_context_len");
    if (!std::isfinite(sm_scale))
        return fail(KV_ERR_INVALID, "sm_scale must be finite");
    int32_t part = partition_size;
    if (part == 0) part = paged_attn_default_partition(d, num_seqs, num_q_heads, max_context_len);
    if (part <= 0 || part % d->block_size != 0)
        return fail(KV_ERR_INVALID, "partition_size must be a positive multiple of block_size (or 0)");
    if (num_q_heads != d->num_kv_heads && part % 32 != 0)
        return fail(KV_ERR_INVALID, "grouped-query partition_size must be a multiple of 32 tokens");
    const int32_t max_parts = max_context_len > 0 ? pbq::ceil_div(max_context_len, part) : 1;
    if (max_parts > 65535) return fail(KV_ERR_INVALID, "too many partitions; use a larger partition_size");
    if (shared_tokens < 0) return fail(KV_ERR_INVALID, "shared_tokens must be >= 0");
    if (shared_tokens > 0) {
        if (partition_size == 0 || part % 32 != 0)
            return fail(KV_ERR_INVALID, "a shared prefix needs an explicit partition_size, a multiple of 32");
        if (shared_tokens % part != 0)
            return fail(KV_ERR_INVALID, "shared_tokens must be a multiple of partition_size");
        if (shared_tokens >= max_context_len)
            return fail(KV_ERR_INVALID, "shared_tokens must be below max_context_len");
        const int64_t nq = (int64_t)num_seqs * (num_q_heads / d->num_kv_heads);
        if ((int64_t)d->num_kv_heads * ((nq + 15) / 16) > 65535)
            return fail(KV_ERR_INVALID, "too many queries per KV head for the shared-prefix launch");
    }
    if (pbq::debug_checks() && (app || shared_tokens > 0)) {
        std::vector<int32_t> ctx, tab, sl;
        const hipStream_t s = (hipStream_t)stream;
        if ((st = pbq::fetch(context_lens, num_seqs, ctx, s)) != KV_OK ||
            (st = pbq::fetch(block_tables, (size_t)num_seqs * max_blocks_per_seq, tab, s)) != KV_OK)
            return st;
        if (app) {   // each sequence stores its current token (position ctx - 1)
            if ((st = pbq::fetch(app->tail_slots, num_seqs, sl, s)) != KV_OK) return st;
            std::vector<int32_t> first(num_seqs);
            for (int32_t i = 0; i < num_seqs; ++i) {
                if (ctx[i] < 1 || ctx[i] > max_context_len)
                    return fail(KV_ERR_INVALID, "decode with append: context_lens must be in [1, max_context_len]");
                first[i] = ctx[i] - 1;
            }
            if ((st = pbq::check_disjoint_writes(d, "paged_attn_decode_append", tab, max_blocks_per_seq, first, ctx,
                                                 sl)) != KV_OK)
                return st;
        }
        if (shared_tokens > 0) {   // the prefix's blocks are sequence 0's for every sequence
            const int32_t nb = shared_tokens / d->block_size;
            for (int32_t i = 0; i < num_seqs; ++i) {
                if (ctx[i] <= shared_tokens)
                    return fail(KV_ERR_INVALID, "shared prefix: a context_lens entry does not exceed shared_tokens");
                for (int32_t j = 0; j < nb; ++j)
                    if (tab[i * (size_t)max_blocks_per_seq + j] != tab[j])
                        return fail(KV_ERR_INVALID, "shared prefix: sequence " + std::to_string(i) + "'s block " +
                                                        std::to_string(j) + " differs from sequence 0's");
            }
        }
    }
    const size_t need = paged_attn_workspace_bytes(d, num_seqs, num_q_heads, max_context_len, part);
    if (use_scratch) {
        if (need > pbq::kScratchBytes)
            return fail(KV_ERR_INVALID, "the call needs " + std::to_string(need) +
                                            " bytes of workspace, more than the library's scratch (" +
                                            std::to_string(pbq::kScratchBytes) +
                                            " bytes); use paged_attn_decode_append");
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            st = pbq::hip_status(pbq::scratch_address(&workspace), "paged_attn_decode_append_noalloc scratch");
            if (st != KV_OK) return st;
            workspace_bytes = pbq::kScratchBytes;
        }
    }
    if (workspace_bytes < need) return fail(KV_ERR_INVALID, "workspace too small");
    if (need > 0 && (!workspace || !pbq::aligned16(workspace)))
        return fail(KV_ERR_INVALID, "workspace must be non-NULL and 16-byte aligned");
    pbq::AttnArgs a{};
    a.block_size = d->block_size;
    a.num_kv_heads = d->num_kv_heads;
    a.head_dim = d->head_dim;
    a.v_codec = d->v_codec;
    a.k_codec = d->k_codec;
    a.k_codes = (const int8_t*)m->k_codes;
    a.v_codes = (const uint8_t*)m->v_codes;
    a.k_scale = (const uint16_t*)m->k_scale;
    a.v_scale = (const uint16_t*)m->v_scale;
    a.v_zp = (const uint8_t*)m->v_zp;
    a.k_zp = (const uint8_t*)m->k_zp;
    a.q = q;
    a.out = out;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.sm_scale = sm_scale;
    a.partition_blocks = part / d->block_size;
    a.max_partitions = max_parts;
    a.shared_tokens = shared_tokens;
    a.shared_parts = shared_tokens / part;
    const size_t rows = (size_t)num_seqs * num_q_heads * max_parts;
    a.ws_out = need ? (float*)workspace : nullptr;
    a.ws_ml = need ? (float*)((char*)workspace + rows * (size_t)d->head_dim * 4) : nullptr;
    if (app && max_parts > 1 && !pbq::split_store_fused(a)) {
        // split partitions the partition kernels do not fuse the store into
        // (grouped query heads, or an MHA kernel that would lose occupancy:
        // all but one work group per sequence and head would carry the fused
        // store's registers for nothing): the store kernel in one-token
        // append mode, then the decode
        pbq::QuantStoreArgs sa{};
        sa.block_size = d->block_size;
        sa.num_kv_heads = d->num_kv_heads;
        sa.head_dim = d->head_dim;
        sa.v_codec = d->v_codec;
        sa.k_codec = d->k_codec;
        sa.k_codes = (int8_t*)m->k_codes;
        sa.v_codes = (uint8_t*)m->v_codes;
        sa.k_scale = (uint16_t*)m->k_scale;
        sa.v_scale = (uint16_t*)m->v_scale;
        sa.v_zp = (uint8_t*)m->v_zp;
        sa.k_zp = (uint8_t*)m->k_zp;
        sa.tail_k = (uint16_t*)m->tail_k;
        sa.tail_v = (uint16_t*)m->tail_v;
        sa.k = app->k_new;
        sa.v = app->v_new;
        sa.num_seqs = num_seqs;
        sa.block_tables = block_tables;
        sa.max_blocks_per_seq = max_blocks_per_seq;
        sa.tail_slots = app->tail_slots;
        sa.tiles_per_seq = 1;
        sa.append_ctx = context_lens;
        st = pbq::hip_status(pbq::launch_quantize_store(sa, (hipStream_t)stream), "paged_attn_decode_append store launch");
        if (st != KV_OK) return st;
    } else if (app) {
        a.k_new = app->k_new;
        a.v_new = app->v_new;
        a.tail_slots = app->tail_slots;
        a.tail_k = (uint16_t*)m->tail_k;
        a.tail_v = (uint16_t*)m->tail_v;
    }
    return pbq::hip_status(pbq::launch_paged_attn(a, (hipStream_t)stream), "paged_attn_decode launch");
}

}  // namespace

extern "C" {

const char* kv_last_error(void) { return pbq::g_last_error.c_str(); }

int32_t kv_set_debug_checks(int32_t on) {
    pbq::debug_checks();   // settle the environment default first
    return pbq::g_debug_checks.exchange(on ? 1 : 0);
}

kv_status kv_pool_bytes(const kv_pool_desc* d, kv_pool_sizes* out) {
    if (!out) return fail(KV_ERR_INVALID, "out is NULL");
    kv_status st = pbq::check_device_desc(d);
    if (st != KV_OK) return st;
    const size_t tile = (size_t)d->block_size * d->head_dim;
    const size_t bh = (size_t)d->num_blocks * d->num_kv_heads;
    out->k_codes = pbq::codec_packed4(d->k_codec) ? bh * tile / 2 : bh * tile;
    out->v_codes = pbq::codec_packed4(d->v_codec) ? bh * tile / 2 : bh * tile;
    out->k_scale = bh * 2;
    out->v_scale = bh * 2;
    out->v_zp = pbq::codec_has_zp(d->v_codec) ? bh : 0;
    out->k_zp = pbq::codec_has_zp(d->k_codec) ? bh : 0;
    out->tail_k = (size_t)d->max_seqs * d->num_kv_heads * tile * 2;
    out->tail_v = out->tail_k;
    return KV_OK;
}

kv_status kv_copy_blocks(const kv_pool_desc* d, const kv_pool_mem* m,
                         const kv_copy* copies_dev, int32_t n, void* stream) {
    kv_status st = pbq::check_device_desc(d);
    if (st != KV_OK) return st;
    if ((st = pbq::check_mem(d, m, true)) != KV_OK) return st;
    if (n < 0) return fail(KV_ERR_INVALID, "n < 0");
    if (n == 0) return KV_OK;
    if (!copies_dev) return fail(KV_ERR_INVALID, "copies_dev is NULL");
    pbq::CopyArgs a{};
    a.block_size = d->block_size;
    a.num_kv_heads = d->num_kv_heads;
    a.head_dim = d->head_dim;
    a.v_codec = d->v_codec;
    a.k_codec = d->k_codec;
    a.k_codes = (int8_t*)m->k_codes;
    a.v_codes = (uint8_t*)m->v_codes;
    a.k_scale = (uint16_t*)m->k_scale;
    a.v_scale = (uint16_t*)m->v_scale;
    a.v_zp = (uint8_t*)m->v_zp;
    a.k_zp = (uint8_t*)m->k_zp;
    a.tail_k = (uint16_t*)m->tail_k;
    a.tail_v = (uint16_t*)m->tail_v;
    a.copies = copies_dev;
    a.n = n;
    return pbq::hip_status(pbq::launch_copy_blocks(a, (hipStream_t)stream), "kv_copy_blocks launch");
}

kv_status kv_swap_blocks(const kv_pool_desc* d, const kv_pool_mem* m, const kv_pool_desc* hd,
                         const kv_pool_mem* hm, const kv_swap* plan, int32_t n, void* stream) {
    kv_status st = pbq::check_device_desc(d);
    if (st != KV_OK) return st;
    if ((st = pbq::check_device_desc(hd)) != KV_OK) return st;
    if (hd->block_size != d->block_size || hd->num_kv_heads != d->num_kv_heads ||
        hd->head_dim != d->head_dim || hd->k_codec != d->k_codec || hd->v_codec != d->v_codec)
        return fail(KV_ERR_INVALID, "host_desc must have the pool's block_size, heads, head_dim and codecs");
    if (n < 0) return fail(KV_ERR_INVALID, "n < 0");
    if (n == 0) return KV_OK;
    if (!plan) return fail(KV_ERR_INVALID, "plan is NULL");
    bool has_slots = false;
    int64_t max_bytes = 0;
    if ((st = pbq::check_swap_plan(d, hd, plan, n, &has_slots, &max_bytes)) != KV_OK) return st;
    if ((st = pbq::check_mem(d, m, has_slots)) != KV_OK) return st;
    if ((st = pbq::check_mem(hd, hm, has_slots)) != KV_OK) return st;
    const int64_t chunks = (max_bytes + pbq::kSwapChunk - 1) / pbq::kSwapChunk;
    if (chunks > 65535) return fail(KV_ERR_INVALID, "a swap entry is too large for the launch grid");
    kv_pool_sizes hs{};
    if ((st = kv_pool_bytes(hd, &hs)) != KV_OK) return st;
    pbq::SwapArgs a{};
    char* dp = nullptr;
    if ((st = pbq::pinned_device_ptr(plan, sizeof(kv_swap) * (size_t)n, "plan", &dp)) != KV_OK) return st;
    a.plan = (const kv_swap*)dp;
    struct {
        void* p;
        size_t bytes;
        char** out;
        const char* name;
    } host[] = {
        {hm->k_codes, hs.k_codes, &a.host.k_codes, "host k_codes"},
        {hm->v_codes, hs.v_codes, &a.host.v_codes, "host v_codes"},
        {hm->k_scale, hs.k_scale, (char**)&a.host.k_scale, "host k_scale"},
        {hm->v_scale, hs.v_scale, (char**)&a.host.v_scale, "host v_scale"},
        {hm->v_zp, hs.v_zp, (char**)&a.host.v_zp, "host v_zp"},
        {hm->k_zp, hs.k_zp, (char**)&a.host.k_zp, "host k_zp"},
        {has_slots ? hm->tail_k : nullptr, hs.tail_k, &a.host.tail_k, "host tail_k"},
        {has_slots ? hm->tail_v : nullptr, hs.tail_v, &a.host.tail_v, "host tail_v"},
    };
    for (auto& e : host)
        if (e.p && e.bytes && (st = pbq::pinned_device_ptr(e.p, e.bytes, e.name, e.out)) != KV_OK) return st;
    a.dev = pbq::SwapSide{(char*)m->k_codes, (char*)m->v_codes, (uint16_t*)m->k_scale,
                          (uint16_t*)m->v_scale, (uint8_t*)m->v_zp, (uint8_t*)m->k_zp, (char*)m->tail_k,
                          (char*)m->tail_v};
    a.n = n;
    a.block_size = d->block_size;
    a.num_kv_heads = d->num_kv_heads;
    a.head_dim = d->head_dim;
    a.v_codec = d->v_codec;
    a.k_codec = d->k_codec;
    a.dev_blocks = d->num_blocks;
    a.dev_slots = d->max_seqs;
    a.host_blocks = hd->num_blocks;
    a.host_slots = hd->max_seqs;
    a.chunks = (int32_t)chunks;
    return pbq::hip_status(pbq::launch_swap_blocks(a, (hipStream_t)stream), "kv_swap_blocks launch");
}

kv_status kv_quantize_store(const kv_pool_desc* d, const kv_pool_mem* m,
                            const uint16_t* k, const uint16_t* v,
                            int32_t num_seqs, const int32_t* cu_seqlens,
                            const int32_t* start_pos, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* tail_slots,
                            int32_t max_new_tokens, void* stream) {
    kv_status st = pbq::check_device_desc(d);
    if (st != KV_OK) return st;
    if ((st = pbq::check_mem(d, m, true)) != KV_OK) return st;
    if (num_seqs < 0 || max_new_tokens < 0 || max_blocks_per_seq < 0)
        return fail(KV_ERR_INVALID, "negative size argument");
    if (num_seqs == 0 || max_new_tokens == 0) return KV_OK;
    if (!k || !v || !pbq::aligned16(k) || !pbq::aligned16(v))
        return fail(KV_ERR_INVALID, "k and v must be non-NULL and 16-byte aligned");
    if (!cu_seqlens || !start_pos || !block_tables || !tail_slots)
        return fail(KV_ERR_INVALID, "index arrays must be non-NULL");
    if (max_blocks_per_seq < 1) return fail(KV_ERR_INVALID, "max_blocks_per_seq must be >= 1");
    if (pbq::debug_checks()) {
        std::vector<int32_t> cu, sp, tab, sl;
        const hipStream_t s = (hipStream_t)stream;
        if ((st = pbq::fetch(cu_seqlens, num_seqs + 1, cu, s)) != KV_OK ||
            (st = pbq::fetch(start_pos, num_seqs, sp, s)) != KV_OK ||
            (st = pbq::fetch(block_tables, (size_t)num_seqs * max_blocks_per_seq, tab, s)) != KV_OK ||
            (st = pbq::fetch(tail_slots, num_seqs, sl, s)) != KV_OK)
            return st;
        std::vector<int32_t> end(num_seqs);
        for (int32_t i = 0; i < num_seqs; ++i) end[i] = sp[i] + (cu[i + 1] - cu[i]);
        if ((st = pbq::check_disjoint_writes(d, "kv_quantize_store", tab, max_blocks_per_seq, sp, end, sl)) != KV_OK)
            return st;
    }
    pbq::QuantStoreArgs a{};
    a.block_size = d->block_size;
    a.num_kv_heads = d->num_kv_heads;
    a.head_dim = d->head_dim;
    a.v_codec = d->v_codec;
    a.k_codec = d->k_codec;
    a.k_codes = (int8_t*)m->k_codes;
    a.v_codes = (uint8_t*)m->v_codes;
    a.k_scale = (uint16_t*)m->k_scale;
    a.v_scale = (uint16_t*)m->v_scale;
    a.v_zp = (uint8_t*)m->v_zp;
    a.k_zp = (uint8_t*)m->k_zp;
    a.tail_k = (uint16_t*)m->tail_k;
    a.tail_v = (uint16_t*)m->tail_v;
    a.k = k;
    a.v = v;
    a.num_seqs = num_seqs;
    a.cu_seqlens = cu_seqlens;
    a.start_pos = start_pos;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.tail_slots = tail_slots;
    // a run of n tokens starting anywhere inside a block spans at most
    // ceil((bs - 1 + n) / bs) blocks
    a.tiles_per_seq = pbq::ceil_div((int64_t)d->block_size - 1 + max_new_tokens, d->block_size);
    // launch grid: (KV heads / 4, blocks per sequence, sequences)
    if (a.tiles_per_seq > 65535 || num_seqs > 65535)
        return fail(KV_ERR_INVALID, "store too large for one launch (max_new_tokens / block_size and "
                                    "num_seqs must stay below 65536)");
    return pbq::hip_status(pbq::launch_quantize_store(a, (hipStream_t)stream), "kv_quantize_store launch");
}

}  // extern "C"

namespace {

// The partition policy over `units` work groups per partition.
int32_t partition_for_units(int64_t units, int32_t max_context_len) {
    const int64_t target = 4 * (int64_t)pbq::device_cu_count();
    const int32_t ctx = max_context_len > 0 ? max_context_len : 1;
    // A single pass (no reduce kernel, no workspace) when the units alone give
    // enough work groups and each stays within 4096 tokens; otherwise
    // 2048-token partitions, halved (down to 256) while the grid is too small
    // to fill the GPU.  Partitions are multiples of 32 tokens.
    if (units >= target && ctx <= 4096) return (int32_t)pbq::ceil_div(ctx, 32) * 32;
    int32_t part = 2048;
    while (part > 256 && units * pbq::ceil_div(ctx, part) < target) part /= 2;
    return part;
}

// Multi-query work groups per partition: sequences x KV heads x tiles of 16
// (query token, group head) pairs.
int32_t multi_default_partition(const kv_pool_desc* d, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_q_len, int32_t max_context_len) {
    if (!d || d->num_kv_heads < 1 || num_seqs < 1 || num_q_heads < 1 || max_q_len < 1) return 0;
    const int64_t group = num_q_heads / d->num_kv_heads;
    return partition_for_units((int64_t)num_seqs * d->num_kv_heads * pbq::ceil_div(max_q_len * group, 16),
                               max_context_len);
}

size_t workspace_rows_bytes(const kv_pool_desc* d, int64_t rows_per_part, int32_t max_context_len,
                            int32_t part) {
    if (part <= 0) return 0;
    const int32_t max_parts = max_context_len > 0 ? pbq::ceil_div(max_context_len, part) : 1;
    if (max_parts <= 1) return 0;
    const size_t rows = (size_t)rows_per_part * max_parts;
    return rows * (size_t)d->head_dim * 4 + rows * 8;
}

}  // namespace

extern "C" {

int32_t paged_attn_default_partition(const kv_pool_desc* d, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t max_context_len) {
    if (!d || d->block_size < 1 || d->num_kv_heads < 1 || num_seqs < 1 || num_q_heads < 1) return 0;
    // Work groups: one per (sequence, head) for one query head per KV head,
    // one per (sequence, KV head, tile of 16 query heads) otherwise.
    const int64_t group = num_q_heads / d->num_kv_heads;
    const int64_t units = (int64_t)num_seqs *
                          (group == 1 ? num_q_heads : (int64_t)d->num_kv_heads * pbq::ceil_div(group, 16));
    return partition_for_units(units, max_context_len);
}

size_t paged_attn_multi_query_workspace_bytes(const kv_pool_desc* d, int32_t num_seqs, int32_t num_tokens,
                                              int32_t num_q_heads, int32_t max_q_len,
                                              int32_t max_context_len, int32_t partition_size) {
    if (!d || num_seqs <= 0 || num_tokens <= 0 || num_q_heads <= 0 || max_context_len < 0 || d->head_dim <= 0)
        return 0;
    const int32_t part = partition_size > 0
                             ? partition_size
                             : multi_default_partition(d, num_seqs, num_q_heads, max_q_len, max_context_len);
    return workspace_rows_bytes(d, (int64_t)num_tokens * num_q_heads, max_context_len, part);
}

kv_status paged_attn_multi_query(const kv_pool_desc* d, const kv_pool_mem* m, const uint16_t* q,
                                 uint16_t* out, int32_t num_seqs, int32_t num_q_heads,
                                 const int32_t* cu_seqlens, int32_t num_tokens, int32_t max_q_len,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len, float sm_scale,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    kv_status st = pbq::check_device_desc(d);
    if (st != KV_OK) return st;
    if ((st = pbq::check_mem(d, m, false)) != KV_OK) return st;
    if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0 || max_context_len < 0 || max_blocks_per_seq < 0)
        return fail(KV_ERR_INVALID, "negative size argument");
    if (num_q_heads < 1 || num_q_heads % d->num_kv_heads != 0)
        return fail(KV_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
    const int32_t group = num_q_heads / d->num_kv_heads;
    if (num_seqs == 0 || num_tokens == 0) return KV_OK;
    if (max_q_len < 1 || max_q_len > max_context_len)
        return fail(KV_ERR_INVALID, "max_q_len must be in [1, max_context_len]");
    if (num_seqs > 65535 || num_q_heads > 65535 || max_q_len > 65535)
        return fail(KV_ERR_INVALID, "num_seqs, num_q_heads and max_q_len must stay below 65536");
    if ((int64_t)d->num_kv_heads * pbq::ceil_div((int64_t)max_q_len * group, 16) > 65535)
        return fail(KV_ERR_INVALID, "too many (query token, head) tiles per sequence for the launch grid");
    if (!q || !out || !pbq::aligned16(q) || !pbq::aligned16(out))
        return fail(KV_ERR_INVALID, "q and out must be non-NULL and 16-byte aligned");
    if (!cu_seqlens || !block_tables || !context_lens) return fail(KV_ERR_INVALID, "index arrays must be non-NULL");
    if ((int64_t)max_blocks_per_seq * d->block_size < max_context_len)
        return fail(KV_ERR_INVALID, "max_blocks_per_seq * block_size < max_context_len");
    if (!std::isfinite(sm_scale)) return fail(KV_ERR_INVALID, "sm_scale must be finite");
    int32_t part = partition_size;
    if (part == 0) part = multi_default_partition(d, num_seqs, num_q_heads, max_q_len, max_context_len);
    if (part <= 0 || part % d->block_size != 0 || part % 32 != 0)
        return fail(KV_ERR_INVALID, "partition_size must be a positive multiple of 32 and of block_size (or 0)");
    const int32_t max_parts = pbq::ceil_div(max_context_len, part);
    if (max_parts > 65535) return fail(KV_ERR_INVALID, "too many partitions; use a larger partition_size");
    const size_t need = workspace_rows_bytes(d, (int64_t)num_tokens * num_q_heads, max_context_len, part);
    if (workspace_bytes < need) return fail(KV_ERR_INVALID, "workspace too small");
    if (need > 0 && (!workspace || !pbq::aligned16(workspace)))
        return fail(KV_ERR_INVALID, "workspace must be non-NULL and 16-byte aligned");
    pbq::AttnArgs a{};
    a.block_size = d->block_size;
    a.num_kv_heads = d->num_kv_heads;
    a.head_dim = d->head_dim;
    a.v_codec = d->v_codec;
    a.k_codec = d->k_codec;
    a.k_codes = (const int8_t*)m->k_codes;
    a.v_codes = (const uint8_t*)m->v_codes;
    a.k_scale = (const uint16_t*)m->k_scale;
    a.v_scale = (const uint16_t*)m->v_scale;
    a.v_zp = (const uint8_t*)m->v_zp;
    a.k_zp = (const uint8_t*)m->k_zp;
    a.q = q;
    a.out = out;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.sm_scale = sm_scale;
    a.partition_blocks = part / d->block_size;
    a.max_partitions = max_parts;
    a.cu_q = cu_seqlens;
    a.max_q_len = max_q_len;
    const size_t rows = (size_t)num_tokens * num_q_heads * max_parts;
    a.ws_out = need ? (float*)workspace : nullptr;
    a.ws_ml = need ? (float*)((char*)workspace + rows * (size_t)d->head_dim * 4) : nullptr;
    return pbq::hip_status(pbq::launch_paged_attn(a, (hipStream_t)stream), "paged_attn_multi_query launch");
}

}  // extern "C"

namespace {

// List entries per wavefront of the streaming read: about 16 waves per
// compute unit over the whole list, at least 16 tiles each.
int64_t stream_tiles_per_wave(int64_t n_tiles) {
    const int64_t waves = 16 * (int64_t)pbq::device_cu_count();
    return std::max<int64_t>(16, (n_tiles + waves - 1) / waves);
}

}  // namespace

extern "C" {

size_t kv_stream_read_sink_words(int64_t n_tiles) {
    if (n_tiles <= 0) return 0;
    return (size_t)pbq::stream_read_groups(n_tiles, stream_tiles_per_wave(n_tiles));
}

kv_status kv_stream_read_tiles(const void* src, int64_t n_src_tiles, int32_t tile_bytes, const int32_t* order,
                               int64_t n_tiles, uint32_t* sink, size_t sink_words, void* stream) {
    int sh = -1;
    if (tile_bytes == 1024) sh = 0;
    else if (tile_bytes == 2048) sh = 1;
    else if (tile_bytes == 4096) sh = 2;
    if (sh < 0) return fail(KV_ERR_INVALID, "tile_bytes must be 1024, 2048 or 4096");
    if (n_tiles < 0 || n_src_tiles < 0) return fail(KV_ERR_INVALID, "negative size argument");
    if (n_tiles == 0) return KV_OK;
    if (!src || !sink || !pbq::aligned16(src)) return fail(KV_ERR_INVALID, "src and sink must be non-NULL, src 16-byte aligned");
    if (!order && n_tiles > n_src_tiles) return fail(KV_ERR_INVALID, "n_tiles exceeds n_src_tiles");
    if (n_src_tiles > ((int64_t)1 << 40 >> (10 + sh))) return fail(KV_ERR_INVALID, "source too large");
    const int64_t tpw = stream_tiles_per_wave(n_tiles);
    const int64_t groups = pbq::stream_read_groups(n_tiles, tpw);
    if (groups > 0x7FFFFFFF) return fail(KV_ERR_INVALID, "too many tiles for one launch");
    if (sink_words < (size_t)groups) return fail(KV_ERR_INVALID, "sink too small: see kv_stream_read_sink_words");
    pbq::StreamReadArgs a{};
    a.src = (const uint8_t*)src;
    a.order = order;
    a.n_tiles = n_tiles;
    a.tiles_per_wave = tpw;
    a.tile_kib_log2 = sh;
    a.sink = sink;
    return pbq::hip_status(pbq::launch_stream_read(a, (hipStream_t)stream), "kv_stream_read_tiles launch");
}

size_t paged_attn_workspace_bytes(const kv_pool_desc* d, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len,
                                  int32_t partition_size) {
    if (!d || num_seqs <= 0 || num_q_heads <= 0 || max_context_len < 0 || d->head_dim <= 0)
        return 0;
    int32_t part = partition_size > 0 ? partition_size
                                      : paged_attn_default_partition(d, num_seqs, num_q_heads, max_context_len);
    return workspace_rows_bytes(d, (int64_t)num_seqs * num_q_heads, max_context_len, part);
}

kv_status paged_attn_decode(const kv_pool_desc* d, const kv_pool_mem* m,
                            const uint16_t* q, uint16_t* out, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float sm_scale,
                            int32_t partition_size, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return decode_impl(d, m, nullptr, q, out, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, sm_scale, partition_size, 0, workspace, workspace_bytes,
                       stream);
}

kv_status paged_attn_decode_append(const kv_pool_desc* d, const kv_pool_mem* m,
                                   const uint16_t* k_new, const uint16_t* v_new,
                                   const int32_t* tail_slots, const uint16_t* q, uint16_t* out,
                                   int32_t num_seqs, int32_t num_q_heads,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   float sm_scale, int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    const AppendArgs app{k_new, v_new, tail_slots};
    return decode_impl(d, m, &app, q, out, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, sm_scale, partition_size, 0, workspace, workspace_bytes,
                       stream);
}

kv_status paged_attn_decode_append_noalloc(const kv_pool_desc* d, const kv_pool_mem* m,
                                           const uint16_t* k_new, const uint16_t* v_new,
                                           const int32_t* tail_slots, const uint16_t* q, uint16_t* out,
                                           int32_t num_seqs, int32_t num_q_heads,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t max_context_len,
                                           float sm_scale, int32_t partition_size, void* stream) {
    const AppendArgs app{k_new, v_new, tail_slots};
    return decode_impl(d, m, &app, q, out, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, sm_scale, partition_size, 0, nullptr, 0, stream,
                       /*use_scratch=*/true);
}

kv_status paged_attn_decode_shared_prefix(const kv_pool_desc* d, const kv_pool_mem* m,
                                          const uint16_t* k_new, const uint16_t* v_new,
                                          const int32_t* tail_slots, const uint16_t* q, uint16_t* out,
                                          int32_t num_seqs, int32_t num_q_heads,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t max_context_len,
                                          float sm_scale, int32_t partition_size, int32_t shared_tokens,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    if (!k_new && (v_new || tail_slots))
        return fail(KV_ERR_INVALID, "k_new, v_new and tail_slots are all NULL (plain decode) or all set");
    const AppendArgs app{k_new, v_new, tail_slots};
    return decode_impl(d, m, k_new ? &app : nullptr, q, out, num_seqs, num_q_heads, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, sm_scale, partition_size,
                       shared_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"

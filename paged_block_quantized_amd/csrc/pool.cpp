// Host block-pool allocator: free stack, block tables, reference counts,
// copy-on-write and tail slots.
//
// Policy (web pages cited by site and section):
//  * deepinsea.top "PagedAttention memory management in depth", "paging
//    mechanism design": a request takes ceil(n / block_size) blocks popped
//    from the end of the free list after checking that enough are free (the
//    call fails as a whole otherwise); freeing appends each block back in
//    table order.
//  * tbr8.org "PagedAttention + block-wise quantization against mobile OOM",
//    §5 point 3: blocks are pre-allocated once and carry logical reference
//    counts, so that releasing a conversation only frees unshared blocks.
//  * deepinsea.top "Copy-on-Write" and yunthe.com "PagedAttention mechanism":
//    forked sequences share prefix blocks; only a block about to be modified
//    is copied, and tokens after a fork go to new blocks.
//  * Tail slots (the pages are silent on how a partial block grows): each live
//    sequence owns an fp16 slot with the exact rows of its partially filled
//    last block, so the block can be re-quantized from exact values; a
//    sequence takes the lowest free slot.
//  * yunthe.com "prefix caching": a new request first looks for pool blocks
//    that already hold its prefix and maps them on a hit.  Readings: full
//    blocks only, matched in order from the first until the first miss; a
//    block is identified by its parent block and its own token ids (so a hit
//    means the whole prefix is equal, with no hash collisions to fear); fresh
//    full blocks enter the index when allocated; a block leaves it when its
//    count reaches zero.
//  * deepinsea.top "Swap": when device memory runs short, KV blocks move to
//    a CPU swap space sized in GB.  Readings: the swap space is a second
//    block pool (own free stack popped from its end, own counts) plus host
//    tail slots; a group of sequences swaps out together and moves only the
//    blocks that no sequence outside the group holds (moving any other frees
//    nothing), each once, in first-seen order; swap-in takes fresh device
//    blocks; both are all-or-nothing.  Swapped tables name host block h as
//    -1 - h (and the host slot likewise).  Each call returns the copy plan
//    that kv_swap_blocks runs.
// The pool is single-threaded per handle; no call touches device memory.

#include <stdint.h>

#include <algorithm>
#include <new>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "pbq_internal.h"

struct SeqState {
    std::vector<int32_t> table;  // device block b >= 0, host block h as -1 - h
    int32_t num_tokens = 0;
    int32_t slot = 0;            // device slot, or -1 - host slot when swapped
    bool swapped = false;
};

inline int32_t host_id(int32_t h) { return -1 - h; }

// Prefix-cache key of a block: the block before it (-1 for the first) and
// its bs token ids.  The index maps a hash of the key to candidate blocks;
// a candidate is a hit only if its stored key is equal.
uint64_t prefix_hash(int32_t parent, const int32_t* ids, int64_t n) {
    uint64_t h = 1469598103934665603ull ^ (uint32_t)parent;   // FNV-1a over the words
    for (int64_t i = 0; i < n; ++i) h = (h ^ (uint32_t)ids[i]) * 1099511628211ull;
    return h;
}

struct kv_pool {
    kv_pool_desc desc{};
    std::vector<int32_t> free_stack;  // popped from the back
    std::vector<int32_t> refcount;
    std::unordered_map<int64_t, SeqState> seqs;
    std::set<int32_t> free_slots;
    std::unordered_multimap<uint64_t, int32_t> prefix_index;   // key hash -> block
    std::vector<uint8_t> indexed;     // per block: in the index
    std::vector<int32_t> key_parent;  // per block: key parent
    std::vector<int32_t> key_ids;     // per block: bs key ids
    std::vector<uint64_t> key_hash;   // per block: key hash
    int32_t n_indexed = 0;
    // swap space
    std::vector<int32_t> host_free_stack;
    std::vector<int32_t> host_refcount;
    std::set<int32_t> host_free_slots;
    int32_t n_swapped = 0;

    // drop n references to device block b; at zero it goes back on the free
    // stack and leaves the prefix index
    void release_block(int32_t b, int32_t n) {
        refcount[b] -= n;
        if (refcount[b] == 0) {
            free_stack.push_back(b);
            if (indexed[b]) leave(b);
        }
    }

    bool key_equal(int32_t b, int32_t parent, const int32_t* ids) const {
        const int64_t bs = desc.block_size;
        return key_parent[b] == parent && std::equal(ids, ids + bs, key_ids.begin() + b * bs);
    }
    int32_t find(int32_t parent, const int32_t* ids) const {
        auto r = prefix_index.equal_range(prefix_hash(parent, ids, desc.block_size));
        for (auto it = r.first; it != r.second; ++it)
            if (key_equal(it->second, parent, ids)) return it->second;
        return -1;
    }
    void enter(int32_t b, int32_t parent, const int32_t* ids) {
        const int64_t bs = desc.block_size;
        key_parent[b] = parent;
        std::copy(ids, ids + bs, key_ids.begin() + b * bs);
        key_hash[b] = prefix_hash(parent, ids, bs);
        prefix_index.emplace(key_hash[b], b);
        indexed[b] = 1;
        ++n_indexed;
    }
    void leave(int32_t b) {
        auto r = prefix_index.equal_range(key_hash[b]);
        for (auto it = r.first; it != r.second; ++it)
            if (it->second == b) {
                prefix_index.erase(it);
                break;
            }
        indexed[b] = 0;
        --n_indexed;
    }
};

namespace {

int64_t blocks_for(int64_t n, int64_t bs) { return (n + bs - 1) / bs; }

kv_status check_host_desc(const kv_pool_desc* d) {
    if (!d) return pbq::fail(KV_ERR_INVALID, "desc is NULL");
    if (d->num_blocks < 1) return pbq::fail(KV_ERR_INVALID, "num_blocks must be >= 1");
    if (d->block_size < 1) return pbq::fail(KV_ERR_INVALID, "block_size must be >= 1");
    if (d->max_seqs < 1) return pbq::fail(KV_ERR_INVALID, "max_seqs must be >= 1");
    if (d->num_kv_heads < 1 || d->head_dim < 1)
        return pbq::fail(KV_ERR_INVALID, "num_kv_heads and head_dim must be >= 1");
    return KV_OK;
}

}  // namespace

extern "C" {

kv_status kv_pool_create(const kv_pool_desc* desc, const int32_t* free_order,
                         kv_pool** out) {
    if (!out) return pbq::fail(KV_ERR_INVALID, "out is NULL");
    *out = nullptr;
    kv_status st = check_host_desc(desc);
    if (st != KV_OK) return st;
    const int32_t n = desc->num_blocks;
    std::vector<int32_t> order(n);
    if (free_order) {
        std::vector<uint8_t> seen(n, 0);
        for (int32_t i = 0; i < n; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= n || seen[b])
                return pbq::fail(KV_ERR_INVALID, "free_order is not a permutation of 0..N-1");
            seen[b] = 1;
            order[i] = b;
        }
    } else {
        for (int32_t i = 0; i < n; ++i) order[i] = i;
    }
    kv_pool* p = new (std::nothrow) kv_pool();
    if (!p) return pbq::fail(KV_ERR_INVALID, "out of host memory");
    p->desc = *desc;
    p->free_stack = std::move(order);
    p->refcount.assign(n, 0);
    p->indexed.assign(n, 0);
    p->key_parent.assign(n, -1);
    p->key_ids.assign((size_t)n * desc->block_size, 0);
    p->key_hash.assign(n, 0);
    p->prefix_index.reserve(n);
    for (int32_t s = 0; s < desc->max_seqs; ++s) p->free_slots.insert(s);
    *out = p;
    return KV_OK;
}

void kv_pool_destroy(kv_pool* pool) { delete pool; }

kv_status kv_seq_alloc(kv_pool* pool, int64_t seq, int32_t num_tokens) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    if (num_tokens < 0) return pbq::fail(KV_ERR_INVALID, "num_tokens < 0");
    if (pool->seqs.count(seq)) return pbq::fail(KV_ERR_STATE, "sequence already present");
    if (pool->free_slots.empty()) return pbq::fail(KV_ERR_NO_SLOTS, "no free tail slot");
    const int64_t need = blocks_for(num_tokens, pool->desc.block_size);
    if (need > (int64_t)pool->free_stack.size())
        return pbq::fail(KV_ERR_NO_BLOCKS, "not enough free blocks");
    SeqState st;
    st.table.reserve(need);
    for (int64_t i = 0; i < need; ++i) {
        int32_t b = pool->free_stack.back();
        pool->free_stack.pop_back();
        pool->refcount[b] = 1;
        st.table.push_back(b);
    }
    st.num_tokens = num_tokens;
    st.slot = *pool->free_slots.begin();
    pool->free_slots.erase(pool->free_slots.begin());
    pool->seqs.emplace(seq, std::move(st));
    return KV_OK;
}

kv_status kv_seq_alloc_prefix(kv_pool* pool, int64_t seq, const int32_t* token_ids,
                              int32_t num_tokens, int32_t* cached_tokens) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    if (num_tokens < 0) return pbq::fail(KV_ERR_INVALID, "num_tokens < 0");
    if (num_tokens > 0 && !token_ids) return pbq::fail(KV_ERR_INVALID, "token_ids is NULL");
    if (pool->seqs.count(seq)) return pbq::fail(KV_ERR_STATE, "sequence already present");
    if (pool->free_slots.empty()) return pbq::fail(KV_ERR_NO_SLOTS, "no free tail slot");
    const int64_t bs = pool->desc.block_size;
    const int64_t need = blocks_for(num_tokens, bs);
    std::vector<int32_t> hits;
    int32_t parent = -1;
    for (int64_t j = 0; j < num_tokens / bs; ++j) {
        const int32_t b = pool->find(parent, token_ids + j * bs);
        if (b < 0) break;
        hits.push_back(b);
        parent = b;
    }
    if (need - (int64_t)hits.size() > (int64_t)pool->free_stack.size())
        return pbq::fail(KV_ERR_NO_BLOCKS, "not enough free blocks");
    SeqState st;
    st.table = hits;
    for (int32_t b : hits) pool->refcount[b] += 1;
    for (int64_t j = (int64_t)hits.size(); j < need; ++j) {
        int32_t b = pool->free_stack.back();
        pool->free_stack.pop_back();
        pool->refcount[b] = 1;
        if ((j + 1) * bs <= num_tokens)   // a full block enters the index
            pool->enter(b, j > 0 ? st.table[j - 1] : -1, token_ids + j * bs);
        st.table.push_back(b);
    }
    st.num_tokens = num_tokens;
    st.slot = *pool->free_slots.begin();
    pool->free_slots.erase(pool->free_slots.begin());
    pool->seqs.emplace(seq, std::move(st));
    if (cached_tokens) *cached_tokens = (int32_t)(hits.size() * bs);
    return KV_OK;
}

kv_status kv_seq_fork(kv_pool* pool, int64_t parent, int64_t child,
                      kv_copy* copies, int32_t cap, int32_t* n_copies) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    auto it = pool->seqs.find(parent);
    if (it == pool->seqs.end()) return pbq::fail(KV_ERR_UNKNOWN_SEQ, "unknown parent");
    if (pool->seqs.count(child)) return pbq::fail(KV_ERR_STATE, "child already present");
    if (it->second.swapped) return pbq::fail(KV_ERR_STATE, "parent is swapped out");
    if (pool->free_slots.empty()) return pbq::fail(KV_ERR_NO_SLOTS, "no free tail slot");
    const SeqState& p = it->second;
    const bool partial = p.num_tokens % pool->desc.block_size != 0;
    if (partial && (cap < 1 || !copies))
        return pbq::fail(KV_ERR_INVALID, "fork needs room for one copy (cap >= 1)");
    SeqState c;
    c.table = p.table;
    c.num_tokens = p.num_tokens;
    c.slot = *pool->free_slots.begin();
    pool->free_slots.erase(pool->free_slots.begin());
    for (int32_t b : c.table) pool->refcount[b] += 1;
    int32_t n = 0;
    if (partial) copies[n++] = kv_copy{KV_COPY_SLOT, p.slot, c.slot};
    if (n_copies) *n_copies = n;
    pool->seqs.emplace(child, std::move(c));
    return KV_OK;
}

kv_status kv_seq_append(kv_pool* pool, int64_t seq, int32_t n_tokens,
                        kv_copy* copies, int32_t cap, int32_t* n_copies) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    if (n_tokens < 0) return pbq::fail(KV_ERR_INVALID, "n_tokens < 0");
    auto it = pool->seqs.find(seq);
    if (it == pool->seqs.end()) return pbq::fail(KV_ERR_UNKNOWN_SEQ, "unknown sequence");
    SeqState& st = it->second;
    if (st.swapped) return pbq::fail(KV_ERR_STATE, "sequence is swapped out");
    const int64_t bs = pool->desc.block_size;
    const int64_t ntok = st.num_tokens;
    if (ntok + (int64_t)n_tokens > INT32_MAX)
        return pbq::fail(KV_ERR_INVALID, "token count overflows int32");
    const bool cow = n_tokens > 0 && ntok % bs != 0 && pool->refcount[st.table.back()] > 1;
    // positions p in [ntok, ntok + n) with p % bs == 0
    const int64_t boundaries = blocks_for(ntok + n_tokens, bs) - blocks_for(ntok, bs);
    if ((cow ? 1 : 0) + boundaries > (int64_t)pool->free_stack.size())
        return pbq::fail(KV_ERR_NO_BLOCKS, "not enough free blocks");
    if (cow && (cap < 1 || !copies))
        return pbq::fail(KV_ERR_INVALID, "append needs room for one copy (cap >= 1)");
    int32_t n = 0;
    if (cow) {
        int32_t src = st.table.back();
        int32_t dst = pool->free_stack.back();
        pool->free_stack.pop_back();
        pool->refcount[src] -= 1;
        pool->refcount[dst] = 1;
        st.table.back() = dst;
        copies[n++] = kv_copy{KV_COPY_BLOCK, src, dst};
    }
    for (int64_t i = 0; i < boundaries; ++i) {
        int32_t b = pool->free_stack.back();
        pool->free_stack.pop_back();
        pool->refcount[b] = 1;
        st.table.push_back(b);
    }
    st.num_tokens = (int32_t)(ntok + n_tokens);
    if (n_copies) *n_copies = n;
    return KV_OK;
}

kv_status kv_seq_free(kv_pool* pool, int64_t seq) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    auto it = pool->seqs.find(seq);
    if (it == pool->seqs.end()) return pbq::fail(KV_ERR_UNKNOWN_SEQ, "unknown sequence");
    for (int32_t b : it->second.table) {
        if (b >= 0) {
            pool->release_block(b, 1);
        } else if (--pool->host_refcount[host_id(b)] == 0) {
            pool->host_free_stack.push_back(host_id(b));
        }
    }
    if (it->second.swapped) {
        pool->host_free_slots.insert(host_id(it->second.slot));
        pool->n_swapped -= 1;
    } else {
        pool->free_slots.insert(it->second.slot);
    }
    pool->seqs.erase(it);
    return KV_OK;
}

kv_status kv_seq_table(const kv_pool* pool, int64_t seq, int32_t* out,
                       int32_t cap, int32_t* n_blocks, int32_t* n_tokens,
                       int32_t* slot) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    auto it = pool->seqs.find(seq);
    if (it == pool->seqs.end()) return pbq::fail(KV_ERR_UNKNOWN_SEQ, "unknown sequence");
    const SeqState& st = it->second;
    const int32_t nb = (int32_t)st.table.size();
    if (out) {
        if (cap < nb) return pbq::fail(KV_ERR_INVALID, "cap smaller than the table");
        std::copy(st.table.begin(), st.table.end(), out);
    }
    if (n_blocks) *n_blocks = nb;
    if (n_tokens) *n_tokens = st.num_tokens;
    if (slot) *slot = st.slot;
    return KV_OK;
}

kv_status kv_batch_tables(const kv_pool* pool, const int64_t* seqs, int32_t n,
                          int32_t* tables, int32_t max_blocks,
                          int32_t* ctx_lens, int32_t* slots) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    if (n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables)))
        return pbq::fail(KV_ERR_INVALID, "bad batch arguments");
    for (int32_t i = 0; i < n; ++i) {  // validate first: no partial output
        auto it = pool->seqs.find(seqs[i]);
        if (it == pool->seqs.end()) return pbq::fail(KV_ERR_UNKNOWN_SEQ, "unknown sequence");
        if (it->second.swapped) return pbq::fail(KV_ERR_STATE, "sequence is swapped out");
        if ((int64_t)it->second.table.size() > max_blocks)
            return pbq::fail(KV_ERR_INVALID, "a table needs more than max_blocks entries");
    }
    for (int32_t i = 0; i < n; ++i) {
        const SeqState& st = pool->seqs.find(seqs[i])->second;
        int32_t* row = tables + (int64_t)i * max_blocks;
        std::fill(row, row + max_blocks, 0);
        std::copy(st.table.begin(), st.table.end(), row);
        if (ctx_lens) ctx_lens[i] = st.num_tokens;
        if (slots) slots[i] = st.slot;
    }
    return KV_OK;
}

kv_status kv_pool_stats(const kv_pool* pool, kv_pool_stats_t* out) {
    if (!pool || !out) return pbq::fail(KV_ERR_INVALID, "NULL argument");
    int32_t used = 0, shared = 0;
    for (int32_t r : pool->refcount) {
        used += r > 0;
        shared += r > 1;
    }
    out->total = pool->desc.num_blocks;
    out->free = (int32_t)pool->free_stack.size();
    out->used = used;
    out->shared = shared;
    out->seqs = (int32_t)pool->seqs.size();
    out->cached = pool->n_indexed;
    out->host_total = (int32_t)pool->host_refcount.size();
    out->host_free = (int32_t)pool->host_free_stack.size();
    out->swapped = pool->n_swapped;
    return KV_OK;
}

kv_status kv_pool_free_list(const kv_pool* pool, int32_t* out, int32_t cap,
                            int32_t* n) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    const int32_t sz = (int32_t)pool->free_stack.size();
    if (out) {
        if (cap < sz) return pbq::fail(KV_ERR_INVALID, "cap smaller than the free list");
        std::copy(pool->free_stack.begin(), pool->free_stack.end(), out);
    }
    if (n) *n = sz;
    return KV_OK;
}

kv_status kv_pool_set_swap_space(kv_pool* pool, int32_t host_blocks, int32_t host_slots) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    if (host_blocks < 0 || host_slots < 0)
        return pbq::fail(KV_ERR_INVALID, "swap space sizes must be >= 0");
    if (pool->n_swapped > 0) return pbq::fail(KV_ERR_STATE, "sequences are swapped out");
    pool->host_free_stack.resize(host_blocks);
    for (int32_t h = 0; h < host_blocks; ++h) pool->host_free_stack[h] = h;
    pool->host_refcount.assign(host_blocks, 0);
    pool->host_free_slots.clear();
    for (int32_t k = 0; k < host_slots; ++k) pool->host_free_slots.insert(k);
    return KV_OK;
}

namespace {

// Checks a swap group: no repeats, every sequence known and in the wanted
// place (resident for swap-out, swapped for swap-in).
kv_status check_group(const kv_pool* pool, const int64_t* seqs, int32_t n, bool want_swapped,
                      int32_t* plan_cap, kv_swap* plan) {
    if (n < 0 || (n > 0 && !seqs)) return pbq::fail(KV_ERR_INVALID, "bad sequence list");
    if (*plan_cap < 0 || (*plan_cap > 0 && !plan)) return pbq::fail(KV_ERR_INVALID, "bad plan buffer");
    std::vector<int64_t> sorted(seqs, seqs + n);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
        return pbq::fail(KV_ERR_INVALID, "a sequence is named twice");
    for (int32_t i = 0; i < n; ++i)
        if (!pool->seqs.count(seqs[i])) return pbq::fail(KV_ERR_UNKNOWN_SEQ, "unknown sequence");
    for (int32_t i = 0; i < n; ++i)
        if (pool->seqs.find(seqs[i])->second.swapped != want_swapped)
            return pbq::fail(KV_ERR_STATE, want_swapped ? "sequence is not swapped out"
                                                        : "sequence is swapped out");
    return KV_OK;
}

// Distinct table entries of the group in first-seen order with the number
// of references the group holds to each: host entries (< 0) when `host`,
// device entries otherwise.
void group_refs(const kv_pool* pool, const int64_t* seqs, int32_t n, bool host,
                std::vector<int32_t>& order, std::unordered_map<int32_t, int32_t>& count) {
    for (int32_t i = 0; i < n; ++i)
        for (int32_t b : pool->seqs.find(seqs[i])->second.table) {
            if ((b < 0) != host) continue;
            auto r = count.emplace(b, 0);
            if (r.second) order.push_back(b);
            r.first->second += 1;
        }
}

}  // namespace

kv_status kv_seq_swap_out(kv_pool* pool, const int64_t* seqs, int32_t n, kv_swap* plan,
                          int32_t cap, int32_t* n_plan) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    kv_status st = check_group(pool, seqs, n, false, &cap, plan);
    if (st != KV_OK) return st;
    std::vector<int32_t> order;
    std::unordered_map<int32_t, int32_t> count;
    group_refs(pool, seqs, n, false, order, count);
    std::vector<int32_t> moving;
    for (int32_t b : order)
        if (count[b] == pool->refcount[b]) moving.push_back(b);
    if ((int64_t)pool->host_free_slots.size() < n)
        return pbq::fail(KV_ERR_NO_SLOTS, "no free host slot");
    if (moving.size() > pool->host_free_stack.size())
        return pbq::fail(KV_ERR_NO_BLOCKS, "not enough free host blocks");
    const int32_t bs = pool->desc.block_size;
    int64_t entries = (int64_t)moving.size();
    for (int32_t i = 0; i < n; ++i) entries += pool->seqs.find(seqs[i])->second.num_tokens % bs != 0;
    if (entries > cap) return pbq::fail(KV_ERR_INVALID, "plan buffer too small (cap)");
    int32_t k = 0;
    std::unordered_map<int32_t, int32_t> where;
    for (int32_t b : moving) {
        const int32_t h = pool->host_free_stack.back();
        pool->host_free_stack.pop_back();
        pool->host_refcount[h] = count[b];
        pool->release_block(b, count[b]);
        where[b] = h;
        plan[k++] = kv_swap{KV_SWAP_BLOCK_OUT, b, h, 0};
    }
    for (int32_t i = 0; i < n; ++i) {
        SeqState& s = pool->seqs.find(seqs[i])->second;
        const int32_t hs = *pool->host_free_slots.begin();
        pool->host_free_slots.erase(pool->host_free_slots.begin());
        const int32_t rows = s.num_tokens % bs;
        if (rows) plan[k++] = kv_swap{KV_SWAP_SLOT_OUT, s.slot, hs, rows};
        pool->free_slots.insert(s.slot);
        for (int32_t& b : s.table) {
            auto w = where.find(b);
            if (w != where.end()) b = host_id(w->second);
        }
        s.slot = host_id(hs);
        s.swapped = true;
        pool->n_swapped += 1;
    }
    if (n_plan) *n_plan = k;
    return KV_OK;
}

kv_status kv_seq_swap_in(kv_pool* pool, const int64_t* seqs, int32_t n, kv_swap* plan,
                         int32_t cap, int32_t* n_plan) {
    if (!pool) return pbq::fail(KV_ERR_INVALID, "pool is NULL");
    kv_status st = check_group(pool, seqs, n, true, &cap, plan);
    if (st != KV_OK) return st;
    std::vector<int32_t> order;
    std::unordered_map<int32_t, int32_t> count;
    group_refs(pool, seqs, n, true, order, count);
    if ((int64_t)pool->free_slots.size() < n) return pbq::fail(KV_ERR_NO_SLOTS, "no free tail slot");
    if (order.size() > pool->free_stack.size())
        return pbq::fail(KV_ERR_NO_BLOCKS, "not enough free blocks");
    const int32_t bs = pool->desc.block_size;
    int64_t entries = (int64_t)order.size();
    for (int32_t i = 0; i < n; ++i) entries += pool->seqs.find(seqs[i])->second.num_tokens % bs != 0;
    if (entries > cap) return pbq::fail(KV_ERR_INVALID, "plan buffer too small (cap)");
    int32_t k = 0;
    std::unordered_map<int32_t, int32_t> where;
    for (int32_t e : order) {
        const int32_t h = host_id(e);
        const int32_t d = pool->free_stack.back();
        pool->free_stack.pop_back();
        pool->refcount[d] = count[e];
        pool->host_refcount[h] -= count[e];
        if (pool->host_refcount[h] == 0) pool->host_free_stack.push_back(h);
        where[e] = d;
        plan[k++] = kv_swap{KV_SWAP_BLOCK_IN, h, d, 0};
    }
    for (int32_t i = 0; i < n; ++i) {
        SeqState& s = pool->seqs.find(seqs[i])->second;
        const int32_t hs = host_id(s.slot);
        const int32_t slot = *pool->free_slots.begin();
        pool->free_slots.erase(pool->free_slots.begin());
        const int32_t rows = s.num_tokens % bs;
        if (rows) plan[k++] = kv_swap{KV_SWAP_SLOT_IN, hs, slot, rows};
        pool->host_free_slots.insert(hs);
        for (int32_t& b : s.table)
            if (b < 0) b = where[b];
        s.slot = slot;
        s.swapped = false;
        pool->n_swapped -= 1;
    }
    if (n_plan) *n_plan = k;
    return KV_OK;
}

}  // extern "C"

/*
 * pbq.h -- C ABI of libpbq: PagedAttention decode over a block-quantized KV
 * cache on one MI355X (gfx950).
 *
 * Sources (web pages, cited by site and section):
 *   [tbr8]      tbr8.org, "How PagedAttention combined with block-wise
 *               quantization solves long-text OOM caused by memory
 *               fragmentation on mobile": §2 block virtualisation, §3
 *               block-wise quantization, §4 the PagedKVCacheManager code
 *               (pool tensors, allocate_for_request, store_kv), §5 advice
 *               (INT8 K / INT4 V, fused QuantizedPagedAttention, pre-allocated
 *               pool with reference counts).
 *   [deepinsea] deepinsea.top, "PagedAttention memory management in depth":
 *               "paging mechanism design" (BlockManager allocate/free),
 *               "Copy-on-Write".
 *   [yunthe]    yunthe.com, "KV-cache quantization and PagedAttention":
 *               "quantization principle" (Q(x) and dequantization formulas),
 *               "PagedAttention mechanism" (block_size, num_blocks sizing,
 *               block_table, prefix sharing, fork writes to new blocks).
 *
 * Conventions for every entry point
 *   - Every call returns kv_status; nothing is thrown or aborted across the
 *     boundary.  On failure kv_last_error() returns a message for the calling
 *     thread.  A failed host call leaves all state unchanged.
 *   - Pointers named *_dev are device pointers (hipMalloc / torch CUDA
 *     memory); all other pointers are host pointers.  The caller owns all
 *     memory, device and host, and the stream.  The library never allocates
 *     device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously on it; the call returns after
 *     enqueueing.  Launch failures return KV_ERR_HIP.
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - A kv_pool handle is not thread-safe: calls on one pool must not
 *     overlap.  Distinct pools are independent.
 */
#ifndef PBQ_H
#define PBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv_status {
    KV_OK = 0,
    KV_ERR_INVALID = 1,     /* bad argument (shape, alignment, size, range) */
    KV_ERR_NO_BLOCKS = 2,   /* not enough free blocks; nothing was taken */
    KV_ERR_UNKNOWN_SEQ = 3, /* sequence id not present */
    KV_ERR_STATE = 4,       /* sequence id already present */
    KV_ERR_NO_SLOTS = 5,    /* every tail slot is in use (max_seqs live) */
    KV_ERR_HIP = 6          /* a HIP launch or runtime call failed */
} kv_status;

/* Codecs, one per (block, head) tile of block_size x head_dim values.
 * Supported (k_codec, v_codec) pairs: (I8_SYM, I8_SYM), (I8_SYM, I4_ASYM),
 * (I8_SYM, I8_ASYM), (FP8_E4M3, FP8_E4M3), (I4_ASYM, I4_ASYM) and
 * (I4_ASYM, I8_SYM).
 * INT4 packing is along the tile's contiguous axis: tokens for V, head dims
 * for K (see the layout under kv_pool_sizes).  INT4 K follows [tbr8] §3 (a
 * block may go to INT8 or even INT4) with [yunthe] Q(x), bits = 4.
 *   KV_CODEC_I8_SYM : int8 codes in [-127, 127], fp16 scale = fp16(absmax/127)
 *                     over the rows the block holds; code = round-half-even
 *                     of the fp32 quotient x / scale, clamped.  This is
 *                     [yunthe] Q(x) with bits = 8 and zero point 128, stored
 *                     as Q - 128; [tbr8] §4 store_kv's absmax/127 scale.
 *   KV_CODEC_I4_ASYM: codes in [0, 15], two per byte (the lower index in the
 *                     low nibble); lo = min(0, min x),
 *                     hi = max(0, max x), scale = fp16((hi - lo) / 15),
 *                     zero point = clamp(round(-lo / scale), 0, 15) as u8;
 *                     code = clamp(round(x / scale + zero point), 0, 15)
 *                     ([yunthe] Q(x) with bits = 4).
 *   A block whose statistics give scale 0 stores scale 0, zero point 0 and
 *   all-zero codes.  Rows a block does not hold yet are zero bytes.
 *   KV_CODEC_FP8_E4M3: OCP FP8 E4M3 bytes (4 exponent bits of bias 7, 3
 *                     mantissa bits, largest finite 448) with an fp16 scale
 *                     = fp16(absmax / 448) over the rows held; code = E4M3 of
 *                     the fp32 quotient x / scale, nearest with ties to the
 *                     even code, saturated at +-448; x_hat = value * scale.
 *                     [yunthe] "vLLM deployment" names the format for the
 *                     cache; the scale granularity is this library's.
 *   KV_CODEC_I8_ASYM : u8 codes in [0, 255] with scale and zero point as
 *                     I4_ASYM with 255 levels ([yunthe] Q(x), bits = 8); V only.
 *   Dequantization is ([yunthe]) x_hat = (code - zero point) * scale. */
typedef enum kv_codec {
    KV_CODEC_I8_SYM = 0,
    KV_CODEC_I4_ASYM = 1,
    KV_CODEC_FP8_E4M3 = 2,
    KV_CODEC_I8_ASYM = 3
} kv_codec;

/* Shape of one layer's block pool ([tbr8] §4 PagedKVCacheManager.__init__). */
typedef struct kv_pool_desc {
    int32_t num_blocks;   /* N physical blocks, >= 1 */
    int32_t block_size;   /* tokens per block: 16 or 32 ([tbr8] §2) */
    int32_t num_kv_heads; /* Hkv >= 1 */
    int32_t head_dim;     /* D: 64 or 128 */
    int32_t k_codec;      /* KV_CODEC_I8_SYM ([tbr8] §5: K in INT8), FP8_E4M3 or I4_ASYM */
    int32_t v_codec;      /* I8_SYM, I4_ASYM, I8_ASYM or FP8_E4M3 (pairs above) */
    int32_t max_seqs;     /* tail slots = most sequences alive at once, >= 1 */
} kv_pool_desc;

/* Byte sizes of the device arrays of one pool (all row-major):
 *   k_codes  int8  [N, Hkv, bs, D]      token-major K tiles ([tbr8] §4;
 *                                        u8 E4M3 bytes for FP8_E4M3)
 *            uint8 [N, Hkv, bs, D / 2]  (I4_ASYM K: two consecutive head
 *                                        dims of a token per byte, the even
 *                                        dim in the low nibble)
 *   v_codes  int8  [N, Hkv, D, bs]      (I8_SYM; u8 for I8_ASYM and FP8_E4M3)
 *                                        dim-major V tiles
 *            uint8 [N, Hkv, D, bs / 2]  (I4_ASYM, two consecutive tokens per
 *                                        byte, the earlier in the low nibble)
 *            The pages show only the K pool; V is stored dim-major so that a
 *            sum over a block's tokens reads one contiguous row per dim.
 *   k_scale  fp16  [N, Hkv]
 *   v_scale  fp16  [N, Hkv]
 *   v_zp     uint8 [N, Hkv]  (0 bytes unless I4_ASYM or I8_ASYM)
 *   tail_k   fp16  [max_seqs, Hkv, bs, D]  exact rows of each sequence's
 *   tail_v   fp16  [max_seqs, Hkv, bs, D]  partially filled last block
 *   k_zp     uint8 [N, Hkv]  (0 bytes unless K is I4_ASYM)
 * Every array must be 16-byte aligned. */
typedef struct kv_pool_sizes {
    size_t k_codes, v_codes, k_scale, v_scale, v_zp, tail_k, tail_v, k_zp;
} kv_pool_sizes;

/* Device pointers to the arrays above (v_zp and k_zp may be NULL when V,
 * or K, has no zero point). */
typedef struct kv_pool_mem {
    void* k_codes;
    void* v_codes;
    void* k_scale;
    void* v_scale;
    void* v_zp;
    void* tail_k;
    void* tail_v;
    void* k_zp;
} kv_pool_mem;

/* A copy the caller must perform on the device before writing new tokens
 * (copy-on-write, [deepinsea] "Copy-on-Write"; [yunthe] fork).
 *   kind KV_COPY_BLOCK: codes, scales and zero point of block src -> dst.
 *   kind KV_COPY_SLOT : fp16 tail slot src -> dst (K and V). */
enum { KV_COPY_BLOCK = 0, KV_COPY_SLOT = 1 };
typedef struct kv_copy {
    int32_t kind;
    int32_t src;
    int32_t dst;
} kv_copy;

/* One entry of a swap plan (kv_seq_swap_out / kv_seq_swap_in write them,
 * kv_swap_blocks performs them):
 *   KV_SWAP_BLOCK_OUT: device block src -> host block dst (codes, scales,
 *                      zero points; rows 0)
 *   KV_SWAP_BLOCK_IN : host block src -> device block dst (rows 0)
 *   KV_SWAP_SLOT_OUT : the first `rows` fp16 rows of every head of device
 *                      tail slot src -> host slot dst (K and V)
 *   KV_SWAP_SLOT_IN  : the same from host slot src to device tail slot dst */
enum { KV_SWAP_BLOCK_OUT = 0, KV_SWAP_BLOCK_IN = 1, KV_SWAP_SLOT_OUT = 2, KV_SWAP_SLOT_IN = 3 };
typedef struct kv_swap {
    int32_t kind;
    int32_t src;
    int32_t dst;
    int32_t rows;
} kv_swap;

typedef struct kv_pool_stats_t {
    int32_t total;      /* N */
    int32_t free;       /* blocks on the free stack */
    int32_t used;       /* blocks with refcount > 0 */
    int32_t shared;     /* blocks with refcount > 1 */
    int32_t seqs;       /* live sequences (resident and swapped) */
    int32_t cached;     /* full blocks in the prefix-cache index */
    int32_t host_total; /* blocks of the swap space */
    int32_t host_free;  /* swap-space blocks on its free stack */
    int32_t swapped;    /* sequences swapped out */
} kv_pool_stats_t;

typedef struct kv_pool kv_pool; /* opaque host state */

/* ---- sizing ------------------------------------------------------------
 * Fills *out with the byte size of every device array for desc (the
 * per-block form of [yunthe] "PagedAttention mechanism": num_blocks =
 * memory / bytes per block).  KV_ERR_INVALID if desc is not supported. */
kv_status kv_pool_bytes(const kv_pool_desc* desc, kv_pool_sizes* out);

/* ---- host allocator ([deepinsea] "paging mechanism design"; [tbr8] §4, §5)
 * The free list is a stack popped from its end.  It starts as free_order
 * (a permutation of 0..N-1, length N) or 0..N-1 when free_order is NULL.
 * KV_ERR_INVALID for a bad desc or a free_order that is not a permutation. */
kv_status kv_pool_create(const kv_pool_desc* desc, const int32_t* free_order,
                         kv_pool** out);
void kv_pool_destroy(kv_pool* pool); /* NULL is ignored */

/* Reserve ceil(num_tokens / bs) blocks (refcount 1) and the lowest free tail
 * slot for a new sequence.  All-or-nothing: KV_ERR_NO_BLOCKS /
 * KV_ERR_NO_SLOTS leave the pool unchanged; KV_ERR_STATE if seq exists;
 * KV_ERR_INVALID if num_tokens < 0. */
kv_status kv_seq_alloc(kv_pool* pool, int64_t seq, int32_t num_tokens);

/* kv_seq_alloc for a request whose token ids are known ([yunthe] "prefix
 * caching": blocks of the pool that already hold the request's prefix are
 * mapped instead of recomputed).  Full blocks j = 0, 1, ... are looked up in
 * order, each by (the physical block before it, its block_size token ids),
 * until the first miss; hits are shared (refcount + 1).  The remaining blocks
 * come from the free stack as in kv_seq_alloc, and each fresh full block is
 * entered in the index at once; the partial last block is private.  A block
 * leaves the index when its count reaches zero.  *cached_tokens (may be NULL)
 * receives the number of leading tokens whose codes are already in the pool
 * (hits x block_size): the caller stores positions cached_tokens ..
 * num_tokens - 1 (kv_quantize_store with start_pos = cached_tokens) before
 * any decode reads this or another sequence's fresh blocks.  token_ids:
 * host int32 [num_tokens] (NULL when 0).  Errors as kv_seq_alloc, all-or-
 * nothing. */
kv_status kv_seq_alloc_prefix(kv_pool* pool, int64_t seq, const int32_t* token_ids,
                              int32_t num_tokens, int32_t* cached_tokens);

/* child shares every block of parent (refcount + 1 each) and takes the lowest
 * free tail slot.  If parent's last block is partial, one KV_COPY_SLOT
 * (parent slot -> child slot) is written to copies[0] (cap >= 1 required
 * then).  *n_copies receives the count (0 or 1). */
kv_status kv_seq_fork(kv_pool* pool, int64_t parent, int64_t child,
                      kv_copy* copies, int32_t cap, int32_t* n_copies);

/* Reserve n_tokens more positions.  If the last block is partial and shared,
 * it is first replaced by a fresh block and one KV_COPY_BLOCK (old -> new) is
 * reported; every position on a block boundary takes a fresh block.
 * All-or-nothing (KV_ERR_NO_BLOCKS).  cap >= 1 is always enough. */
kv_status kv_seq_append(kv_pool* pool, int64_t seq, int32_t n_tokens,
                        kv_copy* copies, int32_t cap, int32_t* n_copies);

/* Decrement every block of seq in table order; blocks reaching 0 are pushed
 * on the free stack at once.  Releases the tail slot. */
kv_status kv_seq_free(kv_pool* pool, int64_t seq);

/* Host copy of seq's block table (cap entries available in out; out may be
 * NULL with cap 0 to query), its token count and tail slot.  Any of the
 * output pointers may be NULL. */
kv_status kv_seq_table(const kv_pool* pool, int64_t seq, int32_t* out,
                       int32_t cap, int32_t* n_blocks, int32_t* n_tokens,
                       int32_t* slot);

/* Batch form for building the decode arguments: for seqs[i], row i of
 * tables[n, max_blocks] (unused entries set to 0), ctx_lens[i] and
 * slots[i] (either of the last two may be NULL).  KV_ERR_INVALID if a table
 * needs more than max_blocks entries. */
kv_status kv_batch_tables(const kv_pool* pool, const int64_t* seqs, int32_t n,
                          int32_t* tables, int32_t max_blocks,
                          int32_t* ctx_lens, int32_t* slots);

kv_status kv_pool_stats(const kv_pool* pool, kv_pool_stats_t* out);

/* The free stack, bottom first (cap entries available; *n gets its size). */
kv_status kv_pool_free_list(const kv_pool* pool, int32_t* out, int32_t cap,
                            int32_t* n);

/* ---- swap space ([deepinsea] "Swap": KV blocks move to CPU memory when the
 * GPU's runs short; the swap space is sized in GB) ---------------------------
 * The swap space is a host-memory copy of the pool's layout: host_blocks
 * blocks and host_slots tail slots, with arrays sized by kv_pool_bytes for a
 * desc whose num_blocks = host_blocks and max_seqs = host_slots (the caller
 * allocates them as pinned memory, hipHostMalloc).  Its blocks have their own
 * free stack, popped from its end and starting as 0..host_blocks-1.  Sizing
 * resets it; KV_ERR_STATE while any sequence is swapped out. */
kv_status kv_pool_set_swap_space(kv_pool* pool, int32_t host_blocks, int32_t host_slots);

/* Swap a group of resident sequences out (forks share blocks: swap them
 * together so that their shared blocks move, once).  Blocks every reference
 * to which comes from the group move to host blocks (first-seen order over
 * the group's tables, in the order given) and return to the device free
 * stack (leaving the prefix index); blocks also held outside the group stay
 * on the device (moving them would free nothing) and the group keeps them.
 * Each sequence trades its device tail slot for the lowest free host slot.
 * plan (host, cap entries) receives the copies, block entries first, and
 * *n_plan their number; at most (distinct blocks + n) entries.  The copies
 * must run (kv_swap_blocks, for every layer's pool) before anything writes
 * the freed blocks or slots.  While swapped, kv_seq_table names host block h
 * as -1 - h and the slot as -1 - host slot; fork, append and
 * kv_batch_tables refuse the sequence (KV_ERR_STATE); kv_seq_free releases
 * it.  All-or-nothing: KV_ERR_INVALID (a repeated sequence, cap too small),
 * KV_ERR_UNKNOWN_SEQ, KV_ERR_STATE (already swapped), KV_ERR_NO_SLOTS (host
 * slots), then KV_ERR_NO_BLOCKS (host blocks). */
kv_status kv_seq_swap_out(kv_pool* pool, const int64_t* seqs, int32_t n, kv_swap* plan,
                          int32_t cap, int32_t* n_plan);

/* Bring a group of swapped sequences back: every host block the group's
 * tables name takes a fresh device block from the free stack (first-seen
 * order) with the group's count of references; a host block whose count
 * reaches zero returns to the host free stack (one still held by a
 * sequence outside the group stays for it).  Returned blocks are not
 * re-entered in the prefix index.  Each sequence takes the lowest free
 * device slot.  Plan and errors as kv_seq_swap_out (KV_ERR_STATE if a
 * sequence is not swapped out; KV_ERR_NO_SLOTS / KV_ERR_NO_BLOCKS for the
 * device side).  The copies must run before the sequences are read. */
kv_status kv_seq_swap_in(kv_pool* pool, const int64_t* seqs, int32_t n, kv_swap* plan,
                         int32_t cap, int32_t* n_plan);

/* ---- device calls -------------------------------------------------------- */

/* Perform n copies (copies_dev: device array of kv_copy) on stream.  Block
 * copies move codes, scales and zero points; slot copies move tail rows.
 * Destinations must be distinct and not also sources in the same call. */
kv_status kv_copy_blocks(const kv_pool_desc* desc, const kv_pool_mem* mem,
                         const kv_copy* copies_dev, int32_t n, void* stream);

/* Perform a swap plan between one layer's device pool (desc, mem) and its
 * swap space (host_desc: the same block_size, num_kv_heads, head_dim and
 * codecs, num_blocks = host blocks, max_seqs = host slots; host_mem: its
 * arrays in pinned host memory, hipHostMalloc).  plan: n entries in pinned
 * host memory; the library checks them on the host (kinds, ranges, rows <=
 * block_size, no destination written twice or also read in the call) and a
 * kernel reads them directly, so the plan must stay unchanged until the
 * stream has run the copy.  One launch moves every entry: the device reads
 * or writes the host arrays over the host link, no staging buffer.  Tail
 * arrays are needed only for slot entries.  KV_ERR_INVALID for a bad entry,
 * geometry or alignment, or host memory that is not pinned. */
kv_status kv_swap_blocks(const kv_pool_desc* desc, const kv_pool_mem* mem,
                         const kv_pool_desc* host_desc, const kv_pool_mem* host_mem,
                         const kv_swap* plan, int32_t n, void* stream);

/* Quantize and store new K/V tokens ([tbr8] §4 store_kv, per (block, head)
 * as the scale tensor's shape gives; [yunthe] Q(x)).
 *   k_dev, v_dev   fp16 [T, Hkv, D], token-major; the new tokens of
 *                  sequence i are rows cu_seqlens[i] .. cu_seqlens[i+1]-1.
 *   cu_seqlens_dev int32 [num_seqs + 1], non-decreasing, cu[0] = 0.
 *   start_pos_dev  int32 [num_seqs]: position of sequence i's first new token
 *                  (its token count before this store).
 *   block_tables_dev int32 [num_seqs, max_blocks_per_seq]: row i covers every
 *                  block up to position start + new - 1.
 *   tail_slots_dev int32 [num_seqs]: each sequence's tail slot.
 *   max_new_tokens >= every sequence's new-token count (sizes the grid).
 *   num_seqs and ceil((block_size - 1 + max_new_tokens) / block_size) must
 *   stay below 65536 (launch grid limits); KV_ERR_INVALID otherwise.
 * Every (block, head) touched is re-quantized from the exact fp16 rows it
 * holds: rows before start_pos come from the tail slot, the rest from k/v.
 * When a sequence's last touched block stays partial, its new rows are also
 * written to the tail slot.  Device-resident indices are not checked: block
 * ids must be < N, slots < max_seqs, and no block may be written twice in one
 * call (shared blocks must have been copied first). */
kv_status kv_quantize_store(const kv_pool_desc* desc, const kv_pool_mem* mem,
                            const uint16_t* k_dev, const uint16_t* v_dev,
                            int32_t num_seqs, const int32_t* cu_seqlens_dev,
                            const int32_t* start_pos_dev,
                            const int32_t* block_tables_dev,
                            int32_t max_blocks_per_seq,
                            const int32_t* tail_slots_dev,
                            int32_t max_new_tokens, void* stream);

/* Workspace bytes paged_attn_decode needs for these sizes (fp32 partial
 * outputs and per-partition max / sum).  partition_size as below. */
size_t paged_attn_workspace_bytes(const kv_pool_desc* desc, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len,
                                  int32_t partition_size);

/* Fused dequantizing decode attention ([tbr8] §5 point 2: dequantize inside
 * the attention, no intermediate buffers; [yunthe] x_hat):
 *   out[s, h, :] = sum_t softmax_t(sm_scale * <q[s,h], K_hat[s, g, t]>) *
 *                  V_hat[s, g, t, :],  g = h / (num_q_heads / Hkv),
 *   over t < context_lens[s], token t read from block
 *   block_tables[s][t / bs], row t % bs.
 *   q_dev, out_dev fp16 [num_seqs, num_q_heads, D]; out written in full.
 *   context_lens_dev int32 [num_seqs]; 0 gives a zero output row.
 *   max_context_len >= every context length (sizes the grid).
 *   partition_size: tokens per split-K partition, a multiple of block_size
 *   (and of 32 when num_q_heads > Hkv), or 0 to let the library choose.
 *   One query head per KV head runs on the vector ALUs; grouped query heads
 *   (up to 16 per KV head, or a multiple of 16) run on MFMA.  Partitions
 *   are combined by a second log-sum-exp kernel.  workspace_dev (16-byte
 *   aligned, workspace_bytes >= paged_attn_workspace_bytes(...)) may be NULL
 *   when that is 0.  num_q_heads must be a multiple of Hkv; num_seqs and
 *   num_q_heads must stay below 65536 (launch grid limits). */
kv_status paged_attn_decode(const kv_pool_desc* desc, const kv_pool_mem* mem,
                            const uint16_t* q_dev, uint16_t* out_dev,
                            int32_t num_seqs, int32_t num_q_heads,
                            const int32_t* block_tables_dev,
                            int32_t max_blocks_per_seq,
                            const int32_t* context_lens_dev,
                            int32_t max_context_len, float sm_scale,
                            int32_t partition_size, void* workspace_dev,
                            size_t workspace_bytes, void* stream);

/* One decode step with the current token's store fused in: for every
 * sequence s with context_lens[s] > 0, first the work of kv_quantize_store
 * for one new token at position context_lens[s] - 1 (its fp16 rows
 * k_new_dev / v_new_dev [num_seqs, Hkv, D], row s; the block's earlier rows
 * from tail slot tail_slots_dev[s]; the same codes, scales, zero point and
 * tail-slot rows, bit for bit), then the attention of paged_attn_decode over
 * context_lens[s] tokens, the new one included.  The caller has reserved the
 * position (kv_seq_append) and performed its copy-on-write copies; the
 * block may not be shared with another sequence of the call.  With a single
 * partition per sequence, the last block's store runs inside the attention
 * kernel (two of the work group's waves quantize its K and V tiles, which
 * the attention then reads from LDS): one launch.  With split partitions
 * and one query head per KV head the same happens in each sequence's last
 * partition when that kernel keeps the plain kernel's occupancy; otherwise
 * (and for grouped query heads) the store kernel runs first, then the
 * decode.  Arguments and errors otherwise as paged_attn_decode; the pool's
 * tail slots must be set in mem.  [tbr8] §4 store_kv and §5 point 2;
 * [yunthe] Q(x) and x_hat. */
kv_status paged_attn_decode_append(const kv_pool_desc* desc, const kv_pool_mem* mem,
                                   const uint16_t* k_new_dev, const uint16_t* v_new_dev,
                                   const int32_t* tail_slots_dev,
                                   const uint16_t* q_dev, uint16_t* out_dev,
                                   int32_t num_seqs, int32_t num_q_heads,
                                   const int32_t* block_tables_dev,
                                   int32_t max_blocks_per_seq,
                                   const int32_t* context_lens_dev,
                                   int32_t max_context_len, float sm_scale,
                                   int32_t partition_size, void* workspace_dev,
                                   size_t workspace_bytes, void* stream);

/* paged_attn_decode (k_new_dev, v_new_dev, tail_slots_dev all NULL) or
 * paged_attn_decode_append (all set) for a call whose sequences share a
 * prefix: the first shared_tokens tokens of every sequence sit in the same
 * physical blocks (block_tables[s][j] equal for every s and
 * j < shared_tokens / block_size, as kv_seq_fork leaves them; a caller
 * contract, not checked).  The same outputs, with the prefix's tiles read
 * once per KV head and 16 queries instead of once per sequence: the prefix
 * partitions run as one matrix-core launch whose queries are all the
 * call's sequences x query heads of a KV head (sequence 0's block table),
 * beside the remaining partitions per sequence, then the log-sum-exp
 * reduce.  The prefix's launch runs on a second stream of the library's
 * (one per device, created by the first such call outside a stream capture
 * and kept until the process ends), forked from `stream` and joined back
 * to it before the reduce with events: the call stays ordered on `stream`,
 * and a captured call records both streams' kernels in the graph.  Calls
 * from several host threads are serialized at the fork.
 * [yunthe] "prefix caching" (blocks shared between requests); the shared
 * pass itself is a scheduling of the same sums.  partition_size must be
 * given (not 0) and a multiple of 32; shared_tokens a positive multiple of
 * it, below max_context_len; every context must exceed shared_tokens.
 * Workspace as paged_attn_workspace_bytes for these sizes.  Errors as
 * paged_attn_decode, plus KV_ERR_INVALID for a bad shared_tokens, a mix of
 * NULL and non-NULL append pointers, or more than 65535 x 16 queries per KV
 * head. */
kv_status paged_attn_decode_shared_prefix(const kv_pool_desc* desc, const kv_pool_mem* mem,
                                          const uint16_t* k_new_dev, const uint16_t* v_new_dev,
                                          const int32_t* tail_slots_dev,
                                          const uint16_t* q_dev, uint16_t* out_dev,
                                          int32_t num_seqs, int32_t num_q_heads,
                                          const int32_t* block_tables_dev,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens_dev,
                                          int32_t max_context_len, float sm_scale,
                                          int32_t partition_size, int32_t shared_tokens,
                                          void* workspace_dev, size_t workspace_bytes,
                                          void* stream);

/* Attention of several query tokens per sequence over the quantized cache:
 * chunked prefill over a cached prefix ([yunthe] "prefix caching": once the
 * prefix's blocks are in the pool only the new tokens are computed), or
 * several candidate / draft tokens of one sequence.  Sequence s's queries
 * are rows cu_seqlens[s] .. cu_seqlens[s+1] - 1 of q_dev and out_dev (fp16
 * [num_tokens, num_q_heads, D], token-major); they are its last
 * n_s = cu_seqlens[s+1] - cu_seqlens[s] stored tokens (store them first,
 * kv_quantize_store), and query i attends causally to tokens
 * 0 .. context_lens[s] - n_s + i:
 *   out[r, h, :] = sum_{t <= pos} softmax_t(sm_scale <q[r,h], K_hat[s,g,t]>)
 *                  V_hat[s, g, t, :],  g = h / (num_q_heads / Hkv).
 * cu_seqlens_dev int32 [num_seqs + 1] (cu[0] = 0, non-decreasing,
 * cu[num_seqs] = num_tokens); max_q_len >= every n_s and <= max_context_len
 * (sizes the grid).  Device-resident arrays are not checked: cu_seqlens as
 * stated, block ids < N and n_s <= context_lens[s] are the caller's contract
 * (a query that sees no token gives a zero row).  All query heads of a KV head and 16 (token, head) pairs at a
 * time run on the matrix cores, for any group size.  partition_size: a
 * multiple of 32 and of block_size, or 0 for the library's choice; a query
 * merges only the partitions its position reaches.  Workspace:
 * paged_attn_multi_query_workspace_bytes.  Errors as paged_attn_decode,
 * plus KV_ERR_INVALID for a bad max_q_len or more than 65535 (token, head)
 * tiles per KV head and sequence. */
kv_status paged_attn_multi_query(const kv_pool_desc* desc, const kv_pool_mem* mem,
                                 const uint16_t* q_dev, uint16_t* out_dev, int32_t num_seqs,
                                 int32_t num_q_heads, const int32_t* cu_seqlens_dev,
                                 int32_t num_tokens, int32_t max_q_len,
                                 const int32_t* block_tables_dev, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens_dev, int32_t max_context_len,
                                 float sm_scale, int32_t partition_size, void* workspace_dev,
                                 size_t workspace_bytes, void* stream);

/* Workspace bytes paged_attn_multi_query needs (fp32 partial outputs and
 * (max, sum) per query token, head and partition; 0 for one partition). */
size_t paged_attn_multi_query_workspace_bytes(const kv_pool_desc* desc, int32_t num_seqs,
                                              int32_t num_tokens, int32_t num_q_heads,
                                              int32_t max_q_len, int32_t max_context_len,
                                              int32_t partition_size);

/* Partition size (tokens) paged_attn_decode uses when given 0: a single
 * pass when num_seqs x (heads, or KV heads x 16-head tiles) gives at least
 * four work groups per compute unit of the current device and every context
 * fits in 4096 tokens; otherwise 2048 tokens, halved (down to 256) while the
 * grid would have fewer work groups than that.  Always a multiple of 32;
 * 0 for invalid arguments. */
int32_t paged_attn_default_partition(const kv_pool_desc* desc,
                                     int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_context_len);

/* paged_attn_decode_append without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc).  The split-K partial results go to
 * the library's own scratch: a device array of 64 MiB (67,108,864 bytes)
 * per GPU, held from library load until the process ends.  A call whose
 * workspace (paged_attn_workspace_bytes with the same arguments) exceeds it
 * fails with KV_ERR_INVALID before any device work.  The call allocates
 * nothing.  Its first call on a device looks up that device's scratch
 * address (a HIP runtime query; KV_ERR_HIP if it fails).  Every call on one
 * GPU shares that GPU's scratch: calls that overlap on one GPU (other
 * streams, or other threads) race and must be ordered by the caller.
 * Otherwise identical to paged_attn_decode_append (arguments, layouts,
 * results bit for bit). */
kv_status paged_attn_decode_append_noalloc(const kv_pool_desc* desc, const kv_pool_mem* mem,
                                           const uint16_t* k_new_dev, const uint16_t* v_new_dev,
                                           const int32_t* tail_slots_dev, const uint16_t* q_dev,
                                           uint16_t* out_dev, int32_t num_seqs, int32_t num_q_heads,
                                           const int32_t* block_tables_dev, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens_dev, int32_t max_context_len,
                                           float sm_scale, int32_t partition_size, void* stream);

/* ---- Measurement: the plain-read ceiling of the decode's access pattern --
 * Reads n_tiles tiles of tile_bytes bytes (1024, 2048 or 4096) from src_dev
 * and computes nothing but an xor of them: tile i of the list is source tile
 * order_dev[i] (a device int32 array of n_tiles ids, each in
 * [0, n_src_tiles): the caller's contract, not checked), or source tile i
 * when order_dev is NULL (then n_tiles <= n_src_tiles).  Each wavefront
 * streams a contiguous run of the list with 16-byte loads contiguous across
 * the wave, as the decode kernels read their tiles; one uint32 per work
 * group is written to sink_dev, which must hold at least
 * kv_stream_read_sink_words(n_tiles) words.  Asynchronous on stream.  The
 * benchmark reports this rate beside the decode's: reading scattered 2 KiB
 * tiles at this rate is what the decode could reach if its arithmetic cost
 * nothing. */
size_t kv_stream_read_sink_words(int64_t n_tiles);
kv_status kv_stream_read_tiles(const void* src_dev, int64_t n_src_tiles, int32_t tile_bytes,
                               const int32_t* order_dev, int64_t n_tiles, uint32_t* sink_dev,
                               size_t sink_words, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* kv_last_error(void);

/* Debug checks of the callers' contracts (returns the previous setting;
 * until the first call the environment variable PBQ_DEBUG_CHECKS, set to
 * anything but "0", turns them on).  Before launching, kv_quantize_store,
 * paged_attn_decode_append (and _noalloc) and paged_attn_decode_shared_prefix
 * with a store then copy their index arrays to the host and fail with
 * KV_ERR_INVALID when one call would write a physical block for two
 * sequences, or a tail slot twice (tiles of one call are written
 * concurrently: shared blocks must be copied first, deepinsea.top
 * "PagedAttention memory management in depth", "Copy-on-Write"); and
 * paged_attn_decode_shared_prefix fails when a sequence's table does not
 * hold sequence 0's blocks for the shared positions or its context does not
 * extend past them.  The copies synchronize the stream: for debugging, not
 * for timed runs.  Process-wide; thread-safe. */
int32_t kv_set_debug_checks(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* PBQ_H */

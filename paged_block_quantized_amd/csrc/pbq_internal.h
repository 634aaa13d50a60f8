// Internal interface between the C-ABI layer (capi.cpp) and the HIP launchers
// (*.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <string>
#include <type_traits>

#include "pbq.h"

namespace pbq {

// Records a message for kv_last_error() on this thread and returns st.
kv_status fail(kv_status st, const std::string& msg);

// Codec facts shared by host and device code.  The kernels are instantiated
// per (K codec, V codec) pair, named by codec_pair(k, v).
constexpr bool codec_has_zp(int c) { return c == KV_CODEC_I4_ASYM || c == KV_CODEC_I8_ASYM; }
constexpr bool codec_packed4(int c) { return c == KV_CODEC_I4_ASYM; }
constexpr int codec_pair(int k, int v) { return 4 * k + v; }
// the pairs the kernels are built for
constexpr bool codec_pair_supported(int k, int v) {
    return (k == KV_CODEC_I8_SYM && (v == KV_CODEC_I8_SYM || v == KV_CODEC_I4_ASYM || v == KV_CODEC_I8_ASYM)) ||
           (k == KV_CODEC_FP8_E4M3 && v == KV_CODEC_FP8_E4M3) ||
           (k == KV_CODEC_I4_ASYM && (v == KV_CODEC_I4_ASYM || v == KV_CODEC_I8_SYM));
}

// f(std::integral_constant<int, codec_pair(k, v)>{}) for a supported pair;
// hipErrorInvalidValue otherwise.
template <class F>
hipError_t with_codec_pair(int k, int v, F&& f) {
    switch (codec_pair(k, v)) {
        case codec_pair(KV_CODEC_I8_SYM, KV_CODEC_I8_SYM):
            return f(std::integral_constant<int, codec_pair(KV_CODEC_I8_SYM, KV_CODEC_I8_SYM)>{});
        case codec_pair(KV_CODEC_I8_SYM, KV_CODEC_I4_ASYM):
            return f(std::integral_constant<int, codec_pair(KV_CODEC_I8_SYM, KV_CODEC_I4_ASYM)>{});
        case codec_pair(KV_CODEC_I8_SYM, KV_CODEC_I8_ASYM):
            return f(std::integral_constant<int, codec_pair(KV_CODEC_I8_SYM, KV_CODEC_I8_ASYM)>{});
        case codec_pair(KV_CODEC_FP8_E4M3, KV_CODEC_FP8_E4M3):
            return f(std::integral_constant<int, codec_pair(KV_CODEC_FP8_E4M3, KV_CODEC_FP8_E4M3)>{});
        case codec_pair(KV_CODEC_I4_ASYM, KV_CODEC_I4_ASYM):
            return f(std::integral_constant<int, codec_pair(KV_CODEC_I4_ASYM, KV_CODEC_I4_ASYM)>{});
        case codec_pair(KV_CODEC_I4_ASYM, KV_CODEC_I8_SYM):
            return f(std::integral_constant<int, codec_pair(KV_CODEC_I4_ASYM, KV_CODEC_I8_SYM)>{});
        default:
            return hipErrorInvalidValue;
    }
}

struct QuantStoreArgs {
    int32_t block_size, num_kv_heads, head_dim, v_codec, k_codec;
    int8_t* k_codes;
    uint8_t* v_codes;
    uint16_t* k_scale;
    uint16_t* v_scale;
    uint8_t* v_zp;
    uint8_t* k_zp;
    uint16_t* tail_k;
    uint16_t* tail_v;
    const uint16_t* k;
    const uint16_t* v;
    int32_t num_seqs;
    const int32_t* cu_seqlens;
    const int32_t* start_pos;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* tail_slots;
    int32_t tiles_per_seq;  // upper bound on blocks touched per sequence
    // one-token append mode (cu_seqlens / start_pos unused): sequence s
    // stores row s of k / v at position append_ctx[s] - 1 (none if 0)
    const int32_t* append_ctx;
};

struct AttnArgs {
    int32_t block_size, num_kv_heads, head_dim, v_codec, k_codec;
    const int8_t* k_codes;
    const uint8_t* v_codes;
    const uint16_t* k_scale;
    const uint16_t* v_scale;
    const uint8_t* v_zp;
    const uint8_t* k_zp;
    const uint16_t* q;
    uint16_t* out;
    int32_t num_seqs, num_q_heads;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    float sm_scale;
    int32_t partition_blocks;  // blocks per split-K partition
    int32_t max_partitions;    // ceil(max_context_len / partition tokens), >= 1
    float* ws_out;             // [S, Hq, max_partitions, D]
    float* ws_ml;              // [S, Hq, max_partitions, 2]  (max, sum) base 2
    // fused store of the current token (all NULL for plain decode): the new
    // token's fp16 K/V rows [S, Hkv, D], tail slots, and the writable pool
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int32_t* tail_slots;
    uint16_t* tail_k;
    uint16_t* tail_v;
    // prefix shared by all sequences (0 for none): its first shared_parts
    // partitions (shared_tokens tokens, sequence 0's block table) run as one
    // grouped launch over every query; the per-sequence grid starts after them
    int32_t shared_tokens;
    int32_t shared_parts;
    // several query tokens per sequence (NULL for one): q and out rows
    // cu_q[s] .. cu_q[s+1] - 1 are sequence s's last tokens; the workspace
    // then has one row per query token and head
    const int32_t* cu_q;
    int32_t max_q_len;
};

struct CopyArgs {
    int32_t block_size, num_kv_heads, head_dim, v_codec, k_codec;
    int8_t* k_codes;
    uint8_t* v_codes;
    uint16_t* k_scale;
    uint16_t* v_scale;
    uint8_t* v_zp;
    uint8_t* k_zp;
    uint16_t* tail_k;
    uint16_t* tail_v;
    const kv_copy* copies;
    int32_t n;
};

// One side of a swap: a pool's arrays (device memory, or the device's
// addresses of pinned host memory).
struct SwapSide {
    char* k_codes;
    char* v_codes;
    uint16_t* k_scale;
    uint16_t* v_scale;
    uint8_t* v_zp;
    uint8_t* k_zp;
    char* tail_k;
    char* tail_v;
};

struct SwapArgs {
    SwapSide dev, host;
    const kv_swap* plan;  // device address of the pinned host plan
    int32_t n;
    int32_t block_size, num_kv_heads, head_dim, v_codec, k_codec;
    int32_t dev_blocks, dev_slots, host_blocks, host_slots;
    int32_t chunks;       // work groups per entry (grid y)
};

// Bytes one swap work group moves (256 threads x 4 x 16 bytes).
constexpr int64_t kSwapChunk = 256 * 4 * 16;

// Plain streaming read of tiles (the measured ceiling of the decode's
// access pattern): tiles of 2^tile_kib_log2 KiB, each wave a contiguous run
// of tiles_per_wave list entries; one xor word per work group to sink.
struct StreamReadArgs {
    const uint8_t* src;
    const int32_t* order;   // NULL: tile i of the list is source tile i
    int64_t n_tiles;
    int64_t tiles_per_wave;
    int32_t tile_kib_log2;
    uint32_t* sink;
};

// The library's device scratch (scratch.hip): kScratchBytes per device for
// the allocation-free decode; scratch_address gives the current device's
// copy (looked up once per device).
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_address(void** out);

hipError_t launch_quantize_store(const QuantStoreArgs& a, hipStream_t stream);
hipError_t launch_stream_read(const StreamReadArgs& a, hipStream_t stream);
int64_t stream_read_groups(int64_t n_tiles, int64_t tiles_per_wave);
hipError_t launch_paged_attn(const AttnArgs& a, hipStream_t stream);
// whether a split-partition decode fuses the current token's store into its
// partition kernel (else the store kernel runs first)
bool split_store_fused(const AttnArgs& a);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);
hipError_t launch_swap_blocks(const SwapArgs& a, hipStream_t stream);

}  // namespace pbq

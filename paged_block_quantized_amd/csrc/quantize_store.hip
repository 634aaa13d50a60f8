// Quantize-and-store kernel: fp16 K/V tokens -> per-(block, head) quantized
// tiles in scattered pool blocks.
//
// What it computes (web pages cited by site and section):
//  * tbr8.org "PagedAttention + block-wise quantization against mobile OOM",
//    §3: every block is quantized on its own; §4 store_kv: K codes are int8
//    with an fp16 scale of absmax / 127, one per (block, head) as the scale
//    tensor [num_blocks, num_heads, 1, 1] has it.
//  * yunthe.com "KV-cache quantization and PagedAttention", "quantization
//    principle": Q(x) = clamp(round(x / scale + zero_point), 0, 2^bits - 1),
//    used here for the INT4 and INT8 asymmetric V codecs (bits = 4, 8) and,
//    with zero point 128 and a signed store, for INT8; "vLLM deployment":
//    the cache may also be kept in FP8 E4M3.
//  Readings: rounding is to nearest with ties to even on the exact quotient;
//  the statistics cover only the rows a block holds; the INT4 range is
//  widened to contain 0 and its zero point is an integer; rows not yet held
//  are zero bytes; a partially filled block is re-quantized from the exact
//  fp16 rows kept in its sequence's tail slot.
//
// Mapping: one wavefront per (sequence, touched block, KV head, tensor); a
// workgroup of four waves takes K and V of two consecutive heads of one
// block, so each token row is read as 2 x D x 2 contiguous bytes and no wave
// carries both tensors' rows.  The per-sequence scalars are loaded together,
// then store_tile (store_tile.h: lane layout, exact rounding) loads every
// fp16 row of the wave's tensor at once, reduces with DPP and readlane, and
// writes the codes.

#include "device_common.h"
#include "pbq_internal.h"
#include "store_tile.h"

namespace pbq {
namespace {

template <int BS, int D, int CP>
__global__ __launch_bounds__(256) void quantize_store_kernel(QuantStoreArgs a) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.x * 2 + (wv >> 1);
    const int jj = blockIdx.y;
    const int s = blockIdx.z;   // < num_seqs by the grid

    // per-sequence scalars, all loaded before the first branch
    const int H = a.num_kv_heads;
    int c0, c1, sp;
    if (a.append_ctx) {   // one token per sequence, at position ctx - 1
        const int cx = a.append_ctx[s];
        c0 = s;
        c1 = s + (cx > 0 ? 1 : 0);
        sp = cx - 1;
    } else {
        c0 = a.cu_seqlens[s];
        c1 = a.cu_seqlens[s + 1];
        sp = a.start_pos[s];
    }
    const int slot = a.tail_slots[s];
    // keep the four loads ahead of the branch (the compiler would otherwise
    // sink each load below it and wait for them one after another)
    __asm__ volatile("" : : "s"(c0), "s"(c1), "s"(sp), "s"(slot));
    const int n_new = c1 - c0;
    const int end = sp + n_new;
    const int j = sp / BS + jj;
    if (g >= H || n_new <= 0 || j * BS >= end) return;
    const int phys = a.block_tables[(int64_t)s * a.max_blocks_per_seq + j];
    const TileStoreArgs t{a.k_codes, a.v_codes, a.k_scale, a.v_scale, a.v_zp, a.k_zp, a.tail_k, a.tail_v, a.k, a.v, H};
    if (wv & 1) store_tile<BS, D, CP, false, false, true>(t, g, slot, c0, sp, end, j, phys, nullptr, nullptr);
    else store_tile<BS, D, CP, false, true, false>(t, g, slot, c0, sp, end, j, phys, nullptr, nullptr);
}

// Grid: x = pairs of KV heads, y = blocks a sequence's new tokens can touch,
// z = sequences.
template <int BS, int D, int CP>
hipError_t launch_qs(const QuantStoreArgs& a, hipStream_t stream) {
    dim3 grid((unsigned)((a.num_kv_heads + 1) / 2), (unsigned)a.tiles_per_seq, (unsigned)a.num_seqs);
    hipLaunchKernelGGL((quantize_store_kernel<BS, D, CP>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_store(const QuantStoreArgs& a, hipStream_t stream) {
#define PBQ_QS(BS, D)                                                                         \
    if (a.block_size == BS && a.head_dim == D)                                                \
        return with_codec_pair(a.k_codec, a.v_codec,                                          \
                               [&](auto cp) { return launch_qs<BS, D, decltype(cp)::value>(a, stream); });
    PBQ_QS(16, 64)
    PBQ_QS(16, 128)
    PBQ_QS(32, 64)
    PBQ_QS(32, 128)
#undef PBQ_QS
    return hipErrorInvalidValue;
}

}  // namespace pbq

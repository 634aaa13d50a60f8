// Swap copies between one layer's device pool and its swap space in pinned
// host memory.
//
// deepinsea.top "PagedAttention memory management in depth", "Swap": when
// device memory runs short, KV-cache blocks move to CPU memory, and the
// host-device transfer is the price.  A block's data is five runs (K codes,
// V codes, two scale rows, zero points) scattered over the pool by the free
// list, so a plan of a few thousand blocks would be tens of thousands of
// small DMA commands.  Instead one launch moves the whole plan: the device
// reads or writes the pinned host arrays directly over the host link, each
// work group moving 16 KiB of one entry with 16-byte accesses, four in
// flight per lane.  A slot entry moves only the held rows of each head.
//
// Every entry's indices and row count were checked on the host; the kernel
// checks them again and skips an entry that is out of range, so a plan
// changed after the call cannot send it outside the arrays.

#include "device_common.h"
#include "pbq_internal.h"

namespace pbq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = (int)(kSwapChunk / (kThreads * 16));

__global__ __launch_bounds__(kThreads) void swap_kernel(SwapArgs a) {
    const kv_swap c = a.plan[blockIdx.x];
    const bool out = c.kind == KV_SWAP_BLOCK_OUT || c.kind == KV_SWAP_SLOT_OUT;
    const bool block = c.kind == KV_SWAP_BLOCK_OUT || c.kind == KV_SWAP_BLOCK_IN;
    if (!block && c.kind != KV_SWAP_SLOT_OUT && c.kind != KV_SWAP_SLOT_IN) return;
    const SwapSide from = out ? a.dev : a.host;
    const SwapSide to = out ? a.host : a.dev;
    const int H = a.num_kv_heads;
    const int64_t tile = (int64_t)a.block_size * a.head_dim;
    const int tid = threadIdx.x;
    const int64_t u0 = (int64_t)blockIdx.y * (kSwapChunk / 16) + tid;

    if (block) {
        const int32_t src_n = out ? a.dev_blocks : a.host_blocks;
        const int32_t dst_n = out ? a.host_blocks : a.dev_blocks;
        if (c.src < 0 || c.src >= src_n || c.dst < 0 || c.dst >= dst_n) return;
        const bool v4 = codec_packed4(a.v_codec), zp = codec_has_zp(a.v_codec);
        const bool k4 = codec_packed4(a.k_codec), kzp = codec_has_zp(a.k_codec);
        const int64_t kb = k4 ? tile * H / 2 : tile * H, vb = v4 ? tile * H / 2 : tile * H;
        const int64_t ku = kb / 16, units = (kb + vb) / 16;
        const char* sk = from.k_codes + c.src * kb;
        const char* sv = from.v_codes + c.src * vb - kb;
        char* dk = to.k_codes + c.dst * kb;
        char* dv = to.v_codes + c.dst * vb - kb;
        u32x4 r[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int64_t u = u0 + j * kThreads;
            if (u < units) r[j] = *(const u32x4*)((u < ku ? sk : sv) + u * 16);
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int64_t u = u0 + j * kThreads;
            if (u < units) *(u32x4*)((u < ku ? dk : dv) + u * 16) = r[j];
        }
        if (blockIdx.y == 0)
            for (int g = tid; g < H; g += kThreads) {
                to.k_scale[(int64_t)c.dst * H + g] = from.k_scale[(int64_t)c.src * H + g];
                to.v_scale[(int64_t)c.dst * H + g] = from.v_scale[(int64_t)c.src * H + g];
                if (zp) to.v_zp[(int64_t)c.dst * H + g] = from.v_zp[(int64_t)c.src * H + g];
                if (kzp) to.k_zp[(int64_t)c.dst * H + g] = from.k_zp[(int64_t)c.src * H + g];
            }
    } else {
        const int32_t src_n = out ? a.dev_slots : a.host_slots;
        const int32_t dst_n = out ? a.host_slots : a.dev_slots;
        if (c.src < 0 || c.src >= src_n || c.dst < 0 || c.dst >= dst_n) return;
        if (c.rows < 1 || c.rows > a.block_size) return;
        // per head and array: rows x D fp16 values = rows x D / 8 units,
        // at the head's offset in the [Hkv, bs, D] slot
        const int64_t hu = (int64_t)c.rows * a.head_dim / 8;
        const int64_t half = hu * H, units = 2 * half;
        const int64_t slot = tile * H * 2;
        u32x4 r[kUnroll];
        int64_t off[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int64_t u = u0 + j * kThreads;
            if (u < units) {
                const bool v = u >= half;
                const int64_t rem = v ? u - half : u;
                const int64_t h = rem / hu;
                off[j] = h * tile * 2 + (rem - h * hu) * 16;
                const char* base = (v ? from.tail_v : from.tail_k) + c.src * slot;
                r[j] = *(const u32x4*)(base + off[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int64_t u = u0 + j * kThreads;
            if (u < units) {
                char* base = (u >= half ? to.tail_v : to.tail_k) + c.dst * slot;
                *(u32x4*)(base + off[j]) = r[j];
            }
        }
    }
}

}  // namespace

hipError_t launch_swap_blocks(const SwapArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(swap_kernel, dim3((unsigned)a.n, (unsigned)a.chunks), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace pbq

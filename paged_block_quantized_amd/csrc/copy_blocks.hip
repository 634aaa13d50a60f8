// Copy-on-write copies of pool blocks and tail slots.
//
// deepinsea.top "PagedAttention memory management in depth", "Copy-on-Write":
// sequences share prefix blocks and only the block about to be modified is
// copied.  A block copy moves a physical block's codes (all heads; they are
// contiguous in the pool layout), scales and zero points; a slot
// copy moves a sequence's fp16 tail rows (K and V).
//
// One workgroup per copy, 16-byte accesses for the bulk data.

#include "device_common.h"
#include "pbq_internal.h"

namespace pbq {
namespace {

__device__ __forceinline__ void copy16(const void* src, void* dst, int64_t bytes, int tid, int nthr) {
    const u32x4* s = (const u32x4*)src;
    u32x4* d = (u32x4*)dst;
    for (int64_t i = tid; i < bytes / 16; i += nthr) d[i] = s[i];
}

__global__ __launch_bounds__(256) void copy_kernel(CopyArgs a) {
    const kv_copy c = a.copies[blockIdx.x];
    const int tid = threadIdx.x;
    const int H = a.num_kv_heads;
    const int64_t tile = (int64_t)a.block_size * a.head_dim;
    const bool v4 = codec_packed4(a.v_codec), zp = codec_has_zp(a.v_codec);
    const bool k4 = codec_packed4(a.k_codec), kzp = codec_has_zp(a.k_codec);
    if (c.kind == KV_COPY_BLOCK) {
        const int64_t codes = tile * H;
        const int64_t kb = k4 ? codes / 2 : codes;
        const int64_t vb = v4 ? codes / 2 : codes;
        copy16(a.k_codes + c.src * kb, a.k_codes + c.dst * kb, kb, tid, blockDim.x);
        copy16(a.v_codes + c.src * vb, a.v_codes + c.dst * vb, vb, tid, blockDim.x);
        for (int g = tid; g < H; g += blockDim.x) {
            a.k_scale[(int64_t)c.dst * H + g] = a.k_scale[(int64_t)c.src * H + g];
            a.v_scale[(int64_t)c.dst * H + g] = a.v_scale[(int64_t)c.src * H + g];
            if (zp) a.v_zp[(int64_t)c.dst * H + g] = a.v_zp[(int64_t)c.src * H + g];
            if (kzp) a.k_zp[(int64_t)c.dst * H + g] = a.k_zp[(int64_t)c.src * H + g];
        }
    } else if (c.kind == KV_COPY_SLOT) {
        const int64_t sb = tile * H * 2;
        copy16((const char*)a.tail_k + c.src * sb, (char*)a.tail_k + c.dst * sb, sb, tid, blockDim.x);
        copy16((const char*)a.tail_v + c.src * sb, (char*)a.tail_v + c.dst * sb, sb, tid, blockDim.x);
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)a.n), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pbq

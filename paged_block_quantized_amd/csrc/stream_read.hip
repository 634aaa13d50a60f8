// Plain streaming read of tiles: the ceiling the decode kernels are measured
// beside.  It reads what the decode reads -- whole tiles of contiguous bytes
// at positions a block table scatters -- and computes nothing but an xor of
// the data (one word per work group written out so that no load is dead;
// the xor of all of them is the xor of every 32-bit word of the listed
// tiles, each counted once per listing).
//
// Mapping: each wavefront takes a contiguous run of the tile list and reads
// it as a stream of 1 KiB chunks (16 bytes per lane, contiguous across the
// wave, non-temporal, as the decode's loads are), eight chunks in flight per
// wave; the tile ids of the wave's next 64 tiles are gathered into lanes
// once and read back with readlane.

#include "device_common.h"
#include "pbq_internal.h"

namespace pbq {
namespace {

constexpr int kWaves = 4;       // waves per work group
constexpr int kInflight = 8;    // 1 KiB chunks in flight per wave

__global__ __launch_bounds__(64 * kWaves) void stream_read_kernel(StreamReadArgs a) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wave = (int64_t)blockIdx.x * kWaves + w;
    const int64_t n_waves = (int64_t)gridDim.x * kWaves;
    // a list: the wave's contiguous run of it.  No list: the k-th tile of
    // the wave is tile wave + k n_waves, so that the waves together sweep
    // memory front to back (the sequential read)
    const int64_t t0 = a.order ? wave * a.tiles_per_wave : 0;
    const int64_t t1 = a.order ? min(t0 + a.tiles_per_wave, a.n_tiles)
                               : (wave < a.n_tiles ? (a.n_tiles - wave + n_waves - 1) / n_waves : 0);
    const int sh = a.tile_kib_log2;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = t0; base < t1; base += 64) {
        const int cnt = (int)min((int64_t)64, t1 - base);
        const int id = a.order ? (lane < cnt ? a.order[base + lane] : 0) : 0;
        const int nch = cnt << sh;
        for (int c = 0; c < nch; c += kInflight) {
            u32x4 v[kInflight];
#pragma unroll
            for (int k = 0; k < kInflight; ++k) {
                const int cc = min(c + k, nch - 1);   // the last batch re-reads its final chunk
                const int ti = cc >> sh;
                const int64_t tile = a.order ? (int64_t)readlane(id, ti) : wave + (base + ti) * n_waves;
                v[k] = load_once<true>((const u32x4*)(a.src + (((tile << sh) + (cc & ((1 << sh) - 1))) << 10) + 16 * lane));
            }
#pragma unroll
            for (int k = 0; k < kInflight; ++k) acc ^= c + k < nch ? v[k] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
    __shared__ uint32_t s_x[kWaves];
    if (lane == 0) s_x[w] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) y ^= s_x[k];
        a.sink[blockIdx.x] = y;
    }
}

}  // namespace

hipError_t launch_stream_read(const StreamReadArgs& a, hipStream_t stream) {
    const int64_t waves = (a.n_tiles + a.tiles_per_wave - 1) / a.tiles_per_wave;
    const int64_t groups = (waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)groups), dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

int64_t stream_read_groups(int64_t n_tiles, int64_t tiles_per_wave) {
    const int64_t waves = (n_tiles + tiles_per_wave - 1) / tiles_per_wave;
    return (waves + kWaves - 1) / kWaves;
}

}  // namespace pbq

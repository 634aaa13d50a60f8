// Fused dequantizing PagedAttention decode: split-K partition kernel plus the
// log-sum-exp reduce kernel.
//
// What it computes (web pages cited by site and section):
//  * tbr8.org "PagedAttention + block-wise quantization against mobile OOM",
//    §5 point 2: a QuantizedPagedAttention operator dequantizes inside the
//    attention, with no intermediate dequantized buffers; §2: K/V live in
//    fixed-size blocks reached through a block table.
//  * yunthe.com "KV-cache quantization and PagedAttention", "quantization
//    principle": x_hat = (Q(x) - zero_point) * scale; "PagedAttention
//    mechanism": block_table maps a sequence's logical blocks to physical ids.
//  The attention itself (softmax of scaled dot products of one query token
//  against every stored token of its sequence) is the standard definition;
//  the pages do not print it.
//
// Arithmetic: the per-(block, head) scales factor out of the inner products,
// score_t = (sm_scale * s_k) * sum_d q_d * code_td and
// acc_d += (p_t * s_v) * (code_td - zp); codes convert to fp32 exactly and all
// accumulation is fp32.  Softmax is online, in base 2 (scores are
// pre-multiplied by log2 e), with a running maximum that is uniform across the
// wavefront so that rescaling is a uniform branch taken only when a block
// raises the maximum.
//
// MHA partition kernel (one query head per KV head): one workgroup per
// (partition, head, sequence); its NW wavefronts take the partition's blocks
// round-robin.  Within a wave, lane l owns head dims (l % (D/16)) * 16 .. +16
// and token rows r * (64 / (D/16)) + l / (D/16) of every block, so one K tile
// (block_size x D int8 codes, contiguous) is read with 16-byte loads that are
// contiguous across the wave (1 KiB per instruction), and the INT8 V tile
// the same way (8-byte loads for INT4 V).  Each lane keeps 16 fp32
// accumulators; lanes are combined once per partition.  The block ids and
// scales of a wave's blocks are gathered into lanes once and read back with
// readlane, so the loop has no dependent scalar loads.  The next block's codes
// are loaded before the current block is computed.
//
// A partition either writes the final fp16 output (when its sequence has one
// partition) or (max, sum) and the normalised fp32 partial output to the
// workspace; the reduce kernel merges partitions with weights
// sum_p * 2^(max_p - max).

#include <math.h>

#include "device_common.h"
#include "pbq_internal.h"

namespace pbq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <bool V4, int NR>
struct VRegs;
template <int NR>
struct VRegs<false, NR> {
    u32x4 r[NR];
};
template <int NR>
struct VRegs<true, NR> {
    u32x2 r[NR];
};

// Code bytes -> fp16 pairs without a conversion instruction: v_perm_b32
// places a code byte u under the byte 0x64, giving the fp16 value 1024 + u
// exactly.  INT8 codes are first offset to u = c + 128 (xor 0x80), so the pair
// holds 1152 + c; INT4 nibbles are split into bytes and give 1024 + u.  The
// constant offsets are removed once per row (K) or once per partition (V).
constexpr uint32_t kF16Hi = 0x64646464u;
constexpr uint32_t kSelLo = 0x04010400u;  // bytes 0,1 -> fp16 pair
constexpr uint32_t kSelHi = 0x04030402u;  // bytes 2,3 -> fp16 pair
constexpr float kI8Bias = 1152.f;
constexpr float kI4Bias = 1024.f;

__device__ __forceinline__ f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }

__device__ __forceinline__ f16x2 perm_lo(uint32_t w) { return as_h2(__builtin_amdgcn_perm(kF16Hi, w, kSelLo)); }
__device__ __forceinline__ f16x2 perm_hi(uint32_t w) { return as_h2(__builtin_amdgcn_perm(kF16Hi, w, kSelHi)); }

template <int BS, int D, bool V4, int NW>
__global__ __launch_bounds__(64 * NW) void attn_partition_mha(AttnArgs a) {
    constexpr int LPR = D / 16;    // lanes per token row (16 dims each)
    constexpr int RPI = 64 / LPR;  // token rows per wave access
    constexpr int NR = BS / RPI;   // rows per lane per block
    constexpr int KT = BS * D;     // K tile bytes
    constexpr int VT = V4 ? KT / 2 : KT;

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int p = blockIdx.x;
    const int h = blockIdx.y;
    const int s = blockIdx.z;
    const int H = a.num_kv_heads;
    const int ctx = a.context_lens[s];
    const int nblk = (ctx + BS - 1) / BS;
    const int PB = a.partition_blocks;
    const int nparts = max(1, (nblk + PB - 1) / PB);
    if (p >= nparts) return;
    const int b0 = p * PB;
    const int b1 = min(b0 + PB, nblk);

    const int dl = (lane % LPR) * 16;
    f16x2 q2[8];
    float qbias;
    {
        const f16x8* qp = (const f16x8*)(a.q + ((int64_t)s * a.num_q_heads + h) * D + dl);
        const f16x8 q0 = qp[0], q1 = qp[1];
        float qs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            q2[e] = f16x2{q0[2 * e], q0[2 * e + 1]};
            q2[4 + e] = f16x2{q1[2 * e], q1[2 * e + 1]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) qs += (float)q0[e] + (float)q1[e];
        qbias = kI8Bias * qs;
    }

    const float c2 = a.sm_scale * kLog2e;
    float m = -INFINITY, l = 0.f, zacc = 0.f;
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;

    const int32_t* tab = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const int row_lane = lane / LPR;

    for (int base = b0 + w; base < b1; base += 64 * NW) {
        // stage this wave's next (up to) 64 blocks: ids, scales, zero points
        const int bi = base + lane * NW;
        int id = 0;
        float sk = 0.f, sv = 0.f, vb = 0.f;
        if (bi < b1) {
            id = tab[bi];
            const int64_t t = (int64_t)id * H + h;
            sk = bits_to_f16f(a.k_scale[t]) * c2;
            sv = bits_to_f16f(a.v_scale[t]);
            if constexpr (V4) vb = kI4Bias + (float)a.v_zp[t];
            else vb = kI8Bias;
        }
        const int cnt = min(64, (b1 - base + NW - 1) / NW);

        auto load = [&](int i, u32x4 (&kr)[NR], VRegs<V4, NR>& vr) {
            const int phys = readlane(id, i);
            const int64_t t = (int64_t)phys * H + h;
            const int8_t* kp = a.k_codes + t * KT + lane * 16;
            const uint8_t* vp = a.v_codes + t * VT + lane * (V4 ? 8 : 16);
#pragma unroll
            for (int r = 0; r < NR; ++r) kr[r] = *(const u32x4*)(kp + r * 1024);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if constexpr (V4) vr.r[r] = *(const u32x2*)(vp + r * 512);
                else vr.r[r] = *(const u32x4*)(vp + r * 1024);
            }
        };

        auto compute = [&](const u32x4 (&kr)[NR], const VRegs<V4, NR>& vr, int i) {
            const int blk = base + i * NW;
            const float skc = readlane(sk, i);
            float sc[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float d = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t u = kr[r][k] ^ 0x80808080u;
                    d = __builtin_amdgcn_fdot2(perm_lo(u), q2[2 * k], d, false);
                    d = __builtin_amdgcn_fdot2(perm_hi(u), q2[2 * k + 1], d, false);
                }
                sc[r] = d - qbias;
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) sc[r] = group_sum<LPR>(sc[r]);
            float bmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int t = blk * BS + r * RPI + row_lane;
                sc[r] = t < ctx ? sc[r] * skc : -INFINITY;
                bmax = fmaxf(bmax, sc[r]);
            }
            bmax = strided_max<LPR>(bmax);
            if (bmax > m) {
                const float alpha = __builtin_amdgcn_exp2f(m - bmax);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] *= alpha;
                l *= alpha;
                zacc *= alpha;
                m = bmax;
            }
            const float svv = readlane(sv, i);
            const float vbias = readlane(vb, i);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float pr = __builtin_amdgcn_exp2f(sc[r] - m);
                l += pr;
                const float pv = pr * svv;
                zacc = __builtin_fmaf(pv, vbias, zacc);
                if constexpr (V4) {
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const uint32_t wv = vr.r[r][k];
                        const uint32_t lo = wv & 0x0F0F0F0Fu;         // dims 8k + 0,2,4,6
                        const uint32_t hi = (wv >> 4) & 0x0F0F0F0Fu;  // dims 8k + 1,3,5,7
                        const f16x2 a0 = perm_lo(lo), a1 = perm_hi(lo);
                        const f16x2 b0 = perm_lo(hi), b1 = perm_hi(hi);
                        acc[8 * k + 0] = __builtin_fmaf(pv, (float)a0[0], acc[8 * k + 0]);
                        acc[8 * k + 2] = __builtin_fmaf(pv, (float)a0[1], acc[8 * k + 2]);
                        acc[8 * k + 4] = __builtin_fmaf(pv, (float)a1[0], acc[8 * k + 4]);
                        acc[8 * k + 6] = __builtin_fmaf(pv, (float)a1[1], acc[8 * k + 6]);
                        acc[8 * k + 1] = __builtin_fmaf(pv, (float)b0[0], acc[8 * k + 1]);
                        acc[8 * k + 3] = __builtin_fmaf(pv, (float)b0[1], acc[8 * k + 3]);
                        acc[8 * k + 5] = __builtin_fmaf(pv, (float)b1[0], acc[8 * k + 5]);
                        acc[8 * k + 7] = __builtin_fmaf(pv, (float)b1[1], acc[8 * k + 7]);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t u = vr.r[r][k] ^ 0x80808080u;
                        const f16x2 a0 = perm_lo(u), a1 = perm_hi(u);
                        acc[4 * k + 0] = __builtin_fmaf(pv, (float)a0[0], acc[4 * k + 0]);
                        acc[4 * k + 1] = __builtin_fmaf(pv, (float)a0[1], acc[4 * k + 1]);
                        acc[4 * k + 2] = __builtin_fmaf(pv, (float)a1[0], acc[4 * k + 2]);
                        acc[4 * k + 3] = __builtin_fmaf(pv, (float)a1[1], acc[4 * k + 3]);
                    }
                }
            }
        };

        // ping-pong: the next block's codes are in flight while one is computed
        u32x4 kA[NR], kB[NR];
        VRegs<V4, NR> vA, vB;
        load(0, kA, vA);
        int i = 0;
        for (; i + 1 < cnt; i += 2) {
            load(i + 1, kB, vB);
            compute(kA, vA, i);
            if (i + 2 < cnt) load(i + 2, kA, vA);
            compute(kB, vB, i + 1);
        }
        if (i < cnt) compute(kA, vA, i);
    }

    // combine the lanes that own the same dims (different token rows)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = strided_sum<LPR>(acc[e]);
    l = strided_sum<LPR>(l);
    zacc = strided_sum<LPR>(zacc);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] -= zacc;

    __shared__ float s_acc[NW][D];
    __shared__ float s_ml[NW][2];
    if (lane < LPR) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s_acc[w][dl + e] = acc[e];
    }
    if (lane == 0) {
        s_ml[w][0] = m;
        s_ml[w][1] = l;
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < D) {
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NW; ++k) M = fmaxf(M, s_ml[k][0]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const float f = s_ml[k][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_ml[k][0] - M);
            L = __builtin_fmaf(s_ml[k][1], f, L);
            o = __builtin_fmaf(s_acc[k][tid], f, o);
        }
        const float res = L > 0.f ? o / L : 0.f;
        const int64_t row = (int64_t)s * a.num_q_heads + h;
        if (nparts == 1) {
            a.out[row * D + tid] = f32_to_f16_bits(res);
        } else {
            const int64_t prow = row * a.max_partitions + p;
            a.ws_out[prow * D + tid] = res;
            if (tid == 0) {
                a.ws_ml[prow * 2] = M;
                a.ws_ml[prow * 2 + 1] = L;
            }
        }
    }
}

// One wavefront per (query head, sequence): merges the partitions of
// sequences that have more than one.
template <int BS, int D>
__global__ __launch_bounds__(64) void attn_reduce(AttnArgs a) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x;
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int ctx = a.context_lens[s];
    const int nblk = (ctx + BS - 1) / BS;
    const int nparts = max(1, (nblk + a.partition_blocks - 1) / a.partition_blocks);
    if (nparts == 1) return;
    const int64_t row = (int64_t)s * a.num_q_heads + h;
    const int64_t prow0 = row * a.max_partitions;
    float M = -INFINITY;
    for (int pp = lane; pp < nparts; pp += 64) M = fmaxf(M, a.ws_ml[(prow0 + pp) * 2]);
    M = wave_max(M);
    float L = 0.f;
    float o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = 0.f;
    for (int pp = 0; pp < nparts; ++pp) {
        const float mp = a.ws_ml[(prow0 + pp) * 2];
        const float lp = a.ws_ml[(prow0 + pp) * 2 + 1];
        const float wgt = mp == -INFINITY ? 0.f : lp * __builtin_amdgcn_exp2f(mp - M);
        L += wgt;
        const float* op = a.ws_out + (prow0 + pp) * D;
#pragma unroll
        for (int k = 0; k < PER; ++k) o[k] = __builtin_fmaf(wgt, op[lane + 64 * k], o[k]);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) a.out[row * D + lane + 64 * k] = f32_to_f16_bits(L > 0.f ? o[k] / L : 0.f);
}

template <int BS, int D, bool V4>
hipError_t launch_mha(const AttnArgs& a, hipStream_t stream) {
    constexpr int NW = 4;
    dim3 grid((unsigned)a.max_partitions, (unsigned)a.num_q_heads, (unsigned)a.num_seqs);
    hipLaunchKernelGGL((attn_partition_mha<BS, D, V4, NW>), grid, dim3(64 * NW), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_partitions <= 1) return e;
    hipLaunchKernelGGL((attn_reduce<BS, D>), dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_attn(const AttnArgs& a, hipStream_t stream) {
    if (a.num_q_heads != a.num_kv_heads) return hipErrorNotSupported;
    const bool v4 = a.v_codec == KV_CODEC_I4_ASYM;
#define PBQ_ATTN(BS, D)                                                        \
    if (a.block_size == BS && a.head_dim == D)                                 \
        return v4 ? launch_mha<BS, D, true>(a, stream) : launch_mha<BS, D, false>(a, stream);
    PBQ_ATTN(16, 64)
    PBQ_ATTN(16, 128)
    PBQ_ATTN(32, 64)
    PBQ_ATTN(32, 128)
#undef PBQ_ATTN
    return hipErrorInvalidValue;
}

}  // namespace pbq

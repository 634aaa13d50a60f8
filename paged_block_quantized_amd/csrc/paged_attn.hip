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
// acc_d += s_v * sum_t p_t * (code_td - zp); codes become fp16 exactly, the
// products are exact and all accumulation is fp32.  The weights p_t (at
// most 1, relative to the running maximum) enter the V products as fp16,
// and the normaliser sums the same rounded values.  Softmax is online, in
// base 2 (scores are pre-multiplied by log2 e), with a running maximum that
// is uniform across the wavefront so that rescaling is a uniform branch
// taken only when a block raises the maximum.
//
// MHA partition kernel (one query head per KV head): one workgroup per
// (partition, head, sequence); each of its NW wavefronts takes a contiguous
// run of the partition's blocks.  Within a wave, lane l owns head dims (l % (D/16)) * 16 .. +16
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

#include <memory>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "device_common.h"
#include "pbq_internal.h"
#include "store_tile.h"

namespace pbq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

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

// Byte codes of the other codecs, four to a dword, become fp16 pairs the
// same way, each pair affine in its codes with a unit and a bias that come
// off outside the inner products: x_hat = unit * (pair - bias) * scale.
//   I8_SYM  : 1152 + c (c xor 0x80 under 0x64), unit 1, bias 1152
//   I8_ASYM : 1024 + u (u under 0x64), unit 1, bias 1024 + zero point
//   FP8_E4M3: value(c) * 2^-8 exactly, unit 256, bias 0: the byte placed in
//             the high byte of a half, shifted right by one with its sign
//             kept and bit 14 cleared, puts E4M3's exponent (bias 7) and
//             mantissa into fp16's fields (bias 15), subnormals included.
constexpr uint32_t kSelF8Lo = 0x010C000Cu;   // bytes 0,1 -> high bytes of two halves
constexpr uint32_t kSelF8Hi = 0x030C020Cu;   // bytes 2,3
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f8_pair(uint32_t w, uint32_t sel) {
    const s16x2 t = __builtin_bit_cast(s16x2, __builtin_amdgcn_perm(0u, w, sel)) >> (s16x2){1, 1};
    return __builtin_bit_cast(uint32_t, t) & 0xBFFFBFFFu;
}
template <int C>
__device__ __forceinline__ uint32_t pair_lo(uint32_t w) {   // bytes 0, 1
    if constexpr (C == KV_CODEC_FP8_E4M3) return f8_pair(w, kSelF8Lo);
    else if constexpr (C == KV_CODEC_I8_SYM) return __builtin_amdgcn_perm(kF16Hi, w ^ 0x80808080u, kSelLo);
    else return __builtin_amdgcn_perm(kF16Hi, w, kSelLo);
}
template <int C>
__device__ __forceinline__ uint32_t pair_hi(uint32_t w) {   // bytes 2, 3
    if constexpr (C == KV_CODEC_FP8_E4M3) return f8_pair(w, kSelF8Hi);
    else if constexpr (C == KV_CODEC_I8_SYM) return __builtin_amdgcn_perm(kF16Hi, w ^ 0x80808080u, kSelHi);
    else return __builtin_amdgcn_perm(kF16Hi, w, kSelHi);
}
template <int C>
constexpr float code_unit() { return C == KV_CODEC_FP8_E4M3 ? 256.f : 1.f; }
// bias of a pair given the block's zero point (asymmetric codecs)
template <int C>
__device__ __forceinline__ float code_bias(float zp) {
    if constexpr (C == KV_CODEC_FP8_E4M3) return 0.f;
    else if constexpr (C == KV_CODEC_I8_SYM) return kI8Bias;
    else return kI4Bias + zp;   // INT4 nibbles and INT8 asymmetric bytes: 1024 + u
}

// The pool arrays and new rows the fused store of a decode call writes.
__device__ __forceinline__ TileStoreArgs fused_store_args(const AttnArgs& a) {
    return TileStoreArgs{const_cast<int8_t*>(a.k_codes), const_cast<uint8_t*>(a.v_codes),
                         const_cast<uint16_t*>(a.k_scale), const_cast<uint16_t*>(a.v_scale),
                         const_cast<uint8_t*>(a.v_zp), const_cast<uint8_t*>(a.k_zp), a.tail_k, a.tail_v,
                         a.k_new, a.v_new, a.num_kv_heads};
}

#ifndef PBQ_MHA_WAVES_PER_EU
#define PBQ_MHA_WAVES_PER_EU 1
#endif
// Cache policy of the split-K partial results (1: non-temporal): written
// once in the middle of the codes' read stream and read once by the reduce,
// they cost the stream less non-temporal (the 512-token partitions of 32
// sequences x 32768 tokens over a shared prefix: 2-4 % on the step).
#ifndef PBQ_WS_NT
#define PBQ_WS_NT 1
#endif

// Software pipeline over cnt >= 1 steps: the codes of the next DEPTH-1 steps
// are in flight while one step is computed.  Every load outside the short
// tail is unconditional (the prologue loads step cnt-1 again when
// cnt < DEPTH, a cache hit), because a load under a branch makes the
// compiler's wait at the join cover every outstanding load, the prefetched
// ones included.  first() runs once, after the first step's loads are issued.
template <int DEPTH, class Regs, class Load, class Compute, class First>
__device__ __forceinline__ void pipelined(int cnt, Load&& load, Compute&& compute, First&& first) {
    Regs r[DEPTH];
    load(0, r[0]);
    first();
#pragma unroll
    for (int k = 1; k < DEPTH; ++k) load(min(k, cnt - 1), r[k]);
    int i = 0;
    for (; i + 2 * DEPTH <= cnt; i += DEPTH) {
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            compute(r[k], i + k);
            load(i + k + DEPTH, r[k]);
        }
    }
    // fewer than 2 DEPTH steps remain; r[k] holds step i + k
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
        if (i + k < cnt) {
            compute(r[k], i + k);
            if (i + k + DEPTH < cnt) load(i + k + DEPTH, r[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
        if (i + DEPTH + k < cnt) compute(r[k], i + DEPTH + k);
}

// Work-group order of the partition kernels: 0 = partition fastest, then
// head, then sequence; 1 = head, partition, sequence; 2 = head, sequence,
// partition (every sequence's first partition is dispatched before any
// second one, so the short, partial last partitions come at the end).
#ifndef PBQ_GRID_ORDER
#define PBQ_GRID_ORDER 0
#endif

__device__ __forceinline__ void grid_coords(int& p, int& h, int& s) {
#if PBQ_GRID_ORDER == 0
    p = blockIdx.x; h = blockIdx.y; s = blockIdx.z;
#elif PBQ_GRID_ORDER == 1
    h = blockIdx.x; p = blockIdx.y; s = blockIdx.z;
#else
    h = blockIdx.x; s = blockIdx.y; p = blockIdx.z;
#endif
}

inline dim3 grid_dims(int parts, int heads, int seqs) {
#if PBQ_GRID_ORDER == 0
    return dim3((unsigned)parts, (unsigned)heads, (unsigned)seqs);
#elif PBQ_GRID_ORDER == 1
    return dim3((unsigned)heads, (unsigned)parts, (unsigned)seqs);
#else
    return dim3((unsigned)heads, (unsigned)seqs, (unsigned)parts);
#endif
}
// Tokens' worth of blocks that waves 0 and 1 of a fused partition hand to
// the other waves for the store they do first.
#ifndef PBQ_STORE_HANDICAP_TOKENS
#define PBQ_STORE_HANDICAP_TOKENS 48
#endif
#ifndef PBQ_MHA_DEPTH
#define PBQ_MHA_DEPTH 2
#endif
#ifndef PBQ_GQA_DEPTH
#define PBQ_GQA_DEPTH 2
#endif

// MHA partition kernel.  K tiles are token-major [bs, D]: lane l owns dims
// (l % (D/16)) * 16 .. +16 of rows r * (64 / (D/16)) + l / (D/16).  V tiles are
// dim-major [D, bs]: lane l owns dims l + 64 k (k < D/64), each a contiguous
// row of the block's tokens.  The softmax weights of a block (times its V
// scale) are broadcast to scalar registers with readlane and every lane
// accumulates its own dims, so no lane combination is needed for V.
template <int BS, int D, int CP, int NW, bool FUSED>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(FUSED ? (BS == 16 ? 5 : (codec_packed4(CP % 4) ? 4 : 3)) : PBQ_MHA_WAVES_PER_EU)))
void attn_partition_mha(AttnArgs a) {
    constexpr int KC = CP / 4, VC = CP % 4;
    constexpr bool V4 = codec_packed4(VC);
    constexpr bool VZP = codec_has_zp(VC);
    constexpr bool K4 = codec_packed4(KC);   // INT4 K: two head dims per byte
    constexpr bool KZP = codec_has_zp(KC);
    constexpr int LPR = D / 16;    // K: lanes per token row (16 dims each)
    constexpr int RPI = 64 / LPR;  // K: token rows per wave access
    constexpr int NR = BS / RPI;   // K: rows per lane per block
    constexpr int KB = K4 ? 8 : 16;          // K bytes per lane and row (16 dims)
    constexpr int KACC = 64 * KB;            // K bytes per wave access
    constexpr int KT = BS * D * KB / 16;     // K tile bytes
    constexpr int DPL = D / 64;    // V: dims per lane
    constexpr int VROW = V4 ? BS / 2 : BS;  // V: bytes per dim row
    constexpr int VT = D * VROW;   // V tile bytes
    constexpr int VW = VROW / 4;   // V: dwords per dim row

    using KReg = std::conditional_t<K4, u32x2, u32x4>;
    struct Regs {
        KReg k[NR];
        uint32_t v[DPL][VW];
    };

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    int p, h, s;
    grid_coords(p, h, s);
    p += a.shared_parts;   // partitions of a shared prefix ran in their own launch
    const int H = a.num_kv_heads;
    const int ctx = a.context_lens[s];
    const int nblk = (ctx + BS - 1) / BS;
    const int PB = a.partition_blocks;
    const int nparts = max(1, (nblk + PB - 1) / PB);
    if (p >= nparts) return;
    const int b0 = p * PB;
    const int b1 = min(b0 + PB, nblk);
    const int32_t* tab = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

    // Fused store of the current token (position ctx - 1): in the sequence's
    // last partition, waves 0 and 1 first re-quantize the last block's K and
    // V tiles from the tail-slot rows and the new row (store_tile, the code
    // of the store kernel) into LDS copies of the codes and scales, and take
    // correspondingly fewer of the other blocks; after a barrier, wave NW - 1
    // adds the last block's contribution from the LDS copy while waves 0 and
    // 1 write the tiles to the pool (writes mixed into the bulk of the reads
    // cost several times their size).
    __shared__ __align__(16) uint8_t s_tile[FUSED ? KT + VT : 16];
    __shared__ uint32_t s_tscale[5];
    const bool fused = FUSED && p == nparts - 1 && nblk > 0;   // uniform in the group
    if (fused && w < 2) {
        const TileStoreArgs t = fused_store_args(a);
        const int last = nblk - 1;
        const int slot = a.tail_slots[s], phys = tab[last];
        if (w == 0) {
            const TileScales ts = store_tile<BS, D, CP, true, true, false>(
                t, h, slot, s, ctx - 1, ctx, last, phys, (int8_t*)s_tile, s_tile + KT, false);
            if (lane == 0) {
                s_tscale[0] = ts.k_scale;
                s_tscale[3] = ts.prev;
            }
        } else {
            const TileScales ts = store_tile<BS, D, CP, true, false, true>(
                t, h, slot, s, ctx - 1, ctx, last, phys, (int8_t*)s_tile, s_tile + KT, false);
            if (lane == 0) {
                s_tscale[1] = ts.v_scale;
                s_tscale[2] = ts.v_zp;
                s_tscale[4] = ts.prev;
            }
        }
    }

    const int dl = (lane % LPR) * 16;
    // the lane's 16 query dims as fp16 pairs in the order the K codes come
    // out of a dword: byte codes give dims (4k, 4k+1), (4k+2, 4k+3); INT4
    // nibbles of dims 8c .. 8c+7 give (0, 2), (4, 6), (1, 3), (5, 7)
    f16x2 q2[8];
    float qs = 0.f;   // sum of the lane's query dims: the K code offset's weight
    {
        const f16x8* qp = (const f16x8*)(a.q + ((int64_t)s * a.num_q_heads + h) * D + dl);
        const f16x8 q0 = qp[0], q1 = qp[1];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const f16x8 x = c ? q1 : q0;
            if constexpr (K4) {
                q2[4 * c + 0] = f16x2{x[0], x[2]};
                q2[4 * c + 1] = f16x2{x[4], x[6]};
                q2[4 * c + 2] = f16x2{x[1], x[3]};
                q2[4 * c + 3] = f16x2{x[5], x[7]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) q2[4 * c + e] = f16x2{x[2 * e], x[2 * e + 1]};
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) qs += (float)q0[e] + (float)q1[e];
    }
    const float qbias = code_bias<KC>(0.f) * qs;   // the K offset's share (INT4 K: per block)

    const float c2 = a.sm_scale * kLog2e * code_unit<KC>();
    constexpr float vunit = code_unit<VC>();
    float m = -INFINITY, l = 0.f, zacc = 0.f;
    float acc[DPL][2];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k][0] = acc[k][1] = 0.f;

    const int row_lane = lane / LPR;

    // One block's contribution: scores, online softmax update, weighted V.
    // kzp: the block's K zero point (INT4 K; unused otherwise).
    auto compute_blk = [&](const Regs& r, int blk, float skc, float svv, float vbias, float kzp) {
        float sc[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            float d = 0.f;
            if constexpr (K4) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {   // dims 8c .. 8c+7 of the lane's 16
                    const uint32_t lo = r.k[j][c] & 0x0F0F0F0Fu, hi = (r.k[j][c] >> 4) & 0x0F0F0F0Fu;
                    d = __builtin_amdgcn_fdot2(perm_lo(lo), q2[4 * c + 0], d, false);
                    d = __builtin_amdgcn_fdot2(perm_hi(lo), q2[4 * c + 1], d, false);
                    d = __builtin_amdgcn_fdot2(perm_lo(hi), q2[4 * c + 2], d, false);
                    d = __builtin_amdgcn_fdot2(perm_hi(hi), q2[4 * c + 3], d, false);
                }
                sc[j] = d - code_bias<KC>(kzp) * qs;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    d = __builtin_amdgcn_fdot2(as_h2(pair_lo<KC>(r.k[j][k])), q2[2 * k], d, false);
                    d = __builtin_amdgcn_fdot2(as_h2(pair_hi<KC>(r.k[j][k])), q2[2 * k + 1], d, false);
                }
                sc[j] = d - qbias;
            }
        }
#pragma unroll
        for (int j = 0; j < NR; ++j) sc[j] = group_sum<LPR>(sc[j]);
        float bmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int t = blk * BS + j * RPI + row_lane;
            sc[j] = t < ctx ? sc[j] * skc : -INFINITY;
            bmax = fmaxf(bmax, sc[j]);
        }
        bmax = strided_max<LPR>(bmax);
        if (bmax > m) {
            const float alpha = __builtin_amdgcn_exp2f(m - bmax);
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
                acc[k][0] *= alpha;
                acc[k][1] *= alpha;
            }
            l *= alpha;
            zacc *= alpha;
            m = bmax;
        }
        // The block's weights 2^(score - max), in (0, 1], rounded to fp16:
        // both the V contraction (v_dot2_f32_f16 over pairs of tokens, the
        // weights from scalar registers) and the normaliser use the rounded
        // values, and the V scale applies to the block's sums in fp32, so
        // that no weight leaves fp16's normal range because of the scale.
        uint32_t ph[NR];
        float ps = 0.f;   // the lane's sum of its rounded weights
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const _Float16 h = (_Float16)__builtin_amdgcn_exp2f(sc[j] - m);
            ph[j] = (uint32_t)__builtin_bit_cast(uint16_t, h);
            ps += (float)h;
        }
        l += ps;
        zacc = __builtin_fmaf(svv * vbias, ps, zacc);
        // weights of all tokens of the block, uniform across the wave, as
        // fp16 pairs in the token order of the V operands
        uint32_t sw[BS];
#pragma unroll
        for (int t = 0; t < BS; ++t) sw[t] = (uint32_t)readlane((int)ph[t / RPI], (t % RPI) * LPR);
        auto wpair = [&](int t0, int t1) { return as_h2(sw[t0] | (sw[t1] << 16)); };
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            float b0 = 0.f, b1 = 0.f;
            if constexpr (V4) {
#pragma unroll
                for (int c = 0; c < VW; ++c) {   // tokens 8c .. 8c+7
                    const uint32_t wv = r.v[k][c];
                    const uint32_t lo = wv & 0x0F0F0F0Fu;         // tokens 0,2,4,6
                    const uint32_t hi = (wv >> 4) & 0x0F0F0F0Fu;  // tokens 1,3,5,7
                    const int t = 8 * c;
                    b0 = __builtin_amdgcn_fdot2(perm_lo(lo), wpair(t + 0, t + 2), b0, false);
                    b1 = __builtin_amdgcn_fdot2(perm_lo(hi), wpair(t + 1, t + 3), b1, false);
                    b0 = __builtin_amdgcn_fdot2(perm_hi(lo), wpair(t + 4, t + 6), b0, false);
                    b1 = __builtin_amdgcn_fdot2(perm_hi(hi), wpair(t + 5, t + 7), b1, false);
                }
            } else {
#pragma unroll
                for (int c = 0; c < VW; ++c) {   // tokens 4c .. 4c+3
                    const int t = 4 * c;
                    b0 = __builtin_amdgcn_fdot2(as_h2(pair_lo<VC>(r.v[k][c])), wpair(t, t + 1), b0, false);
                    b1 = __builtin_amdgcn_fdot2(as_h2(pair_hi<VC>(r.v[k][c])), wpair(t + 2, t + 3), b1, false);
                }
            }
            acc[k][0] = __builtin_fmaf(b0, svv, acc[k][0]);
            acc[k][1] = __builtin_fmaf(b1, svv, acc[k][1]);
        }
    };

    // Codes of one (block, head) tile: K from kp (the tile's first byte), V
    // from vp; either may point into the pool (nt: read once, non-temporal)
    // or into the LDS copy of a tile.
    auto load_tile = [&](auto nt, const int8_t* kp, const uint8_t* vp, Regs& r) {
        constexpr bool NT = decltype(nt)::value;
        kp += lane * KB;
#pragma unroll
        for (int j = 0; j < NR; ++j) r.k[j] = load_once<NT>((const KReg*)(kp + j * KACC));
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            const uint8_t* row = vp + (lane + 64 * k) * VROW;
            if constexpr (VROW == 8) {
                const u32x2 x = load_once<NT>((const u32x2*)row);
                r.v[k][0] = x[0];
                r.v[k][1] = x[1];
            } else {
#pragma unroll
                for (int c = 0; c < VROW / 16; ++c) {
                    const u32x4 x = load_once<NT>((const u32x4*)(row + 16 * c));
                    r.v[k][4 * c + 0] = x[0];
                    r.v[k][4 * c + 1] = x[1];
                    r.v[k][4 * c + 2] = x[2];
                    r.v[k][4 * c + 3] = x[3];
                }
            }
        }
    };

    // Each wave takes a contiguous run of the partition's blocks.  In a fused
    // partition the last block is left out, and waves 0 and 1 (which store
    // it) take `hc` fewer blocks each, spread over the other waves.
    const int b_end = fused ? nblk - 1 : b1;
    const int n = b_end - b0;
    const int hc = fused ? min(PBQ_STORE_HANDICAP_TOKENS / BS, n / NW) : 0;
    const int q = (n + 2 * hc) / NW, rem = (n + 2 * hc) % NW;
    const int w_start = b0 + w * q + min(w, rem) - min(w, 2) * hc;
    const int w_stop = w_start + q + (w < rem ? 1 : 0) - (w < 2 ? hc : 0);

    for (int base = w_start; base < w_stop; base += 64) {
        // stage this wave's next (up to) 64 blocks: ids, then (after the first
        // block's codes are in flight) scales and zero points
        const int bi = base + lane;
        const int id = bi < w_stop ? tab[bi] : 0;
        const int cnt = min(64, w_stop - base);
        // raw fp16 scale bits and zero point, converted where they are used
        // (any arithmetic here would make the first step's wait cover the
        // prefetched codes too)
        int sk = 0, sv = 0, zp = 0, kz = 0;

        auto load = [&](int i, Regs& r) {
            const int64_t t = (int64_t)readlane(id, i) * H + h;
            load_tile(std::true_type{}, a.k_codes + t * KT, a.v_codes + t * VT, r);
        };

        auto compute = [&](const Regs& r, int i) {
            compute_blk(r, base + i, bits_to_f16f((uint16_t)readlane(sk, i)) * c2,
                        bits_to_f16f((uint16_t)readlane(sv, i)) * vunit,
                        code_bias<VC>((float)readlane(zp, i)), (float)readlane(kz, i));
        };

        // scale bits of the staged blocks, issued after the first codes; only
        // the wave's own blocks (i < cnt) are ever read back, so lanes past
        // the end may hold any value
        auto scales = [&]() {
            const int64_t t = (int64_t)id * H + h;
            sk = a.k_scale[t];
            sv = a.v_scale[t];
            if constexpr (VZP) zp = a.v_zp[t];
            if constexpr (KZP) kz = a.k_zp[t];
        };
        pipelined<PBQ_MHA_DEPTH, Regs>(cnt, load, compute, scales);
    }
    if (FUSED && fused) {
        __syncthreads();   // waves 0 and 1 have left the tiles in LDS
        if (w < 2) {
            const TileStoreArgs t = fused_store_args(a);
            write_stored_tile<BS, D, CP>(t, w, h, a.tail_slots[s], s, ctx - 1, tab[nblk - 1], s_tile, s_tile + KT,
                                         s_tscale);
        }
        if (w == NW - 1) {
            Regs r;
            load_tile(std::false_type{}, (const int8_t*)s_tile, s_tile + KT, r);
            compute_blk(r, b_end, bits_to_f16f((uint16_t)s_tscale[0]) * c2,
                        bits_to_f16f((uint16_t)s_tscale[1]) * vunit, code_bias<VC>((float)s_tscale[2]),
                        (float)(s_tscale[0] >> 16));
        }
    }

    // every token row is held by LPR lanes: full-wave sums count it LPR times
    const float inv_lpr = 1.0f / (float)LPR;
    l = group_sum<64>(l) * inv_lpr;
    zacc = group_sum<64>(zacc) * inv_lpr;

    __shared__ float s_acc[NW][D];
    __shared__ float s_ml[NW][2];
#pragma unroll
    for (int k = 0; k < DPL; ++k) s_acc[w][lane + 64 * k] = acc[k][0] + acc[k][1] - zacc;
    if (lane == 0) {
        s_ml[w][0] = m;
        s_ml[w][1] = l;
    }
    __syncthreads();
    for (int tid = threadIdx.x; tid < D; tid += 64 * NW) {
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
            store_once<PBQ_WS_NT>(res, &a.ws_out[prow * D + tid]);
            if (tid == 0) {
                store_once<PBQ_WS_NT>(M, &a.ws_ml[prow * 2]);
                store_once<PBQ_WS_NT>(L, &a.ws_ml[prow * 2 + 1]);
            }
        }
    }
}

// ---- grouped-query attention on MFMA ---------------------------------------
//
// Several query heads share one KV head, so the contraction is dense enough
// for matrix cores: per 32-token step and per group of up to 16 query heads,
// S^T[32 tok x 16 heads] = K_hat[32 x D] * Q^T[D x 16] takes 2 x D/32
// v_mfma_f32_16x16x32_f16, and O^T[D x 16] += V_hat^T[D x 32] * P^T[32 x 16]
// takes D/16 more.  Codes become fp16 exactly (v_perm under 0x64); the
// constant offset of the K codes comes off each score (Q and the K codes
// are exact, so the offset's product is too), while the V operands are
// turned into code - zero point by one exact packed subtraction, so the PV
// accumulators carry no offset.  Products are exact in fp32.
//
// MFMA 16x16x32 f16 lane layout (A: m = l%16, k = 8(l/16)+i; B: n = l%16,
// k = 8(l/16)+i; C: n = l%16, m = 4(l/16)+i).  Token order inside a step is
// arranged so that no value moves between lanes:
//   * the PV contraction slot j of lane group g is token 8g + kappa(j), where
//     kappa is the order in which v_perm emits a V row's codes (identity for
//     INT8, even-then-odd tokens for INT4 nibbles);
//   * the QK product's M slot 4g+i of tile mt is token 8g + kappa(4mt + i),
//     so lane (head n, group g) ends up holding the scores of exactly the
//     tokens its PV B operand needs.
// A lane group g therefore touches the tokens 8g..8g+7 of the step, i.e. one
// block (bs 32) or block g/2 (bs 16): its V scale, zero point and K scale are
// per-lane values.
#ifndef PBQ_GQA_WAVES_PER_EU
#define PBQ_GQA_WAVES_PER_EU 3
#endif

// Codes reach LDS by direct-to-LDS loads (global_load_lds_dwordx4: lane i's
// 16 bytes land at the instruction's LDS base + 16 i), so every load
// instruction reads 1 KiB of contiguous pool memory and the MFMA operands
// are then gathered from LDS.  0 keeps the codes in registers, loaded in the
// operand layout straight from the pool.  The kernel with the fused store
// keeps the register path by default: with its LDS tile copy, staging would
// leave room for three work groups per CU instead of four.
#ifndef PBQ_GQA_STAGE
#define PBQ_GQA_STAGE 1
#endif
// Multi-query groups with byte-coded V that do not stage jointly (one tile
// per wave, or the four-wave groups of split partitions) keep the register
// path too: their waves re-read codes the L2 mostly holds (measured before
// joint staging existed: 4 % faster than per-wave staging on 512-query
// chunks over 4096 tokens, MHA, INT8).
#ifndef PBQ_MULTI_BYTEV_STAGE
#define PBQ_MULTI_BYTEV_STAGE 0
#endif
// Two-wave multi-query groups of two tiles per wave share one staging area:
// both waves stream every step, each for its own 32 queries, reading a
// step's V operands only after its softmax so that three waves fit per SIMD
// (512-query chunks over 4096 tokens: MHA with INT8 652 -> 702 TFLOP/s, 64
// query heads over 8 with INT8 K / INT4 V 741-757 -> 768-775).
#ifndef PBQ_MULTI_JOINT_STAGE
#define PBQ_MULTI_JOINT_STAGE 1
#endif
#ifndef PBQ_GQA_STAGE_FUSED
#define PBQ_GQA_STAGE_FUSED 0
#endif
#ifndef PBQ_GQA_STAGES
#define PBQ_GQA_STAGES 2
#endif
// Single-pass grouped-query decode in paired groups (see attn_partition_gqa).
#ifndef PBQ_GQA_PAIR
#define PBQ_GQA_PAIR 1
#endif
// Most sequences a paired group ranks by context length (each of its
// threads ranks one sequence, or half of one's keys, against all S).
#ifndef PBQ_PAIR_RANK_MAX
#define PBQ_PAIR_RANK_MAX 256
#endif
constexpr int kPairRankMax = PBQ_PAIR_RANK_MAX;
// Loop steps the two waves of a paired group that quantize the stored tiles
// and take the stored steps give up to the other two, measured on a layer
// of 64 query heads over 8 KV heads with 128 sequences of 500-2000 tokens:
// 6 of its 32-token steps (3 was slower, 9 within the noise), and 12 of the
// shorter INT4 K steps (against 6: 1-2 us less).
#ifndef PBQ_PAIR_HANDICAP
#define PBQ_PAIR_HANDICAP 6
#endif
#ifndef PBQ_PAIR_HANDICAP_K4
#define PBQ_PAIR_HANDICAP_K4 12
#endif
// LDS of a paired group (two per CU must fit): per wave two stages of a
// step's codes (or a result slot, if larger), one more slot, and with the
// fused store both sequences' stored K and V tiles
constexpr int kPairLdsMax = 76 * 1024;   // the ranking's arrays need a few KiB more
template <int BS, int D, int CP, bool FUSED>
constexpr int gqa_pair_lds() {
    constexpr bool V4 = codec_packed4(CP % 4), K4 = codec_packed4(CP / 4);
    constexpr int stg = (32 * (K4 ? D / 2 : D) / 1024) * (1024 + 64) + (32 / BS) * D * (V4 ? BS / 2 : BS);
    constexpr int slot = 16 * (D + 4) * 4 + 16 * 8;
    constexpr int part = ((PBQ_GQA_STAGES * stg > slot ? PBQ_GQA_STAGES * stg : slot) + 15) / 16 * 16;
    return 4 * part + slot + (FUSED ? 2 * (BS * (K4 ? D / 2 : D) + D * (V4 ? BS / 2 : BS)) : 0);
}

// Waits for the direct-to-LDS loads are the kernel's own: the compiler cannot
// tell the stages apart and would wait for every such load in flight.
// Vector memory loads complete in issue order, so vmcnt(N) leaves only the N
// most recent ones outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    __asm__ volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
}
// NT: the non-temporal cache policy (codes read once; the policy immediate
// 2 is the instruction's nt bit)
template <bool NT>
__device__ __forceinline__ void load_to_lds(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0,
                                     NT && PBQ_NT_CODES ? 2 : 0);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS reads of staged codes, written as instructions the compiler does not
// see: it would otherwise make each of them wait for every direct-to-LDS
// load in flight, the prefetched steps included.  Their results are valid
// after wait_lds(); lds_fence(x) then hands x back to the compiler, so no use
// of x can be scheduled before the wait.
template <int OFF>
__device__ __forceinline__ void lds_read(u32x4& x, uint32_t a) {
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(a), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read(u32x2& x, uint32_t a) {
    __asm__ volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(x) : "v"(a), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read(uint32_t& x, uint32_t a) {
    __asm__ volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(x) : "v"(a), "i"(OFF));
}
template <class T>
__device__ __forceinline__ void lds_fence(T& x) {
    __asm__ volatile("" : "+v"(x));
}

template <int I>
using int_c = std::integral_constant<int, I>;
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(int_c<I>{}), ...);
}
// f(int_c<0>{}), ..., f(int_c<N - 1>{})
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// 16-byte chunk swizzle of a staged K row r (chunk c is kept at c ^ swz(r)):
// the rows that one operand read gathers (even or odd rows, or runs of four,
// depending on the token order) then fall in distinct bank groups.
__device__ __forceinline__ constexpr int kswz(int r) { return ((r >> 1) ^ ((r & 1) << 1)) & 3; }

template <bool V4>
__device__ __forceinline__ int kappa(int j) {
    if constexpr (V4) return (j & 4) ? 2 * (j & 3) + 1 : 2 * (j & 3);
    else return j;
}

typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// SHARED: the partitions of a prefix that every sequence of the call holds in
// the same physical blocks (sequence 0's table); the queries sharing a KV
// head are then all sequences' query heads of that group, 16 to a work
// group (query i: sequence i / G, head kvh * G + i % G), so each of the
// prefix's tiles is read once per 16 queries instead of once per sequence.
// Results always go to the workspace, for the reduce.
//
// MULTI: several query tokens per sequence, the last n of its stored tokens
// (rows cu_q[s] .. cu_q[s+1] - 1 of q), each attending causally up to its
// own position.  Query i of a sequence's tiles is token i / G with head
// kvh * G + i % G; a work group reads only the tokens its last query can
// see, and the steps past a wave's first query's position mask per query.
// Byte-coded V with D = 128 stages 34 KiB of LDS per 2-wave group, which caps
// the staged kernels at two waves per SIMD: their register budget is then
// that of two waves (no spills into AGPRs).  Two-wave multi-query groups use
// at most about 26 KiB (a shared three-stage area, or a merge through one
// wave's slot), room for three waves per SIMD, and get that register budget.
#ifndef PBQ_MULTI_WAVES_PER_EU
#define PBQ_MULTI_WAVES_PER_EU 3
#endif
template <int D, int CP, bool FUSED, bool MULTI, int NW, bool PAIR>
constexpr int gqa_waves_per_eu() {
    if (PAIR) return 2;   // two four-wave groups per CU
    if (MULTI && NW == 2) return PBQ_MULTI_WAVES_PER_EU;
    return MULTI || (!FUSED && D == 128 && !codec_packed4(CP % 4)) ? 2 : PBQ_GQA_WAVES_PER_EU;
}

//
// TPW: 16-query tiles per wave (MULTI only).  With two, every K and V code
// converted to fp16 feeds the matrix products of both tiles, which halves
// the conversion work per query; the softmax stays per tile.  Two-wave
// groups (single-pass launches) stream every step through one shared
// staging area, each wave for its own two tiles (JOINT); the four-wave
// groups of split partitions divide the steps and merge.
//
// PAIR (single-pass decode): each streaming wave's rate is set by its own
// loads in flight, so the step ends when the wave with the most steps does.
// A four-wave group takes two sequences -- those ranked `pair` and S - 1 -
// pair by context length (ties by index), so a long one with a short one --
// for one (KV head, query tile), and its waves split the two sequences'
// steps, laid end to end, into four equal runs.  The wave whose run crosses
// from the first sequence to the second leaves its first result in LDS; at
// the end waves 1 and 3 each merge one sequence's results and write its
// output.  With the fused store each wave loads one tile's exact rows (K or
// V of either sequence) before its loop and quantizes them after it.
template <int BS, int D, int CP, int NW, bool FUSED, bool SHARED = false, bool MULTI = false, int TPW = 1,
          bool PAIR = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(gqa_waves_per_eu<D, CP, FUSED, MULTI, NW, PAIR>())))
void attn_partition_gqa(AttnArgs a) {
    constexpr int KC = CP / 4, VC = CP % 4;
    constexpr bool V4 = codec_packed4(VC);
    constexpr bool VZP = codec_has_zp(VC);
    constexpr bool K4 = codec_packed4(KC);   // INT4 K: two head dims per byte
    constexpr bool KZP = codec_has_zp(KC);
    static_assert(!(FUSED && SHARED), "the shared prefix holds no current token");
    static_assert(!(MULTI && (FUSED || SHARED)), "multi-query launches store nothing and share nothing");
    static_assert(BS == 16 || BS == 32, "block size");
    static_assert(TPW == 1 || (MULTI && TPW == 2), "two tiles per wave only for multi-query launches");
    static_assert(!PAIR || (!MULTI && !SHARED && NW == 4), "paired groups: single-pass decode, four waves");
    constexpr int QT = 16 * TPW;               // queries per wave
    // JOINT: both waves stream every step of the partition from one staging
    // area, wave w for queries w QT .. of the group (no merge of waves)
    // (INT4 K rows are not staged: their codes stay on the register path)
    constexpr bool JOINT = MULTI && NW == 2 && TPW == 2 && PBQ_MULTI_JOINT_STAGE && !K4;
    constexpr int QW = JOINT ? NW * QT : QT;   // queries per work group
    // INT4 K is staged in paired groups (D 128: 64-byte rows, four chunks);
    // other INT4 K launches keep its codes on the register path
    constexpr bool STAGED = K4 ? (PAIR && D == 128)
                          : PAIR ? true
                          : FUSED ? PBQ_GQA_STAGE_FUSED
                          : (JOINT ? true : (MULTI && !V4 ? PBQ_MULTI_BYTEV_STAGE : PBQ_GQA_STAGE));
    // PAIR with the fused store: the stored tiles have LDS of their own (the
    // launcher pairs only when it fits)
    constexpr bool EARLY = PAIR && FUSED;
    static_assert(!PAIR || gqa_pair_lds<BS, D, CP, FUSED>() <= kPairLdsMax, "two paired groups per CU");
    constexpr int KS = D / 32;                 // QK k-steps
    constexpr int DT = D / 16;                 // PV dim tiles
    constexpr int KROW = K4 ? D / 2 : D;       // K bytes per token row
    constexpr int KCH = KROW / 4;              // K bytes per lane per row
    constexpr int NKC = KCH >= 16 ? KCH / 16 : 1;   // their 16-byte chunks (INT4 K, D 64: one of 8 bytes)
    using KChunk = std::conditional_t<(KCH >= 16), u32x4, u32x2>;
    constexpr int BPS = 32 / BS;               // blocks per 32-token step
    constexpr int SPB = 64 / BPS;              // steps whose block ids one wave stages at once
    constexpr int VROW = V4 ? BS / 2 : BS;     // V bytes per dim row
    constexpr int KT = BS * KROW;
    constexpr int VT = D * VROW;
    // codes read once per call (a decode work group owns its (sequence, KV
    // head)); multi-query and shared-prefix tiles reread them through L2
    constexpr bool NTL = !MULTI && !SHARED;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int n16 = lane & 15;       // head (C/B layouts) or M row (A layout)
    const int grp = lane >> 4;       // lane group
    const int G = a.num_q_heads / a.num_kv_heads;
    int p, tile, s;
    if constexpr (MULTI) {
        // Work groups go to the 8 XCDs (each with its own L2) round-robin by
        // launch order.  Renumber so that each XCD takes a contiguous range
        // of work items, ordered partition, then query tile, then KV head,
        // then sequence: the tiles of one (sequence, KV head), which read the
        // same codes, then run on one XCD at about the same time and share
        // its L2 instead of each XCD fetching them.
        const int P = gridDim.x, NT = gridDim.y;
        const int total = P * NT * gridDim.z;
        const int lin = blockIdx.x + P * (blockIdx.y + NT * blockIdx.z);
        const int xcd = lin % 8, k = lin / 8, q8 = total / 8, r8 = total % 8;
        const int work = xcd * q8 + min(xcd, r8) + k;
        p = work % P;
        tile = (work / P) % NT;
        s = work / (P * NT);
    } else if constexpr (PAIR) {
        p = 0;
        tile = blockIdx.y;
        s = 0;   // the pair's first sequence, below
    } else {
        grid_coords(p, tile, s);
    }
    // Ranks by context length, longest first (ties by index; beyond
    // kPairRankMax sequences, the call's own order).  PAIR: the group's
    // sequences are those of ranks pair and S - 1 - pair -- the first at
    // least as long as the second; an odd S leaves the middle rank alone
    // (seq_b -1).  Other single passes (one sequence per group): group z
    // takes the sequence at position z of the longest-first order with every
    // other run of 64 reversed, so that the compute units, which receive
    // consecutive groups in turn, each get long and short sequences.
    int seq_a = 0, seq_b = -1;
    // the group's sequences' context lengths (the second: PAIR), and (PAIR,
    // fused) tail slots
    int pctx[2] = {0, 0}, pslot[2] = {0, 0};
    bool have_ctx = false;
    // (four-wave groups without PAIR serve split partitions only: no ranking, no LDS for it)
    constexpr bool RANKED = !MULTI && !SHARED && (PAIR || NW != 4);
    if (RANKED && (PAIR || a.max_partitions == 1)) {   // uniform
        constexpr int NT = 64 * NW, HT = NT / 2;
        const int S = a.num_seqs;
        int want0, want1 = -1;
        if constexpr (PAIR) {
            want0 = blockIdx.z;
            want1 = S - 1 - (int)blockIdx.z != (int)blockIdx.z ? S - 1 - (int)blockIdx.z : -1;
        } else {
            const int b = s, start = b / 64 * 64, size = min(64, S - start);
            want0 = (b / 64) % 2 == 0 ? b : start + size - 1 - b % 64;
        }
        if (S <= kPairRankMax) {
            // Each thread reads one sequence's length (and, paired and fused,
            // its tail slot) into LDS.  Keys: the length (clamped; only the
            // order depends on it), then the reversed index, so that all keys
            // differ and the rank is the number of larger keys; two threads
            // per sequence when S <= NT / 2, each counting over half of the
            // keys (four at a time).  A length below the clamp is read back
            // from its key.
            __shared__ int s_pair[2];
            __shared__ __align__(16) uint32_t s_key[kPairRankMax];
            __shared__ int s_half[kPairRankMax / 2];   // the second half's counts
            __shared__ int s_slot[FUSED ? kPairRankMax : 1];
            const int S4 = (S + 3) & ~3;
            for (int i = threadIdx.x; i < S4; i += NT) {
                const int len = i < S ? a.context_lens[i] : 0;
                s_key[i] = i < S ? ((uint32_t)min(len, (1 << 22) - 1) << 9) | (uint32_t)(511 - i) : 0u;
                if constexpr (FUSED)
                    if (i < S) s_slot[i] = a.tail_slots[i];
            }
            if (threadIdx.x < 2) s_pair[threadIdx.x] = -1;
            __syncthreads();
            auto count = [&](int i, int j0, int j1) {   // keys j0 .. j1 - 1 above sequence i's
                const uint32_t ki = s_key[i];
                int cnt = 0;
#pragma unroll 4
                for (int j = j0; j < j1; j += 4) {
                    const u32x4 k4 = *(const u32x4*)&s_key[j];
                    cnt += (k4[0] > ki) + (k4[1] > ki) + (k4[2] > ki) + (k4[3] > ki);
                }
                return cnt;
            };
            auto found = [&](int i, int rank) {
                if (rank == want0) s_pair[0] = i;
                if (rank == want1) s_pair[1] = i;
            };
            if (S <= HT) {   // uniform
                const int i = (int)threadIdx.x % HT, half = (int)threadIdx.x / HT;
                const int mid = (S4 / 8) * 4;   // S4 / 2 rounded down to 4
                const int cnt = i < S ? count(i, half ? mid : 0, half ? S4 : mid) : 0;
                if (half == 1 && i < S) s_half[i] = cnt;   // i < NT / 2 <= kPairRankMax / 2
                __syncthreads();
                if (half == 0 && i < S) found(i, cnt + s_half[i]);
            } else {
                for (int i = threadIdx.x; i < S; i += NT) found(i, count(i, 0, S4));
            }
            __syncthreads();
            seq_a = s_pair[0];
            seq_b = s_pair[1];
            auto len_of = [&](int i) {
                const int k = (int)(s_key[i] >> 9);
                return k < (1 << 22) - 1 ? k : a.context_lens[i];
            };
            pctx[0] = len_of(seq_a);
            if constexpr (FUSED) pslot[0] = s_slot[seq_a];
            if constexpr (PAIR) {
                if (seq_b >= 0) pctx[1] = len_of(seq_b);
                if (FUSED && seq_b >= 0) pslot[1] = s_slot[seq_b];
            }
        } else {
            seq_a = PAIR ? want0 : s;
            seq_b = want1;
            pctx[0] = a.context_lens[seq_a];
            if constexpr (FUSED) pslot[0] = a.tail_slots[seq_a];
            if constexpr (PAIR) {
                if (seq_b >= 0) pctx[1] = a.context_lens[seq_b];
                if (FUSED && seq_b >= 0) pslot[1] = a.tail_slots[seq_b];
            }
        }
        s = seq_a;
        have_ctx = true;
    }
    if constexpr (!SHARED && !MULTI) p += a.shared_parts;   // shared partitions ran in their own launch
    const int q_row0 = MULTI ? a.cu_q[s] : 0;               // the sequence's first query row
    const int n_tok = MULTI ? a.cu_q[s + 1] - q_row0 : 1;   // its query tokens
    // queries that share a KV head's tiles
    const int NQ = SHARED ? a.num_seqs * G : n_tok * G;
    const int n_ht = (NQ + QW - 1) / QW;
    const int n_ht_grid = MULTI ? (a.max_q_len * G + QW - 1) / QW : n_ht;
    const int kvh = tile / n_ht_grid;
    const int ht = tile % n_ht_grid;
    if (MULTI && ht >= n_ht) return;
    const int H = a.num_kv_heads;
    int ctx_seq = SHARED ? a.shared_tokens : have_ctx ? pctx[0] : a.context_lens[s];
    // position of query token 0, and the tokens this tile's last query sees
    const int pos0 = ctx_seq - n_tok;
    int ctx = MULTI ? pos0 + (min(NQ, ht * QW + QW) - 1) / G + 1 : ctx_seq;
    int nblk = (ctx + BS - 1) / BS;
    const int PB = a.partition_blocks;
    const int nparts = max(1, (nblk + PB - 1) / PB);
    if (p >= nparts) return;
    // the partial results go to the workspace unless the sequence has a
    // single partition (the reduce merges by sequence)
    const int nblk_seq = (ctx_seq + BS - 1) / BS;
    const bool direct = SHARED ? false : (MULTI ? nblk_seq <= PB : nparts == 1);
    const int tok0 = p * PB * BS;
    int tok1 = min(tok0 + PB * BS, ctx);
    int nsteps = (tok1 - tok0 + 31) / 32;
    const int q0 = ht * QW + (JOINT ? w * QT : 0);   // the wave's first query
    const int nheads = max(0, min(QT, NQ - q0));      // the wave's queries (tile T: 16 T ..)
    // row of query ht * QT + i in q and out ([rows, Hq, D])
    auto query_row = [&](int i) -> int64_t {
        const int qi = q0 + i;
        if constexpr (SHARED) return (int64_t)(qi / G) * a.num_q_heads + kvh * G + qi % G;
        else if constexpr (MULTI) return (int64_t)(q_row0 + qi / G) * a.num_q_heads + kvh * G + qi % G;
        else return (int64_t)s * a.num_q_heads + kvh * G + qi;
    };
    // MULTI: the last token this lane's query sees (lanes without a query
    // see the whole tile, so that their scores stay finite), and the first
    // token that some query of the tile does not see
    int qlim[TPW];
#pragma unroll
    for (int T = 0; T < TPW; ++T)
        qlim[T] = MULTI && 16 * T + n16 < nheads ? pos0 + (q0 + 16 * T + n16) / G : ctx - 1;
    const int mask_from = MULTI ? pos0 + q0 / G + 1 : ctx;
    const int blk0 = tok0 / BS;
    int blk_end = (tok1 + BS - 1) / BS;

    // Q as the B operand of the QK product.  Byte-coded K: the contraction
    // index of k-step j, lane group grp, element i is head dim 64 (j/2) +
    // 16 grp + 8 (j%2) + i, so that a lane's K codes for two k-steps are 16
    // contiguous bytes and the four lane groups of one row read 64
    // contiguous bytes.  INT4 K: lane group grp holds the row's dims
    // 2 KCH grp .. + 2 KCH - 1 (KCH contiguous bytes), k-step j its dword j,
    // whose nibbles come out as dims 8j + (0, 2, 4, 6, 1, 3, 5, 7).
    f16x8v qop[TPW][KS];
    float qsum[TPW], qbias[TPW];
    // the loads of sequence `seq`'s query operands (PAIR: of either sequence)
    auto load_q_into = [&](f16x8v (&dst)[TPW][KS], int seq) {
#pragma unroll
        for (int T = 0; T < TPW; ++T) {
            const bool live = 16 * T + n16 < nheads;
            const int s_saved = s;
            s = seq;
            const uint16_t* qp = a.q + query_row(live ? 16 * T + n16 : 0) * D + (K4 ? 2 * KCH : 16) * grp;
            s = s_saved;
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                f16x8v x = (f16x8v)(_Float16)0;
                if (live) x = *(const f16x8v*)(qp + (K4 ? 8 * j : 64 * (j / 2) + 8 * (j % 2)));
                if constexpr (K4) dst[T][j] = __builtin_shufflevector(x, x, 0, 2, 4, 6, 1, 3, 5, 7);
                else dst[T][j] = x;
            }
        }
    };
    // the sum of each query's elements (the K codes' offset times it is
    // taken off the scores), once the loads above have landed
    auto q_sums = [&](const f16x8v (&qq)[TPW][KS], float (&qs_out)[TPW], float (&qb_out)[TPW]) {
#pragma unroll
        for (int T = 0; T < TPW; ++T) {
            float qs = 0.f;
#pragma unroll
            for (int j = 0; j < KS; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) qs += (float)qq[T][j][i];
            qs += shfl_xor_f(qs, 16);
            qs += shfl_xor_f(qs, 32);
            qs_out[T] = qs;
            qb_out[T] = code_bias<KC>(0.f) * qs;   // INT4 K: per block, from its zero point
        }
    };
    if constexpr (!PAIR) {
        load_q_into(qop, s);
        q_sums(qop, qsum, qbias);
    }

    const float c2 = a.sm_scale * kLog2e * code_unit<KC>();
    constexpr float vunit = code_unit<VC>();
    float m[TPW], l[TPW];
    f32x4 acc[TPW][DT];
#pragma unroll
    for (int T = 0; T < TPW; ++T) {
        m[T] = -INFINITY;
        l[T] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[T][t] = (f32x4)0.f;
    }

    // V-scale normaliser.  The PV product takes the weights p sv as fp16, so
    // a block whose fp16 V scale is tiny would give subnormal (imprecise)
    // weights, and a large one could overflow.  The weights are therefore
    // p sv 2^(15 + kVTop - vF): vF (wave-uniform) is an fp16 exponent field
    // that follows the largest V scale of the current step, changed only
    // when that scale's field rises above vF or falls more than kVHyst below
    // it, so that steady-state steps never change it.  The largest scale's
    // weights then lie in [2^kVTop, 2^(kVTop + 1)) times p, far above fp16's
    // subnormal range (p <= 1 in decode; MULTI's lazy softmax lets p reach
    // 2^kLazy, so its top is lower).  On a change the accumulators are
    // rescaled by the power of two (exact), and the result is multiplied
    // back once at the end, with the codec's unit.
    constexpr int kVHyst = 8;
    constexpr int kVTop = MULTI ? 6 : 10;
    int vF = 0;            // none yet: the first step sets it
    float vmul = 1.f;      // 2^(15 + kVTop - vF)
    auto vnorm_step = [&](int vbits) -> float {   // vbits: fp16 bits of the step's largest V scale
        const int f = max(1, (vbits >> 10) & 31);
        if (f > vF || f < vF - kVHyst) {
            const float r = __builtin_amdgcn_ldexpf(1.f, vF - f);
#pragma unroll
            for (int T = 0; T < TPW; ++T)
#pragma unroll
                for (int t = 0; t < DT; ++t) acc[T][t] *= r;
            vF = f;
            vmul = __builtin_amdgcn_ldexpf(1.f, 15 + kVTop - f);
        }
        return vmul;
    };

    const int32_t* tab = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // PAIR: switch the per-sequence state to sequence seq of context c (one
    // pass: tokens 0 .. c - 1), and the online softmax state
    auto set_unit = [&](int seq, int c) {
        s = seq;
        ctx_seq = ctx = c;
        nblk = (c + BS - 1) / BS;
        tok1 = min(tok0 + PB * BS, c);
        nsteps = (tok1 - tok0 + 31) / 32;
        blk_end = (tok1 + BS - 1) / BS;
        tab = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
    };
    auto reset_state = [&]() {
#pragma unroll
        for (int T = 0; T < TPW; ++T) {
            m[T] = -INFINITY;
            l[T] = 0.f;
#pragma unroll
            for (int t = 0; t < DT; ++t) acc[T][t] = (f32x4)0.f;
        }
        vF = 0;
        vmul = 1.f;
    };
    // lanes of one head split its tokens by group: sum their partial sums,
    // and undo the V-scale normaliser (times the codec's unit)
    auto finish_state = [&]() {
        const float vb = __builtin_amdgcn_ldexpf(vunit, vF - 15 - kVTop);
#pragma unroll
        for (int T = 0; T < TPW; ++T) {
            l[T] += shfl_xor_f(l[T], 16);
            l[T] += shfl_xor_f(l[T], 32);
#pragma unroll
            for (int t = 0; t < DT; ++t) acc[T][t] *= vb;
        }
    };
    // the block (within a step) whose K row this lane loads for tile mt, and
    // the row inside it: token 8(n16/4) + kappa(4mt + n16%4)
    int krow[2], kblk[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int tk = 8 * (n16 >> 2) + kappa<V4>(4 * mt + (n16 & 3));
        kblk[mt] = tk / BS;
        krow[mt] = tk % BS;
    }
    const int my_blk = (8 * grp) / BS;       // block of tokens 8grp..8grp+7
    const int vcol = ((8 * grp) % BS) / (V4 ? 2 : 1);

    using VReg = std::conditional_t<V4, uint32_t, u32x2>;   // a lane's V codes of one dim tile
    struct Raw {
        KChunk k[2][NKC];
        VReg v[DT];
    };

    // Codes of one 32-token step: the lane's K rows and V row come from the
    // tile of block 0 or block 1 of the step (bs 16), whose K and V tile
    // bases are given (pool or LDS copy).
    auto load_step = [&](auto nt, const int8_t* k0, const int8_t* k1, const uint8_t* v0, const uint8_t* v1,
                         Raw& r) {
        constexpr bool NT = decltype(nt)::value;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int8_t* kp = (BPS == 1 || !kblk[mt] ? k0 : k1) + krow[mt] * KROW + (K4 ? KCH : 16) * grp;
#pragma unroll
            for (int c = 0; c < NKC; ++c) r.k[mt][c] = load_once<NT>((const KChunk*)(kp + 64 * c));
        }
        const uint8_t* vp = (BPS == 1 || !my_blk ? v0 : v1) + vcol;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            r.v[t] = load_once<NT>((const VReg*)(vp + (16 * t + n16) * VROW));
        }
    };

    // One step: scores on MFMA, online softmax, PV on MFMA.  sk, sv, zpv are
    // this lane's block's scales (sk times sm_scale log2 e, sv times the
    // V-scale normaliser 2^(15 - vF)) and V zero point, kzv its K zero
    // point (INT4 K).
    // MULTI's lazy rescale threshold (base 2): the fp16 weights p sv 2^(15 +
    // kVTop - vF) stay below 2^(kLazy + kVTop + 1) = 2^15 (the normalised
    // scale is below 2^(kVTop + 1)), inside fp16's finite range for every
    // codec.
    constexpr float kLazy = MULTI ? 8.f : 0.f;
    // before_pv(r) runs after the softmax, before the V operands are used
    // (the shared-staging path reads them from LDS only then).
    auto compute_step = [&](Raw& r, int st, float sk, float sv, float zpv, float kzv, auto&& before_pv) {
        // ---- S^T = K_hat Q^T (each converted K operand serves every tile) --
        f32x4 sc[TPW][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int T = 0; T < TPW; ++T) sc[T][mt] = (f32x4)0.f;
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                uint32_t a4[4];
                if constexpr (K4) {   // dword j: dims 8j + (0, 2, 4, 6 | 1, 3, 5, 7)
                    const uint32_t w = r.k[mt][0][j];
                    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
                    a4[0] = __builtin_amdgcn_perm(kF16Hi, lo, kSelLo);
                    a4[1] = __builtin_amdgcn_perm(kF16Hi, lo, kSelHi);
                    a4[2] = __builtin_amdgcn_perm(kF16Hi, hi, kSelLo);
                    a4[3] = __builtin_amdgcn_perm(kF16Hi, hi, kSelHi);
                } else {
                    const uint32_t w0 = r.k[mt][j / 2][2 * (j & 1)];
                    const uint32_t w1 = r.k[mt][j / 2][2 * (j & 1) + 1];
                    a4[0] = pair_lo<KC>(w0);
                    a4[1] = pair_hi<KC>(w0);
                    a4[2] = pair_lo<KC>(w1);
                    a4[3] = pair_hi<KC>(w1);
                }
                const f16x8v aop = __builtin_bit_cast(f16x8v, a4);
#pragma unroll
                for (int T = 0; T < TPW; ++T)
                    sc[T][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, qop[T][j], sc[T][mt], 0, 0, 0);
            }
        }
        f16x8v pop[TPW];
#pragma unroll
        for (int T = 0; T < TPW; ++T) {
            // lane (head n16, group grp): sc[T][mt][i] is token 8 grp + kappa(4 mt + i)
            // (sc - qbias) sk as one rounding of sc sk plus the product -qbias sk
            float x[8];
            const float nb = -(K4 ? code_bias<KC>(kzv) * qsum[T] : qbias[T]) * sk;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) x[4 * mt + e] = __builtin_fmaf(sc[T][mt][e], sk, nb);
            // slot j holds token base + kappa(j) of the lane group's run
            const int base = tok0 + 32 * st + 8 * grp;
            if constexpr (MULTI) {
                if (tok0 + 32 * (st + 1) > mask_from) {   // causal mask, per query
                    const int lim = qlim[T] - base;          // slots with kappa(j) > lim are masked
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (kappa<V4>(j) > lim) x[j] = -INFINITY;
                }
            } else if (tok0 + 32 * (st + 1) > tok1) {   // the partition's last step: mask its end
                const int lim = tok1 - base;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (kappa<V4>(j) >= lim) x[j] = -INFINITY;
            }
            float bmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < 8; ++j) bmax = fmaxf(bmax, x[j]);
            // every step holds a token each query sees (MULTI: not always, see
            // mref below), so bmax is finite
            bmax = fmaxf(bmax, shfl_xor_f(bmax, 16));
            bmax = fmaxf(bmax, shfl_xor_f(bmax, 32));
            // per head; lanes of one head agree.  MULTI rescales only when the
            // maximum grows by more than kLazy (base 2): the weights
            // exp2(x - m) then stay at most 2^kLazy and most steps skip the
            // rescale of the accumulators (the final division by l uses the
            // same m, so the result is the same softmax)
            if (bmax > m[T] + kLazy) {
                const float alpha = __builtin_amdgcn_exp2f(m[T] - bmax);
#pragma unroll
                for (int t = 0; t < DT; ++t) acc[T][t] *= alpha;
                l[T] *= alpha;
                m[T] = bmax;
            }
            uint32_t pw[4];
            // a query that has seen no token yet (MULTI: all masked so far) keeps
            // m = -inf; its weights are 0, not exp2(-inf + inf)
            const float mref = MULTI && m[T] == -INFINITY ? 0.f : m[T];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(x[2 * e] - mref);
                const float p1 = __builtin_amdgcn_exp2f(x[2 * e + 1] - mref);
                l[T] += p0 + p1;
                const f16x2 h2 = f16x2{(_Float16)(p0 * sv), (_Float16)(p1 * sv)};
                pw[e] = __builtin_bit_cast(uint32_t, h2);
            }
            pop[T] = __builtin_bit_cast(f16x8v, pw);
        }

        before_pv(r);
        // ---- O^T += (V codes - zero point)^T P^T (each converted V operand
        // serves every tile).  v_perm gives bias + u; one packed fp16
        // subtraction of bias + zp (both integers below 2048: exact) leaves
        // u - zp, so no constant offset is carried through the accumulators
        // and cancelled at the end (its weights' sum would have to match the
        // matrix core's treatment of every fp16 weight, subnormals included).
        const _Float16 nb = (_Float16)(-code_bias<VC>(zpv));
        const f16x2 nb2 = f16x2{nb, nb};
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            uint32_t a4[4];
            if constexpr (V4) {
                const uint32_t wv = r.v[t];
                const uint32_t lo = wv & 0x0F0F0F0Fu, hi = (wv >> 4) & 0x0F0F0F0Fu;
                a4[0] = __builtin_amdgcn_perm(kF16Hi, lo, kSelLo);
                a4[1] = __builtin_amdgcn_perm(kF16Hi, lo, kSelHi);
                a4[2] = __builtin_amdgcn_perm(kF16Hi, hi, kSelLo);
                a4[3] = __builtin_amdgcn_perm(kF16Hi, hi, kSelHi);
            } else {
                a4[0] = pair_lo<VC>(r.v[t][0]);
                a4[1] = pair_hi<VC>(r.v[t][0]);
                a4[2] = pair_lo<VC>(r.v[t][1]);
                a4[3] = pair_hi<VC>(r.v[t][1]);
            }
            if constexpr (VC != KV_CODEC_FP8_E4M3) {
#pragma unroll
                for (int i = 0; i < 4; ++i) a4[i] = __builtin_bit_cast(uint32_t, as_h2(a4[i]) + nb2);
            }
            const f16x8v vop = __builtin_bit_cast(f16x8v, a4);
#pragma unroll
            for (int T = 0; T < TPW; ++T)
                acc[T][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[T], acc[T][t], 0, 0, 0);
        }
    };

    // Fused store of the current token (position ctx - 1), single-partition
    // launches: waves 0 and 1 re-quantize the last block's K and V tiles
    // (store_tile) into LDS copies and take fewer of the other steps; after a
    // barrier, wave NW - 1 computes the last step with the last block read
    // from LDS while waves 0 and 1 write the tiles to the pool (only the first
    // 16-head tile of a KV head writes).
    __shared__ __align__(16) uint8_t s_tile[FUSED && !PAIR ? KT + VT : 16];
    __shared__ uint32_t s_tscale[PAIR ? 10 : 5];   // PAIR: five per sequence
    __shared__ __align__(16) uint8_t s_ptile[EARLY ? 2 * (KT + VT) : 16];   // PAIR: each sequence's K, V tiles
    const bool fused = FUSED && nblk > 0;   // one partition: this group holds the last block
    // PAIR: the second sequence, and the tile whose exact rows this wave
    // loads now and quantizes after its loop (wave w: K for even w, else V,
    // of the first sequence for w < 2, else of the second)
    const int ctx_b = pctx[1];
    const bool fused_b = FUSED && ctx_b > 0;
    // PAIR, fused: wave 0 loads the first sequence's stored tile rows (K and
    // V), wave 3 the second's; each quantizes them once its first steps'
    // codes are in flight, and takes that sequence's stored step itself
    TileRows<BS> trows_k, trows_v;
    int t_seq = -1, t_ctx = 0, t_slot = 0, t_phys = 0;
    uint32_t prev_k = 0u, prev_v = 0u;
    if constexpr (PAIR && FUSED) {
        const int u = w == 0 ? 0 : w == NW - 1 ? 1 : -1;
        if (u >= 0) {
            t_seq = u ? seq_b : seq_a;
            t_ctx = pctx[u];
            t_slot = pslot[u];
        }
        if (t_seq >= 0 && t_ctx > 0) {
            // the last block's id, for the pool's previous scale bits (the
            // rows are loaded after the first steps' block ids)
            t_phys = a.block_tables[(int64_t)t_seq * a.max_blocks_per_seq + (t_ctx - 1) / BS];
        } else {
            t_seq = -1;
        }
    }
    // PAIR: both sequences' query operands, in registers
    const int nblk_a = nblk, nblk_b = (ctx_b + BS - 1) / BS;
    f16x8v qop_a[TPW][KS], qop_b[TPW][KS];
    float qsum_a[TPW], qsum_b[TPW], qbias_a[TPW], qbias_b[TPW];
    if constexpr (PAIR) {   // (loads only: their sums are taken once the first steps are in flight)
        load_q_into(qop_a, seq_a);
#pragma unroll
        for (int k = 0; k < KS; ++k) qop_b[0][k] = (f16x8v)(_Float16)0;
        if (seq_b >= 0) load_q_into(qop_b, seq_b);
    }
    if (!PAIR && fused && w < 2) {
        const TileStoreArgs t = fused_store_args(a);
        const int last = nblk - 1;
        const int slot = have_ctx ? pslot[0] : a.tail_slots[s], phys = tab[last];
        if (w == 0) {
            const TileScales ts = store_tile<BS, D, CP, true, true, false>(
                t, kvh, slot, s, ctx - 1, ctx, last, phys, (int8_t*)s_tile, s_tile + KT, false);
            if (lane == 0) {
                s_tscale[0] = ts.k_scale;
                s_tscale[3] = ts.prev;
            }
        } else {
            const TileScales ts = store_tile<BS, D, CP, true, false, true>(
                t, kvh, slot, s, ctx - 1, ctx, last, phys, (int8_t*)s_tile, s_tile + KT, false);
            if (lane == 0) {
                s_tscale[1] = ts.v_scale;
                s_tscale[2] = ts.v_zp;
                s_tscale[4] = ts.prev;
            }
        }
        // the staged loads' waits count on loads alone: let the stores drain
        if constexpr (STAGED) wait_vmem<0>();
    }

    // Each wave takes a contiguous run of the steps (the last one excluded in
    // a fused group, where waves 0 and 1 take `hc` fewer).  Lane L stages the
    // block id and raw scale bits of sub-block L % BPS of the run's
    // (L / BPS)-th step of the batch; the loop reads them with readlane.  The
    // next steps' codes are loaded while one is computed.
    const int n_loop = fused ? nsteps - 1 : nsteps;
    const int hc = fused ? min(PBQ_STORE_HANDICAP_TOKENS / 32, n_loop / NW) : 0;
    const int q = (n_loop + 2 * hc) / NW, rem = (n_loop + 2 * hc) % NW;
    const int w_start = JOINT ? 0 : w * q + min(w, rem) - min(w, 2) * hc;
    const int w_stop = JOINT ? n_loop : w_start + q + (w < rem ? 1 : 0) - (w < 2 ? hc : 0);
    // PAIR: the loop steps of both sequences (with the fused store, each
    // one's last step comes after the loop), laid end to end
    const int n_a = fused ? nsteps - 1 : nsteps;
    const int n_b = PAIR && seq_b >= 0 ? (fused_b ? (ctx_b + 31) / 32 - 1 : (ctx_b + 31) / 32) : 0;

    // Staging area of the direct-to-LDS path, per wave (one for the group in
    // the joint mode) and stage: the step's 32 K rows as 1 KiB loads (RPR
    // rows each, chunks swizzled by kswz, padded by 64 bytes), then its BPS V
    // tiles as in the pool.
    constexpr int SD = JOINT ? 3 : PBQ_GQA_STAGES;
    constexpr int CPR = KROW / 16;             // 16-byte chunks per K row
    constexpr int RPR = 1024 / KROW;           // K rows per load
    constexpr int NKL = 32 * KROW / 1024;      // K loads per step
    constexpr int KREG = 1024 + 64;
    constexpr int NVL = BPS * VT / 1024;       // V loads per step
    constexpr int NI = NKL + NVL;
    constexpr int STG = NKL * KREG + BPS * VT;
    static_assert(SD == 2 || SD == 3, "stages");
    static_assert(BPS * VT % 1024 == 0 && (VT % 1024 == 0 || (BPS == 2 && VT == 512)), "V tile loads");
    // PAIR: wave w's part of the area holds its stages, then (after its
    // loop) its result slot (QT rows of D + 4 floats, then QT (max, sum)
    // pairs); one more slot, for the first result of the wave whose run
    // crosses to the second sequence, follows the parts
    constexpr int SLOT = QT * (D + 4) * 4 + QT * 8;
    constexpr int PART_MIN = SLOT;
    constexpr int PART = PAIR ? ((STAGED && SD * STG > PART_MIN ? SD * STG : PART_MIN) + 15) / 16 * 16 : SD * STG;
    constexpr int STAGE_BYTES = PAIR ? NW * PART + SLOT : STAGED ? (JOINT ? 1 : NW) * SD * STG : 16;
    // two-wave multi-query groups merge through one wave's slot (the other
    // wave merges from its registers), which leaves LDS room for a third
    // work group of waves per SIMD
    constexpr bool HALF = MULTI && NW == 2 && !JOINT;
    constexpr int ACC_BYTES = JOINT || PAIR ? 16 : (HALF ? 1 : NW) * QT * (D + 4) * 4;
    __shared__ __align__(16) uint8_t s_stage[STAGE_BYTES > ACC_BYTES ? STAGE_BYTES : ACC_BYTES];
    uint8_t* const my_stage = s_stage + (JOINT ? 0 : w * PART);   // w is wave-uniform
    // lane offsets: where this lane's 16 bytes of a K load come from (row
    // lane / CPR of the load), and where its operands sit in a stage
    // (unsigned: a uniform base plus a 32-bit lane offset is the
    // instruction's scalar-base form)
    const int dma_r = lane / CPR;
    const uint32_t dma_k = (uint32_t)(dma_r * KROW + 16 * ((lane % CPR) ^ kswz(dma_r)));
    const uint32_t dma_v = 16u * (uint32_t)lane;
    int ko[2][NKC];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int R = kblk[mt] * BS + krow[mt];   // row within the step
#pragma unroll
        for (int c = 0; c < NKC; ++c)
            ko[mt][c] = (R / RPR) * KREG + (R % RPR) * KROW + 16 * ((grp + 4 * c) ^ kswz(R % RPR));
    }
    const int vo = NKL * KREG + my_blk * VT + vcol + n16 * VROW;

    // direct-to-LDS loads of one step (blocks id0, id1) into stage `buf`
    auto stage_step = [&](int id0, int id1, int buf) {
        uint8_t* sb = my_stage + buf * STG;
        const int8_t* kb0 = a.k_codes + ((int64_t)id0 * H + kvh) * KT;
        const int8_t* kb1 = a.k_codes + ((int64_t)id1 * H + kvh) * KT;
#pragma unroll
        for (int g = 0; g < NKL; ++g) {
            const int row0 = g * RPR;             // a load lies in one block
            if (!JOINT || g % NW == w)            // JOINT: the waves take turns
                load_to_lds<NTL>((row0 / BS ? kb1 : kb0) + (row0 % BS) * KROW + dma_k, sb + g * KREG);
        }
        const uint8_t* vb0 = a.v_codes + ((int64_t)id0 * H + kvh) * VT;
        const uint8_t* vb1 = a.v_codes + ((int64_t)id1 * H + kvh) * VT;
#pragma unroll
        for (int g = 0; g < NVL; ++g) {
            const uint8_t* src;
            if constexpr (VT >= 1024) src = ((1024 * g) / VT ? vb1 : vb0) + (1024 * g) % VT + dma_v;
            else src = (lane < 32 ? vb0 : vb1) + (dma_v & 511u);
            if (!JOINT || (NKL + g) % NW == w) load_to_lds<NTL>(src, sb + NKL * KREG + 1024 * g);
        }
    };
    // the lane's operands of the step in stage B (K rows: the second chunk
    // of a row is 64 bytes after the first, as kswz leaves bit 2 alone)
    const uint32_t la_k0 = lds_addr(my_stage) + (uint32_t)ko[0][0];
    const uint32_t la_k1 = lds_addr(my_stage) + (uint32_t)ko[1][0];
    const uint32_t la_v = lds_addr(my_stage) + (uint32_t)vo;
    auto read_stage_k = [&](auto bc, Raw& r) {
        constexpr int B = decltype(bc)::value;
        static_for<NKC>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            lds_read<B * STG + 64 * c>(r.k[0][c], la_k0);
            lds_read<B * STG + 64 * c>(r.k[1][c], la_k1);
        });
        wait_lds();
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
            lds_fence(r.k[0][c]);
            lds_fence(r.k[1][c]);
        }
    };
    auto read_stage_v = [&](auto bc, Raw& r) {
        constexpr int B = decltype(bc)::value;
        static_for<DT>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            lds_read<B * STG + 16 * t * VROW>(r.v[t], la_v);
        });
        wait_lds();
#pragma unroll
        for (int t = 0; t < DT; ++t) lds_fence(r.v[t]);
    };
    auto read_stage = [&](auto bc, Raw& r) {
        constexpr int B = decltype(bc)::value;
        static_for<NKC>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            lds_read<B * STG + 64 * c>(r.k[0][c], la_k0);
            lds_read<B * STG + 64 * c>(r.k[1][c], la_k1);
        });
        static_for<DT>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            lds_read<B * STG + 16 * t * VROW>(r.v[t], la_v);
        });
        wait_lds();
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
            lds_fence(r.k[0][c]);
            lds_fence(r.k[1][c]);
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) lds_fence(r.v[t]);
    };

    // A batch's block ids (lane L: sub-block L % BPS of its (L / BPS)-th
    // step), raw scale bits and zero points (converted at use).
    int id_l = 0, sk_l = 0, sv_l = 0, zp_l = 0, kz_l = 0;
    auto batch_tables = [&](int base, int w_stop) {
        const int st_l = base + lane / BPS;
        const int blk_l = blk0 + st_l * BPS + lane % BPS;
        const bool ok_l = st_l < w_stop && blk_l < blk_end;
        id_l = ok_l ? tab[blk_l] : 0;
        zp_l = 0;
        kz_l = 0;
    };
    auto batch_scales = [&]() {
        const int64_t t = (int64_t)id_l * H + kvh;
        sk_l = a.k_scale[t];
        sv_l = a.v_scale[t];
        if constexpr (VZP) zp_l = a.v_zp[t];
        if constexpr (KZP) kz_l = a.k_zp[t];
    };
    // direct-to-LDS loads of step i of the batch into stage buf
    auto stage_batch_step = [&](int i, int buf) {
        stage_step(readlane(id_l, i * BPS), readlane(id_l, i * BPS + BPS - 1), buf);
    };
    // The staged path's start of run [w_start, w_stop): the first batch's
    // tables and scales, and its first SD steps in flight.  run_steps(...,
    // true) then continues from there.
    auto issue_first = [&](int w_start, int w_stop, bool have_tables) {
        if (!have_tables) batch_tables(w_start, w_stop);
        batch_scales();
        const int cnt = min(SPB, w_stop - w_start);
        stage_batch_step(0, 0);
#pragma unroll
        for (int k = 1; k < SD; ++k)
            if (k < cnt) stage_batch_step(k, k);
    };
    // steps w_start .. w_stop - 1 of the sequence (pre: issue_first ran)
    auto run_steps = [&](int w_start, int w_stop, bool pre) {
    for (int base = w_start; base < w_stop; base += SPB) {
        const bool issued = pre && base == w_start;
        if (!issued) batch_tables(base, w_stop);
        const int cnt = min(SPB, w_stop - base);

        // Loads are unconditional: a block past the partition's end has id 0
        // (any valid block); its tokens are masked, so its codes only meet
        // zero softmax weights.  (Branches here would also make the compiler
        // wait for every outstanding load, the prefetch included.)
        auto load = [&](int i, Raw& r) {
            const int id0 = readlane(id_l, i * BPS), id1 = readlane(id_l, i * BPS + BPS - 1);
            load_step(std::integral_constant<bool, NTL>{}, a.k_codes + ((int64_t)id0 * H + kvh) * KT,
                      a.k_codes + ((int64_t)id1 * H + kvh) * KT,
                      a.v_codes + ((int64_t)id0 * H + kvh) * VT, a.v_codes + ((int64_t)id1 * H + kvh) * VT, r);
        };

        auto compute_with = [&](Raw& r, int i, auto&& before_pv) {
            const int st = base + i;
            // per-lane scales of the block holding this lane group's tokens.
            // The second block of a 16-token pair may lie past the end (its
            // staged id is 0): its tokens are masked, and its scales are
            // replaced by 0 so that stale pool contents cannot reach the sums.
            if constexpr (BPS == 1) {
                const int v0 = readlane(sv_l, i);
                const float vm = vnorm_step(v0);
                compute_step(r, st, bits_to_f16f((uint16_t)readlane(sk_l, i)) * c2,
                             bits_to_f16f((uint16_t)v0) * vm, (float)readlane(zp_l, i),
                             (float)readlane(kz_l, i), before_pv);
            } else {
                const bool live1 = blk0 + st * BPS + 1 < blk_end;
                const int k0 = readlane(sk_l, 2 * i), k1 = live1 ? readlane(sk_l, 2 * i + 1) : 0;
                const int v0 = readlane(sv_l, 2 * i), v1 = live1 ? readlane(sv_l, 2 * i + 1) : 0;
                const int z0 = readlane(zp_l, 2 * i), z1 = live1 ? readlane(zp_l, 2 * i + 1) : 0;
                const int kz0 = readlane(kz_l, 2 * i), kz1 = live1 ? readlane(kz_l, 2 * i + 1) : 0;
                const float vm = vnorm_step(max(v0, v1));   // fp16 bits of non-negative scales order as values
                compute_step(r, st, bits_to_f16f((uint16_t)(my_blk ? k1 : k0)) * c2,
                             bits_to_f16f((uint16_t)(my_blk ? v1 : v0)) * vm, (float)(my_blk ? z1 : z0),
                             (float)(my_blk ? kz1 : kz0), before_pv);
            }
        };
        auto compute = [&](Raw& r, int i) { compute_with(r, i, [](Raw&) {}); };

        auto scales = [&]() { batch_scales(); };
        if constexpr (JOINT) {
            // One staging area for both waves, three stages: step i + 2 is
            // loaded into the stage of step i - 1 once every wave has passed
            // the barrier of step i (so has read step i - 1), and two steps
            // are in flight while one is computed.  Each wave issues its
            // share of a step's loads (NIW) and waits for its own; the
            // barrier then makes the whole step visible.
            constexpr int NIW0 = (NI + 1) / 2, NIW1 = NI / 2;
            auto stage = [&](int i, int buf) {
                stage_step(readlane(id_l, i * BPS), readlane(id_l, i * BPS + BPS - 1), buf);
            };
            __builtin_amdgcn_s_barrier();   // the previous batch's stages are read
            scales();
            stage(0, 0);
            if (1 < cnt) stage(1, 1);
            auto one = [&](auto bc, int i) {
                constexpr int B = decltype(bc)::value;
                if (i + 1 < cnt) {   // step i + 1 was issued after step i
                    if (w == 0) wait_vmem<NIW0>();
                    else wait_vmem<NIW1>();
                } else {
                    wait_vmem<0>();
                }
                __builtin_amdgcn_s_barrier();
                Raw r;
                read_stage_k(bc, r);
                if (i + 2 < cnt) stage(i + 2, (B + 2) % 3);
                // V operands only after the softmax: fewer registers live
                compute_with(r, i, [&](Raw& rr) { read_stage_v(bc, rr); });
            };
            for (int i = 0; i < cnt; i += 3) {
                static_for<3>([&](auto bc) {
                    if (i + decltype(bc)::value < cnt) one(bc, i + decltype(bc)::value);
                });
            }
        } else if constexpr (STAGED) {
            // SD stages: step i + SD is loaded into step i's stage once its
            // operands are in registers, so SD steps are in flight while one
            // is computed.  Each wait leaves outstanding only the loads issued
            // after the step's own (the scale loads come first).
            auto stage = [&](int i, int buf) { stage_batch_step(i, buf); };
            if (!issued) {
                scales();
                stage(0, 0);
#pragma unroll
                for (int k = 1; k < SD; ++k)
                    if (k < cnt) stage(k, k);
            }
            auto one = [&](auto bc, int i) {
                constexpr int B = decltype(bc)::value;
                const int ahead = cnt - 1 - i;   // steps staged after step i
                if (SD == 3 && ahead >= 2) wait_vmem<(SD - 1) * NI>();
                else if (ahead >= 1) wait_vmem<NI>();
                else wait_vmem<0>();
                Raw r;
                read_stage(bc, r);
                if (i + SD < cnt) stage(i + SD, B);
                compute(r, i);
            };
            for (int i = 0; i < cnt; i += SD) {
                static_for<SD>([&](auto bc) {
                    if (i + decltype(bc)::value < cnt) one(bc, i + decltype(bc)::value);
                });
            }
        } else {
            pipelined<PBQ_GQA_DEPTH, Raw>(cnt, load, compute, scales);
        }
    }
    };

    // The last step of a fused single pass: its last block from the LDS copy
    // (lk, lv; sc: that block's scale bits as s_tscale holds them); in a
    // 16-token pair whose second block is the last one, the first block from
    // the pool.
    auto last_step = [&](const int8_t* lk, const uint8_t* lv, const uint32_t* sc) {
        const int st = nsteps - 1;
        const int last = nblk - 1;
        const int first = blk0 + st * BPS;            // == last when it is alone
        const int64_t t0 = (int64_t)tab[first] * H + kvh;
        const bool from_pool = first != last;         // block `first` comes from the pool
        Raw r;
        load_step(std::false_type{}, from_pool ? a.k_codes + t0 * KT : lk, lk, from_pool ? a.v_codes + t0 * VT : lv,
                  lv, r);
        const uint32_t ks0 = from_pool ? a.k_scale[t0] : sc[0] & 0xFFFFu;
        const uint32_t vs0 = from_pool ? a.v_scale[t0] : sc[1];
        const uint32_t z0 = from_pool ? (VZP ? a.v_zp[t0] : 0u) : sc[2];
        const uint32_t kz0 = from_pool ? (KZP ? a.k_zp[t0] : 0u) : sc[0] >> 16;
        // a lane group's block: `first` (my_blk 0) or the block after it,
        // which is the last block or lies past the end (masked)
        const bool mine_last = BPS == 1 || my_blk ? true : !from_pool;
        const int vl = __builtin_amdgcn_readfirstlane((int)sc[1]);
        const float vm = vnorm_step(from_pool ? max(vl, (int)vs0) : vl);
        compute_step(r, st, bits_to_f16f((uint16_t)(mine_last ? sc[0] : ks0)) * c2,
                     bits_to_f16f((uint16_t)(mine_last ? sc[1] : vs0)) * vm,
                     (float)(mine_last ? sc[2] : z0), (float)(mine_last ? sc[0] >> 16 : kz0), [](Raw&) {});
    };

    if constexpr (PAIR) {
        static_assert(STAGED && TPW == 1, "paired groups stream through the staged path");
        // Waves 0 and NW - 1 quantize a stored tile pair and take a stored
        // step each (fused): they get hc fewer loop steps.  Run k of the
        // loop steps laid end to end is [px(k), px(k + 1)).
        const int N = n_a + n_b;
        const int hc = FUSED ? min(K4 ? PBQ_PAIR_HANDICAP_K4 : PBQ_PAIR_HANDICAP, N / 4) : 0;
        auto px = [&](int k) { return (k * (N + 2 * hc)) / NW - (k > 0 ? hc : 0) - (k == NW ? hc : 0); };
        const bool last_a = FUSED && nblk_a > 0;                  // stored steps: wave 0 ...
        const bool last_b = FUSED && seq_b >= 0 && nblk_b > 0;    // ... and wave NW - 1
        auto seg_a = [&](int k) { return min(px(k + 1), n_a) > px(k) || (last_a && k == 0); };
        auto seg_b = [&](int k) { return px(k + 1) > max(px(k), n_a) || (last_b && k == NW - 1); };
        const int x0 = px(w), x1 = px(w + 1);
        const bool in_a = seg_a(w), in_b = seg_b(w);
        // a result slot: lane (n16, grp) holds dims 16t + 4 grp .. +3 of
        // query n16, and (grp 0) its (max, sum)
        auto write_slot = [&](uint8_t* sl) {
            float (*sa)[D + 4] = reinterpret_cast<float (*)[D + 4]>(sl);
            float (*sm)[2] = reinterpret_cast<float (*)[2]>(sl + QT * (D + 4) * 4);
#pragma unroll
            for (int t = 0; t < DT; ++t) *(f32x4*)&sa[n16][16 * t + 4 * grp] = acc[0][t];
            if (grp == 0) {
                sm[n16][0] = m[0];
                sm[n16][1] = l[0];
            }
        };
        auto use_q = [&](int u) {   // sequence u's query operands (uniform)
#pragma unroll
            for (int k = 0; k < KS; ++k) qop[0][k] = u ? qop_b[0][k] : qop_a[0][k];
            qsum[0] = u ? qsum_b[0] : qsum_a[0];
            qbias[0] = u ? qbias_b[0] : qbias_a[0];
        };
        // the wave's stored tiles (sequence w == 0 ? 0 : 1) in LDS
        const int tu = w == 0 ? 0 : 1;
        const int8_t* const tk = (const int8_t*)(s_ptile + tu * (KT + VT));
        const uint8_t* const tv = s_ptile + tu * (KT + VT) + KT;
        uint32_t* const tsc = s_tscale + 5 * tu;
        if (!in_a && in_b) set_unit(seq_b, ctx_b);
        const int r0 = in_a ? x0 : max(x0, n_a) - n_a;
        const int r1 = in_a ? min(x1, n_a) : x1 - n_a;
        // The first run's block ids, then (waves 0 and NW - 1) the stored
        // tiles' rows, then the first steps' scales and codes: loads complete
        // in issue order, so the rows must not come before what the first
        // steps wait for.  The tiles are quantized while those are in flight.
        if (r0 < r1) batch_tables(r0, r1);
        if constexpr (FUSED) {
            if (t_seq >= 0) {
                const TileStoreArgs t = fused_store_args(a);
                const int last = (t_ctx - 1) / BS;
                trows_k = load_tile_rows<BS, D, CP, false, true>(t, kvh, t_slot, t_seq, t_ctx - 1, t_ctx, last, 0);
                trows_v = load_tile_rows<BS, D, CP, false, false>(t, kvh, t_slot, t_seq, t_ctx - 1, t_ctx, last, 0);
            }
        }
        if (r0 < r1) issue_first(r0, r1, true);
        if constexpr (FUSED) {   // the pool's scale bits before the store (used after the loop)
            if (t_seq >= 0) {
                const int64_t tt = (int64_t)t_phys * H + kvh;
                prev_k = a.k_scale[tt] | (KZP ? (uint32_t)a.k_zp[tt] << 16 : 0u);
                prev_v = a.v_scale[tt] | (VZP ? (uint32_t)a.v_zp[tt] << 16 : 0u);
            }
        }
        q_sums(qop_a, qsum_a, qbias_a);
        if (seq_b >= 0) q_sums(qop_b, qsum_b, qbias_b);
        use_q(in_a ? 0 : 1);
        if constexpr (FUSED) {
            if (t_seq >= 0) {
                const TileStoreArgs t = fused_store_args(a);
                const int last = (t_ctx - 1) / BS;
                const TileScales ks = quantize_tile_rows<BS, D, CP, true, true, false>(
                    t, trows_k, kvh, t_slot, t_ctx - 1, t_ctx, last, t_phys, (int8_t*)tk, nullptr, false);
                const TileScales vs = quantize_tile_rows<BS, D, CP, true, false, true>(
                    t, trows_v, kvh, t_slot, t_ctx - 1, t_ctx, last, t_phys, nullptr, (uint8_t*)tv, false);
                if (lane == 0) {
                    tsc[0] = ks.k_scale;
                    tsc[1] = vs.v_scale;
                    tsc[2] = vs.v_zp;
                }
                wait_lds();
                __asm__ volatile("" : : : "memory");
            }
        }
        if (in_a) {
            if (w == 0 && last_a) last_step(tk, tv, tsc);
            run_steps(x0, min(x1, n_a), true);
        }
        if (in_b) {
            if (in_a) {   // crossing: the first sequence's result goes to the extra slot
                finish_state();
                write_slot(s_stage + NW * PART);
                reset_state();
                set_unit(seq_b, ctx_b);
                use_q(1);
            }
            run_steps(max(x0, n_a) - n_a, x1 - n_a, !in_a);
            if (w == NW - 1 && last_b) last_step(tk, tv, tsc);
        }
        if constexpr (FUSED) {
            if (t_seq >= 0 && ht == 0) {   // the first 16-head tile of a KV head writes the pool
                const TileStoreArgs t = fused_store_args(a);
                if (lane == 0) {   // the pool's scale bits before the store (loaded at the start)
                    tsc[3] = prev_k;
                    tsc[4] = prev_v;
                }
                wait_lds();
                write_stored_tile<BS, D, CP>(t, 0, kvh, t_slot, t_seq, t_ctx - 1, t_phys, (const uint8_t*)tk, tv, tsc);
                write_stored_tile<BS, D, CP>(t, 1, kvh, t_slot, t_seq, t_ctx - 1, t_phys, (const uint8_t*)tk, tv, tsc);
            }
        }
        finish_state();
        write_slot(s_stage + w * PART);   // its stages are no longer read
        __syncthreads();
        // Merge each sequence's results over the slots of the waves whose
        // runs ended on it (and the crossing wave's first result), in wave
        // order: a thread takes 8 dims of one query row -- the row's weights
        // once, then 8 outputs, written as 16 bytes.
        bool crossed = false;
        uint32_t tag = 0;   // bit k: wave k's result is the second sequence's
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            crossed |= seg_a(k) && seg_b(k);
            tag |= (seg_b(k) ? 1u : 0u) << k;
        }
        constexpr int CPR8 = D / 8;   // 8-dim chunks per row
        const int n_chunks = (seq_b >= 0 ? 2 : 1) * nheads * CPR8;
        for (int c = threadIdx.x; c < n_chunks; c += 64 * NW) {
            const int row_i = c / CPR8, d0 = (c % CPR8) * 8;
            const int u = row_i >= nheads ? 1 : 0, hh = row_i - (u ? nheads : 0);
            float mk[NW + 1], lk[NW + 1];
#pragma unroll
            for (int k = 0; k <= NW; ++k) {   // every slot is read; the unused ones are masked after
                const float (*sm)[2] = reinterpret_cast<const float (*)[2]>(s_stage + k * PART + QT * (D + 4) * 4);
                const bool use = k < NW ? ((tag >> k) & 1u) == (uint32_t)u : (u == 0 && crossed);
                mk[k] = use ? sm[hh][0] : -INFINITY;   // (an unused slot may hold anything)
                lk[k] = use ? sm[hh][1] : 0.f;
            }
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k <= NW; ++k) M = fmaxf(M, mk[k]);
            float f[NW + 1], L = 0.f;
#pragma unroll
            for (int k = 0; k <= NW; ++k) {
                f[k] = mk[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk[k] - M);
                L = __builtin_fmaf(lk[k], f[k], L);
            }
            const float rl = L > 0.f ? 1.f / L : 0.f;
            f32x4 o0 = (f32x4)0.f, o1 = (f32x4)0.f;
#pragma unroll
            for (int k = 0; k <= NW; ++k) {
                const float* sa = reinterpret_cast<const float*>(s_stage + k * PART) + hh * (D + 4) + d0;
                const f32x4 x0 = *(const f32x4*)sa, x1 = *(const f32x4*)(sa + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // a masked slot's values meet f = 0 only if finite: select
                    o0[i] = __builtin_fmaf(f[k] > 0.f ? x0[i] : 0.f, f[k], o0[i]);
                    o1[i] = __builtin_fmaf(f[k] > 0.f ? x1[i] : 0.f, f[k], o1[i]);
                }
            }
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                h[i] = (uint32_t)f32_to_f16_bits(o0[2 * i] * rl) | ((uint32_t)f32_to_f16_bits(o0[2 * i + 1] * rl) << 16);
                h[2 + i] = (uint32_t)f32_to_f16_bits(o1[2 * i] * rl) | ((uint32_t)f32_to_f16_bits(o1[2 * i + 1] * rl) << 16);
            }
            const int64_t row = (int64_t)(u ? seq_b : seq_a) * a.num_q_heads + kvh * G + q0 + hh;
            *(u32x4*)&a.out[row * D + d0] = u32x4{h[0], h[1], h[2], h[3]};
        }
        return;
    }
    run_steps(w_start, w_stop, false);
    if (FUSED && fused) {
        __syncthreads();   // waves 0 and 1 have left the last block's tiles in LDS
        if (w < 2 && ht == 0) {   // the first 16-head tile of a KV head writes the pool
            const TileStoreArgs t = fused_store_args(a);
            write_stored_tile<BS, D, CP>(t, w, kvh, have_ctx ? pslot[0] : a.tail_slots[s], s, ctx - 1, tab[nblk - 1],
                                         s_tile, s_tile + KT, s_tscale);
        }
        if (w == NW - 1) last_step((const int8_t*)s_tile, s_tile + KT, s_tscale);
    }
    // lanes of one head split its tokens by group: sum their partial sums,
    // and undo the V-scale normaliser (times the codec's unit)
    const float vback = __builtin_amdgcn_ldexpf(vunit, vF - 15 - kVTop);
#pragma unroll
    for (int T = 0; T < TPW; ++T) {
        l[T] += shfl_xor_f(l[T], 16);
        l[T] += shfl_xor_f(l[T], 32);
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[T][t] *= vback;
    }

    // Merge the waves' partial results in LDS (over the staging area, once
    // every wave is done with it).  Rows are padded by 4 floats so that the
    // 16-byte writes of one instruction spread over the banks.
    constexpr int DP = D + 4;
    float (*s_acc)[QT][DP] = reinterpret_cast<float (*)[QT][DP]>(s_stage);
    __shared__ float s_ml[PAIR ? 1 : NW][QT][2];   // (paired groups merge in their slots)
    if constexpr (STAGED) __syncthreads();
    if constexpr (JOINT) {
        // each wave holds every token of its queries: normalise and write
        // from the registers (lane: dims 16t + 4 grp .. +3 of query 16T + n16)
#pragma unroll
        for (int T = 0; T < TPW; ++T) {
            const int qq = 16 * T + n16;
            if (qq < nheads) {
                const int64_t row = query_row(qq);
                const float L = l[T];
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    float res[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) res[i] = L > 0.f ? acc[T][t][i] / L : 0.f;
                    const int d = 16 * t + 4 * grp;
                    if (direct) {
                        const uint32_t lo = (uint32_t)f32_to_f16_bits(res[0]) | ((uint32_t)f32_to_f16_bits(res[1]) << 16);
                        const uint32_t hi = (uint32_t)f32_to_f16_bits(res[2]) | ((uint32_t)f32_to_f16_bits(res[3]) << 16);
                        *(u32x2*)&a.out[row * D + d] = u32x2{lo, hi};
                    } else {
                        const int64_t prow = row * a.max_partitions + p;
                        store_once<PBQ_WS_NT>(f32x4{res[0], res[1], res[2], res[3]}, (f32x4*)&a.ws_out[prow * D + d]);
                        if (t == 0 && grp == 0) {
                            store_once<PBQ_WS_NT>(m[T], &a.ws_ml[prow * 2]);
                            store_once<PBQ_WS_NT>(L, &a.ws_ml[prow * 2 + 1]);
                        }
                    }
                }
            }
        }
        return;
    }
    if constexpr (HALF) {
        // wave 1 leaves its partial result in the slot; wave 0 combines it
        // with its own (the same arithmetic, in the same order, as the merge
        // over all waves below) and leaves the normalised result there, with
        // the combined (max, sum) in s_ml[0]
        if (w == 1) {
#pragma unroll
            for (int T = 0; T < TPW; ++T) {
                const int qq = 16 * T + n16;
                if (qq < nheads) {
#pragma unroll
                    for (int t = 0; t < DT; ++t) *(f32x4*)&s_acc[0][qq][16 * t + 4 * grp] = acc[T][t];
                    if (grp == 0) {
                        s_ml[1][qq][0] = m[T];
                        s_ml[1][qq][1] = l[T];
                    }
                }
            }
        }
        __syncthreads();
        if (w == 0) {
#pragma unroll
            for (int T = 0; T < TPW; ++T) {
                const int qq = 16 * T + n16;
                if (qq < nheads) {
                    const float m1 = s_ml[1][qq][0], l1 = s_ml[1][qq][1];
                    const float M = fmaxf(m[T], m1);
                    const float f0 = m[T] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[T] - M);
                    const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
                    const float L = __builtin_fmaf(l1, f1, l[T] * f0);
#pragma unroll
                    for (int t = 0; t < DT; ++t) {
                        f32x4* slot = (f32x4*)&s_acc[0][qq][16 * t + 4 * grp];
                        const f32x4 o1 = *slot;
                        f32x4 res;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float o = __builtin_fmaf(o1[i], f1, acc[T][t][i] * f0);
                            res[i] = L > 0.f ? o / L : 0.f;
                        }
                        *slot = res;
                    }
                    if (grp == 0) {
                        s_ml[0][qq][0] = M;
                        s_ml[0][qq][1] = L;
                    }
                }
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nheads * D; idx += 64 * NW) {
            const int hh = idx / D, d = idx % D;
            const float res = s_acc[0][hh][d];
            const int64_t row = query_row(hh);
            if (direct) {
                a.out[row * D + d] = f32_to_f16_bits(res);
            } else {
                const int64_t prow = row * a.max_partitions + p;
                store_once<PBQ_WS_NT>(res, &a.ws_out[prow * D + d]);
                if (d == 0) {
                    store_once<PBQ_WS_NT>(s_ml[0][hh][0], &a.ws_ml[prow * 2]);
                    store_once<PBQ_WS_NT>(s_ml[0][hh][1], &a.ws_ml[prow * 2 + 1]);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int T = 0; T < TPW; ++T) {
        const int qq = 16 * T + n16;   // the lane's query in the work group
        if (qq < nheads) {
            // acc[T][t] holds dims 16t + 4 grp .. +3 of query qq
#pragma unroll
            for (int t = 0; t < DT; ++t) *(f32x4*)&s_acc[w][qq][16 * t + 4 * grp] = acc[T][t];
            if (grp == 0) {
                s_ml[w][qq][0] = m[T];
                s_ml[w][qq][1] = l[T];
            }
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nheads * D; idx += 64 * NW) {
        const int hh = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NW; ++k) M = fmaxf(M, s_ml[k][hh][0]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const float f = s_ml[k][hh][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_ml[k][hh][0] - M);
            L = __builtin_fmaf(s_ml[k][hh][1], f, L);
            o = __builtin_fmaf(s_acc[k][hh][d], f, o);
        }
        const float res = L > 0.f ? o / L : 0.f;
        const int64_t row = query_row(hh);
        if (direct) {
            a.out[row * D + d] = f32_to_f16_bits(res);
        } else {
            const int64_t prow = row * a.max_partitions + p;
            store_once<PBQ_WS_NT>(res, &a.ws_out[prow * D + d]);
            if (d == 0) {
                store_once<PBQ_WS_NT>(M, &a.ws_ml[prow * 2]);
                store_once<PBQ_WS_NT>(L, &a.ws_ml[prow * 2 + 1]);
            }
        }
    }
}

// Merges partitions 0 .. nparts-1 of workspace row `row` into out (one
// wavefront).  Lane p holds partition p's (max, sum) and weight; the partial
// outputs are read 32 partitions at a time so that their loads are in
// flight together.
template <int D>
__device__ __forceinline__ void merge_partitions(const AttnArgs& a, int64_t row, int nparts) {
    constexpr int PER = D / 64;
    constexpr int BATCH = 32;   // 8: 12.1 us, 32: 10.1 us for 32 sequences x 32 heads x 64 partitions
    const int lane = threadIdx.x;
    const int64_t prow0 = row * a.max_partitions;
    const float* ml = a.ws_ml + prow0 * 2;
    const float* op = a.ws_out + prow0 * D + lane;

    float M = -INFINITY;
    for (int pp = lane; pp < nparts; pp += 64) M = fmaxf(M, ml[2 * pp]);
    M = wave_max(M);

    float L = 0.f;
    float o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = 0.f;
    for (int base = 0; base < nparts; base += 64) {
        const int pp = base + lane;
        float wgt = 0.f;
        if (pp < nparts) {
            const float mp = ml[2 * pp];
            wgt = mp == -INFINITY ? 0.f : ml[2 * pp + 1] * __builtin_amdgcn_exp2f(mp - M);
        }
        L += wgt;
        const int cnt = min(64, nparts - base);
        for (int i = 0; i < cnt; i += BATCH) {
            float v[BATCH][PER];
#pragma unroll
            for (int b = 0; b < BATCH; ++b)
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    v[b][k] = i + b < cnt ? op[(int64_t)(base + i + b) * D + 64 * k] : 0.f;
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const float wb = readlane(wgt, min(i + b, 63));
#pragma unroll
                for (int k = 0; k < PER; ++k) o[k] = __builtin_fmaf(wb, v[b][k], o[k]);
            }
        }
    }
    L = group_sum<64>(L);
#pragma unroll
    for (int k = 0; k < PER; ++k) a.out[row * D + lane + 64 * k] = f32_to_f16_bits(L > 0.f ? o[k] / L : 0.f);
}

// One wavefront per (query head, sequence): merges the partitions of
// sequences that have more than one.
// With a shared prefix every sequence must hold more tokens than the prefix
// (the prefix's partitions were computed over all of it); a sequence that
// does not gets a NaN row instead of a silently wrong one.
template <int BS, int D>
__global__ __launch_bounds__(64) void attn_reduce(AttnArgs a) {
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int ctx = a.context_lens[s];
    const int64_t row = (int64_t)s * a.num_q_heads + h;
    if (a.shared_tokens > 0 && ctx <= a.shared_tokens) {
        for (int d = threadIdx.x; d < D; d += 64) a.out[row * D + d] = 0x7E00u;   // fp16 NaN
        return;
    }
    const int nblk = (ctx + BS - 1) / BS;
    const int nparts = max(1, (nblk + a.partition_blocks - 1) / a.partition_blocks);
    if (nparts == 1) return;
    merge_partitions<D>(a, row, nparts);
}

// Multi-query form: one wavefront per (query head, query token, sequence);
// a query at position pos merges the partitions that hold tokens 0 .. pos.
template <int BS, int D>
__global__ __launch_bounds__(64) void attn_reduce_multi(AttnArgs a) {
    const int h = blockIdx.x;
    const int i = blockIdx.y;
    const int s = blockIdx.z;
    const int r0 = a.cu_q[s];
    const int n = a.cu_q[s + 1] - r0;
    if (i >= n) return;
    const int ctx = a.context_lens[s];
    const int PB = a.partition_blocks;
    if ((ctx + BS - 1) / BS <= PB) return;   // one partition: written directly
    const int pos = ctx - n + i;
    merge_partitions<D>(a, (int64_t)(r0 + i) * a.num_q_heads + h, (pos / BS) / PB + 1);
}

// Waves per work group of the MHA kernel: 8 when a partition holds at least
// 64 blocks, else 4, so that each wave still streams several blocks.
// join: an event the reduce waits for (the shared prefix's partitions on the
// side stream), or nullptr.
template <int BS, int D, int CP>
hipError_t launch_mha(const AttnArgs& a, hipStream_t stream, hipEvent_t join) {
    const dim3 grid = grid_dims(a.max_partitions - a.shared_parts, a.num_q_heads, a.num_seqs);
    const bool fused = a.k_new != nullptr;
    if (a.partition_blocks >= 64) {
        if (fused) hipLaunchKernelGGL((attn_partition_mha<BS, D, CP, 8, true>), grid, dim3(64 * 8), 0, stream, a);
        else hipLaunchKernelGGL((attn_partition_mha<BS, D, CP, 8, false>), grid, dim3(64 * 8), 0, stream, a);
    } else {
        if (fused) hipLaunchKernelGGL((attn_partition_mha<BS, D, CP, 4, true>), grid, dim3(64 * 4), 0, stream, a);
        else hipLaunchKernelGGL((attn_partition_mha<BS, D, CP, 4, false>), grid, dim3(64 * 4), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_partitions <= 1) return e;
    if (join && (e = hipStreamWaitEvent(stream, join, 0)) != hipSuccess) return e;
    hipLaunchKernelGGL((attn_reduce<BS, D>), dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(64), 0,
                       stream, a);
    return hipGetLastError();
}

// Work groups of one kernel that fit a compute unit at once (0 if unknown).
int groups_per_cu(const void* kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

// Whether the MHA kernel carrying the fused store fits as many work groups
// per compute unit as the plain one (looked up once per instantiation).
template <int BS, int D, int CP, int NW>
bool mha_fused_keeps_occupancy() {
    static const bool same = [] {
        const int f = groups_per_cu((const void*)&attn_partition_mha<BS, D, CP, NW, true>, 64 * NW);
        const int p = groups_per_cu((const void*)&attn_partition_mha<BS, D, CP, NW, false>, 64 * NW);
        return f > 0 && f == p;
    }();
    return same;
}

// Waves per work group of the grouped-query kernel: 2 for a single pass (the
// sequences' work groups then all fit on the GPU at once), else 4; the
// single pass with the fused store uses PBQ_GQA_FUSED_WAVES.
#ifndef PBQ_GQA_FUSED_WAVES
#define PBQ_GQA_FUSED_WAVES 3
#endif
#ifndef PBQ_GQA_SINGLE_WAVES
#define PBQ_GQA_SINGLE_WAVES 2
#endif
template <int BS, int D, int CP>
hipError_t launch_gqa(const AttnArgs& a, hipStream_t stream, hipEvent_t join) {
    const int G = a.num_q_heads / a.num_kv_heads;
    const int n_ht = (G + 15) / 16;
    // paired four-wave groups, (KV head x 16-query tile, pair of sequences):
    // single passes whose contexts fit the groups' LDS block tables (INT4 K
    // at head_dim 64 keeps its codes on the register path, which pairs do
    // not use)
    if constexpr (PBQ_GQA_PAIR && (!codec_packed4(CP / 4) || D == 128)) {
        const dim3 pg(1u, (unsigned)(a.num_kv_heads * n_ht), (unsigned)((a.num_seqs + 1) / 2));
        if (a.max_partitions == 1 && a.shared_parts == 0) {
            if constexpr (gqa_pair_lds<BS, D, CP, true>() <= kPairLdsMax) {
                if (a.k_new != nullptr) {
                    hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, 4, true, false, false, 1, true>), pg, dim3(256),
                                       0, stream, a);
                    return hipGetLastError();
                }
            }
            if (a.k_new == nullptr) {
                hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, 4, false, false, false, 1, true>), pg, dim3(256), 0,
                                   stream, a);
                return hipGetLastError();
            }
        }
    }
    const dim3 grid = grid_dims(a.max_partitions - a.shared_parts, a.num_kv_heads * n_ht, a.num_seqs);
    if (a.max_partitions == 1) {
        if (a.k_new != nullptr)
            hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, PBQ_GQA_FUSED_WAVES, true>), grid,
                               dim3(64 * PBQ_GQA_FUSED_WAVES), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, PBQ_GQA_SINGLE_WAVES, false>), grid,
                               dim3(64 * PBQ_GQA_SINGLE_WAVES), 0, stream, a);
    } else {
        hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, 4, false>), grid, dim3(64 * 4), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_partitions <= 1) return e;
    if (join && (e = hipStreamWaitEvent(stream, join, 0)) != hipSuccess) return e;
    hipLaunchKernelGGL((attn_reduce<BS, D>), dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

// The partitions of a prefix shared by every sequence: one grouped launch
// over (shared partition, KV head x 16-query tile), before the per-sequence
// partitions.
template <int BS, int D, int CP>
hipError_t launch_shared(const AttnArgs& a, hipStream_t stream) {
    const int NQ = a.num_seqs * (a.num_q_heads / a.num_kv_heads);
    const dim3 grid = grid_dims(a.shared_parts, a.num_kv_heads * ((NQ + 15) / 16), 1);
    hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, 2, false, true>), grid, dim3(64 * 2), 0, stream, a);
    return hipGetLastError();
}

// The partition launch of a multi-query call with TPW 16-query tiles per
// work group.
template <int BS, int D, int CP, int TPW>
hipError_t launch_multi_tiles(const AttnArgs& a, hipStream_t stream) {
    const int G = a.num_q_heads / a.num_kv_heads;
    // queries per work group: two-wave groups of two-tile waves share their
    // staging and take 64 (the kernel's JOINT mode), others 16 TPW
    const int QW = (a.max_partitions == 1 && TPW == 2 && PBQ_MULTI_JOINT_STAGE && !codec_packed4(CP / 4))
                       ? 64 : 16 * TPW;
    const int n_ht = (a.max_q_len * G + QW - 1) / QW;
    // x = partition, y = KV head x query tile, z = sequence (the kernel
    // renumbers the work groups over the XCDs)
    const dim3 grid((unsigned)a.max_partitions, (unsigned)(a.num_kv_heads * n_ht), (unsigned)a.num_seqs);
    if (a.max_partitions == 1)
        hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, 2, false, false, true, TPW>), grid, dim3(64 * 2), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((attn_partition_gqa<BS, D, CP, 4, false, false, true, TPW>), grid, dim3(64 * 4), 0,
                           stream, a);
    return hipGetLastError();
}

// Several query tokens per sequence: the grouped-query kernel for any group
// size (MHA included: its 16-query tiles are then 16 tokens of one head),
// over (partition, KV head x query tile, sequence), then the per-query reduce.
// Work groups take two 16-query tiles when a sequence's queries of one KV
// head fill more than one.
template <int BS, int D, int CP>
hipError_t launch_multi(const AttnArgs& a, hipStream_t stream) {
    const int G = a.num_q_heads / a.num_kv_heads;
    const hipError_t e = a.max_q_len * G > 16 ? launch_multi_tiles<BS, D, CP, 2>(a, stream)
                                              : launch_multi_tiles<BS, D, CP, 1>(a, stream);
    if (e != hipSuccess || a.max_partitions <= 1) return e;
    hipLaunchKernelGGL((attn_reduce_multi<BS, D>), dim3((unsigned)a.num_q_heads, (unsigned)a.max_q_len,
                                                        (unsigned)a.num_seqs), dim3(64), 0, stream, a);
    return hipGetLastError();
}

// A second stream per device for a shared prefix's partitions, which then
// run beside the per-sequence partitions: forked from the caller's stream
// and joined back before the reduce with events, so that a captured call
// stays one graph.  Created on first use outside a stream capture (creating
// it while the caller's stream captures could end the capture) and kept
// until the process ends; until then, or when it cannot be created, the
// prefix's partitions run on the caller's stream first.  The mutex keeps one
// call's record / wait pairs together when several host threads launch at
// once.
#ifndef PBQ_SIDE_STREAM
#define PBQ_SIDE_STREAM 1
#endif
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex mu;
};

SideStream* side_stream(hipStream_t caller) {
    static std::mutex mu;
    static std::vector<std::unique_ptr<SideStream>> per_device;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if ((int)per_device.size() <= dev) per_device.resize(dev + 1);
    if (!per_device[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
            (void)hipGetLastError();
            return nullptr;
        }
        auto ss = std::make_unique<SideStream>();
        if (hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            ss->s = nullptr;
        }
        per_device[dev] = std::move(ss);
    }
    return per_device[dev]->s ? per_device[dev].get() : nullptr;
}

template <int BS, int D, int CP>
hipError_t launch_per_sequence(const AttnArgs& a, hipStream_t stream, hipEvent_t join) {
    if (a.num_q_heads != a.num_kv_heads) return launch_gqa<BS, D, CP>(a, stream, join);
    return launch_mha<BS, D, CP>(a, stream, join);
}

template <int BS, int D, int CP>
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
    if (a.cu_q) return launch_multi<BS, D, CP>(a, stream);
    if (a.shared_parts == 0) return launch_per_sequence<BS, D, CP>(a, stream, nullptr);
    SideStream* ss = PBQ_SIDE_STREAM ? side_stream(stream) : nullptr;
    if (!ss) {
        const hipError_t e = launch_shared<BS, D, CP>(a, stream);
        return e != hipSuccess ? e : launch_per_sequence<BS, D, CP>(a, stream, nullptr);
    }
    std::lock_guard<std::mutex> lock(ss->mu);
    hipError_t e;
    if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess ||
        (e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess ||
        (e = launch_shared<BS, D, CP>(a, ss->s)) != hipSuccess || (e = hipEventRecord(ss->join, ss->s)) != hipSuccess)
        return e;
    return launch_per_sequence<BS, D, CP>(a, stream, ss->join);
}

// Whether a split-partition decode with the current token's store fuses the
// store into its partition kernel: for MHA launches whose fused kernel keeps
// the plain kernel's occupancy (otherwise the store kernel runs first).
#ifndef PBQ_SPLIT_STORE_FUSED
#define PBQ_SPLIT_STORE_FUSED 1
#endif
bool split_store_fused(const AttnArgs& a) {
    if (!PBQ_SPLIT_STORE_FUSED || a.cu_q || a.num_q_heads != a.num_kv_heads) return false;
    auto pick = [&](auto bs, auto d) {
        constexpr int BS = decltype(bs)::value, D = decltype(d)::value;
        bool same = false;
        (void)with_codec_pair(a.k_codec, a.v_codec, [&](auto cp) {
            constexpr int CP = decltype(cp)::value;
            same = a.partition_blocks >= 64 ? mha_fused_keeps_occupancy<BS, D, CP, 8>()
                                            : mha_fused_keeps_occupancy<BS, D, CP, 4>();
            return hipSuccess;
        });
        return same;
    };
    using I16 = std::integral_constant<int, 16>;
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    if (a.block_size == 16 && a.head_dim == 64) return pick(I16{}, I64{});
    if (a.block_size == 16 && a.head_dim == 128) return pick(I16{}, I128{});
    if (a.block_size == 32 && a.head_dim == 64) return pick(I32{}, I64{});
    if (a.block_size == 32 && a.head_dim == 128) return pick(I32{}, I128{});
    return false;
}

hipError_t launch_paged_attn(const AttnArgs& a, hipStream_t stream) {
#define PBQ_ATTN(BS, D)                                                       \
    if (a.block_size == BS && a.head_dim == D)                                \
        return with_codec_pair(a.k_codec, a.v_codec,                          \
                               [&](auto cp) { return launch_attn<BS, D, decltype(cp)::value>(a, stream); });
    PBQ_ATTN(16, 64)
    PBQ_ATTN(16, 128)
    PBQ_ATTN(32, 64)
    PBQ_ATTN(32, 128)
#undef PBQ_ATTN
    return hipErrorInvalidValue;
}

}  // namespace pbq

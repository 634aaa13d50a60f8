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
//    used here for the INT4 V codec (bits = 4) and, with zero point 128 and a
//    signed store, for INT8.
//  Readings: rounding is to nearest with ties to even on the exact quotient;
//  the statistics cover only the rows a block holds; the INT4 range is
//  widened to contain 0 and its zero point is an integer; rows not yet held
//  are zero bytes; a partially filled block is re-quantized from the exact
//  fp16 rows kept in its sequence's tail slot.
//
// Mapping: one wavefront per (sequence, touched block, KV head); a workgroup
// of four waves takes four consecutive heads of one block, so each token row
// is read as 4 x D x 2 contiguous bytes.  All of a wave's fp16 rows are
// loaded before any arithmetic, and reductions use DPP within rows of 16
// lanes plus readlane, so a store is a short chain: the sequence's scalars,
// the rows (with the block id beside them), the reductions, the codes.
// K tiles are token-major ([block_size, D] codes): lane l holds rows it * (64 / (D/8)) + l / (D/8) and
// dims (l % (D/8)) * 8 .. + 8.  V tiles are dim-major ([D, block_size] codes,
// INT4 packing two consecutive tokens per byte): lane l holds the D/64
// adjacent dims starting at l * D/64 of every row, so each fp16 row read and
// the lane's code rows are contiguous.
//
// Exact codes without a per-element division: n = rint(x * (1/s)) is within
// one of the answer; the remainder x - n*s is exact in one FMA (x and s are
// fp16 values, |n| <= 255), and comparing |rem| with s/2 (also exact) decides
// the nearest integer and the tie, so the result equals round-half-even of
// the exact quotient, which is what a correctly rounded fp32 division
// followed by rint gives for fp16 operands.

#include "device_common.h"
#include "pbq_internal.h"

namespace pbq {
namespace {

// Round-half-even of x / s + zp for s > 0, x and s fp16 values held in fp32.
__device__ __forceinline__ int rne_quot(float x, float s, float rcp, float half_s, int zp) {
    const float n = __builtin_rintf(x * rcp);
    const float rem = __builtin_fmaf(-n, s, x);  // exact
    const float arem = __builtin_fabsf(rem);
    const int dir = rem > 0.f ? 1 : -1;
    int q = (int)n + zp;
    q += arem > half_s ? dir : 0;                     // n was one off
    q += (arem == half_s && (q & 1)) ? dir : 0;       // exact tie -> even
    return q;
}

template <int BS, int D, bool V4>
__global__ __launch_bounds__(256) void quantize_store_kernel(QuantStoreArgs a) {
    constexpr int LPR = D / 8;     // lanes per token row
    constexpr int RPI = 64 / LPR;  // rows per wave access
    constexpr int NIT = BS / RPI;  // accesses per lane per tensor
    constexpr int DPL = D / 64;    // V: dims per lane
    const int lane = threadIdx.x & 63;
    const int g = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jj = blockIdx.y;
    const int s = blockIdx.z;   // < num_seqs by the grid

    // per-sequence scalars, all loaded before the first branch
    const int H = a.num_kv_heads;
    const int c0 = a.cu_seqlens[s];
    const int c1 = a.cu_seqlens[s + 1];
    const int sp = a.start_pos[s];
    const int slot = a.tail_slots[s];
    // keep the four loads ahead of the branch (the compiler would otherwise
    // sink each load below it and wait for them one after another)
    __asm__ volatile("" : : "s"(c0), "s"(c1), "s"(sp), "s"(slot));
    const int n_new = c1 - c0;
    const int end = sp + n_new;
    const int j = sp / BS + jj;
    if (g >= H || n_new <= 0 || j * BS >= end) return;
    const int row0 = j * BS;
    const int valid = min(BS, end - row0);   // >= 1
    const int phys = a.block_tables[(int64_t)s * a.max_blocks_per_seq + j];
    const int r_in = lane / LPR;
    const int col = (lane % LPR) * 8;

    // Row r of the block comes from the tail slot (positions before sp) or
    // from the new tokens.  Every row is loaded unconditionally -- rows past
    // `valid` read row 0 again and are then replaced by zeros -- and the
    // source is chosen arithmetically, so that all loads are in flight
    // together, beside the block id's.
    const int64_t tail_base = ((int64_t)slot * H + g) * BS * D;
    auto row_src = [&](const uint16_t* tail, const uint16_t* fresh, int r) -> const uint16_t* {
        const int rr = r < valid ? r : 0;
        const int p = row0 + rr;
        const uintptr_t t = (uintptr_t)(tail + tail_base + rr * D);
        const uintptr_t f = (uintptr_t)(fresh + ((int64_t)(c0 + p - sp) * H + g) * D);
        const uintptr_t from_tail = (uintptr_t)0 - (uintptr_t)(p < sp);
        return (const uint16_t*)(f ^ ((t ^ f) & from_tail));
    };
    f16x8 kx[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) kx[it] = *(const f16x8*)(row_src(a.tail_k, a.k, it * RPI + r_in) + col);
    uint32_t vw[BS];   // V row r: dims DPL*lane .. +DPL-1 (fp16 bits)
#pragma unroll
    for (int r = 0; r < BS; ++r) {
        const uint16_t* src = row_src(a.tail_v, a.v, r) + DPL * lane;
        vw[r] = DPL == 2 ? *(const uint32_t*)src : (uint32_t)*src;
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it)
        if (it * RPI + r_in >= valid) kx[it] = (f16x8)(_Float16)0;
    _Float16 vx[DPL][BS];
#pragma unroll
    for (int r = 0; r < BS; ++r) {
        const uint32_t w = r < valid ? vw[r] : 0u;
        vx[0][r] = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
        if constexpr (DPL == 2) vx[1][r] = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }

    const int64_t tile = (int64_t)phys * H + g;

    // ---- K: INT8 symmetric -------------------------------------------------
    {
        uint32_t amax = 0;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const uint32_t b = absmax_bits_f16x8(kx[it]);
            amax = amax > b ? amax : b;
        }
        amax = wave_max_u32_uniform(amax);
        const float absmax = bits_to_f16f((uint16_t)amax);
        const uint16_t s16 = f32_to_f16_bits(absmax / 127.0f);
        const float sc = bits_to_f16f(s16);
        const float rcp = sc > 0.f ? 1.0f / sc : 0.f;
        const float half_s = 0.5f * sc;
        int8_t* dst = a.k_codes + tile * (BS * D);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            uint32_t w[2] = {0u, 0u};
            if (sc > 0.f) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int q = rne_quot((float)kx[it][e], sc, rcp, half_s, 0);
                    q = q > 127 ? 127 : (q < -127 ? -127 : q);
                    w[e >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (e & 3));
                }
            }
            const int r = it * RPI + r_in;
            *(u32x2*)(dst + r * D + col) = u32x2{w[0], w[1]};
        }
        if (lane == 0) a.k_scale[tile] = s16;
    }

    // ---- V (dim-major tile): INT8 symmetric or INT4 asymmetric ----------------
    if constexpr (!V4) {
        uint32_t amax = 0;
#pragma unroll
        for (int k = 0; k < DPL; ++k)
#pragma unroll
            for (int r = 0; r < BS; ++r) {
                const _Float16 x = vx[k][r];
                const uint32_t b = __builtin_bit_cast(uint16_t, x) & 0x7FFFu;
                amax = amax > b ? amax : b;
            }
        amax = wave_max_u32_uniform(amax);
        const float absmax = bits_to_f16f((uint16_t)amax);
        const uint16_t s16 = f32_to_f16_bits(absmax / 127.0f);
        const float sc = bits_to_f16f(s16);
        const float rcp = sc > 0.f ? 1.0f / sc : 0.f;
        const float half_s = 0.5f * sc;
        uint8_t* dst = a.v_codes + tile * (BS * D);
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            uint32_t w[BS / 4];
#pragma unroll
            for (int i = 0; i < BS / 4; ++i) w[i] = 0u;
            if (sc > 0.f) {
#pragma unroll
                for (int r = 0; r < BS; ++r) {
                    int q = rne_quot((float)vx[k][r], sc, rcp, half_s, 0);
                    q = q > 127 ? 127 : (q < -127 ? -127 : q);
                    w[r >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (r & 3));
                }
            }
            uint32_t* drow = (uint32_t*)(dst + (DPL * lane + k) * BS);
#pragma unroll
            for (int i = 0; i < BS / 16; ++i)
                *(u32x4*)(drow + 4 * i) = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        }
        if (lane == 0) a.v_scale[tile] = s16;
    } else {
        float lo = 0.f, hi = 0.f;  // range widened to contain 0
#pragma unroll
        for (int k = 0; k < DPL; ++k)
#pragma unroll
            for (int r = 0; r < BS; ++r) {
                const float x = (float)vx[k][r];
                lo = fminf(lo, x);
                hi = fmaxf(hi, x);
            }
        lo = wave_min_uniform(lo);
        hi = wave_max_uniform(hi);
        const uint16_t s16 = f32_to_f16_bits((hi - lo) / 15.0f);
        const float sc = bits_to_f16f(s16);
        int zp = 0;
        if (sc > 0.f) {
            const float z = __builtin_rintf(-lo / sc);
            zp = z > 15.f ? 15 : (z < 0.f ? 0 : (int)z);
        }
        const float rcp = sc > 0.f ? 1.0f / sc : 0.f;
        const float half_s = 0.5f * sc;
        uint8_t* dst = a.v_codes + tile * (BS * D / 2);
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            uint32_t w[BS / 8];
#pragma unroll
            for (int i = 0; i < BS / 8; ++i) w[i] = 0u;
            if (sc > 0.f) {
#pragma unroll
                for (int r = 0; r < BS; ++r) {
                    if (r < valid) {
                        int q = rne_quot((float)vx[k][r], sc, rcp, half_s, zp);
                        q = q > 15 ? 15 : (q < 0 ? 0 : q);
                        w[r >> 3] |= (uint32_t)q << (4 * (r & 7));
                    }
                }
            }
            uint32_t* drow = (uint32_t*)(dst + (DPL * lane + k) * (BS / 2));
            if constexpr (BS == 16) {
                *(u32x2*)drow = u32x2{w[0], w[1]};
            } else {
#pragma unroll
                for (int i = 0; i < BS / 32; ++i)
                    *(u32x4*)(drow + 4 * i) = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            }
        }
        if (lane == 0) {
            a.v_scale[tile] = s16;
            a.v_zp[tile] = (uint8_t)zp;
        }
    }

    // ---- tail slot: exact rows of a block that stays partial ----------------
    if (end % BS != 0 && j == (end - 1) / BS) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int r = it * RPI + r_in;
            if (r < valid && row0 + r >= sp) *(f16x8*)(a.tail_k + tail_base + r * D + col) = kx[it];
        }
#pragma unroll
        for (int r = 0; r < BS; ++r) {
            if (r < valid && row0 + r >= sp) {
                uint16_t* t = a.tail_v + tail_base + r * D + DPL * lane;
                if constexpr (DPL == 2) {
                    const _Float16 x0 = vx[0][r], x1 = vx[1][r];
                    *(uint32_t*)t = (uint32_t)__builtin_bit_cast(uint16_t, x0) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
                } else {
                    const _Float16 x0 = vx[0][r];
                    *t = __builtin_bit_cast(uint16_t, x0);
                }
            }
        }
    }
}

// Grid: x = groups of four KV heads, y = blocks a sequence's new tokens can
// touch, z = sequences.
template <int BS, int D, bool V4>
hipError_t launch_qs(const QuantStoreArgs& a, hipStream_t stream) {
    dim3 grid((unsigned)((a.num_kv_heads + 3) / 4), (unsigned)a.tiles_per_seq, (unsigned)a.num_seqs);
    hipLaunchKernelGGL((quantize_store_kernel<BS, D, V4>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_store(const QuantStoreArgs& a, hipStream_t stream) {
    const bool v4 = a.v_codec == KV_CODEC_I4_ASYM;
#define PBQ_QS(BS, D)                                                          \
    if (a.block_size == BS && a.head_dim == D)                                 \
        return v4 ? launch_qs<BS, D, true>(a, stream) : launch_qs<BS, D, false>(a, stream);
    PBQ_QS(16, 64)
    PBQ_QS(16, 128)
    PBQ_QS(32, 64)
    PBQ_QS(32, 128)
#undef PBQ_QS
    return hipErrorInvalidValue;
}

}  // namespace pbq

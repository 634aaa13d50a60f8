// Quantization of one (block, KV head) tile from its exact fp16 rows: shared
// by the store kernel and the fused store + decode kernels, so both write
// the same bytes.
//
// The codec (web pages cited by site and section): tbr8.org "PagedAttention +
// block-wise quantization against mobile OOM", §3 and §4 store_kv -- INT8
// codes with an fp16 absmax/127 scale per (block, head); yunthe.com
// "KV-cache quantization and PagedAttention", "quantization principle" --
// Q(x) = clamp(round(x / scale + zero_point), 0, 2^bits - 1), used for INT4 V
// (bits = 4) and, with zero point 128 and a signed store, for INT8.
// Readings: round half to even on the exact quotient; statistics over the
// rows the block holds; the INT4 range widened to contain 0 with an integer
// zero point; rows not yet held are zero bytes.
//
// Lane mapping (one full wave per tile): K tiles are token-major ([bs, D]
// codes): lane l holds rows it * (64 / (D/8)) + l / (D/8) and dims
// (l % (D/8)) * 8 .. + 8.  V tiles are dim-major ([D, bs] codes, INT4 packing
// two consecutive tokens per byte): lane l holds the D/64 adjacent dims
// starting at l * D/64 of every row, so each fp16 row read and the lane's
// code rows are contiguous.
//
// Exact codes without a per-element division (Quantizer, quantizer.h): a
// fast pass that is exact except on ties, which send the wave through an
// exact routine whose result equals round-half-even of the exact quotient.
//
// Further codecs: FP8 E4M3 (yunthe.com "vLLM deployment" names the format)
// with an fp16 absmax/448 scale per (block, head), each code the E4M3 of the
// correctly rounded fp32 quotient x / scale, clamped to +-448 and converted
// by v_cvt_pk_fp8_f32 (round to nearest even); INT8 asymmetric, the INT4
// recipe with 255 levels and byte codes; and INT4 K (tbr8.org §3: blocks may
// go to INT4), the INT4 recipe on the token-major K tile, two consecutive
// head dims of a token per byte (the even dim in the low nibble).
#pragma once

#include "device_common.h"
#include "pbq_internal.h"
#include "quantizer.h"

// Cache policy of the store's row loads and code writes (1: non-temporal).
// Off: with the decode's reads the store's mixed traffic ran slower
// non-temporal (prefill 55 % against 62 % of the HBM peak).
#ifndef PBQ_STORE_NT_LOADS
#define PBQ_STORE_NT_LOADS 0
#endif
#ifndef PBQ_STORE_NT_WRITES
#define PBQ_STORE_NT_WRITES 0
#endif

namespace pbq {

// Pool arrays a tile store writes and the fp16 rows it reads.
struct TileStoreArgs {
    int8_t* k_codes;
    uint8_t* v_codes;
    uint16_t* k_scale;
    uint16_t* v_scale;
    uint8_t* v_zp;
    uint8_t* k_zp;
    uint16_t* tail_k;      // [max_seqs, H, bs, D] fp16
    uint16_t* tail_v;
    const uint16_t* k;     // new rows, token-major [T, H, D] fp16
    const uint16_t* v;
    int32_t num_kv_heads;
};

// Raw bits of the scales (and zero point) a tile store wrote -- k_scale
// carries the K zero point in its upper half for INT4 K; with LDS set, also
// what the pool held for the tile before (prev: K scale (| K zero point <<
// 16), or V scale | zero point << 16), for write_stored_tile.
struct TileScales {
    uint32_t k_scale, v_scale, v_zp, prev;
};

// Four values (already divided by the scale) -> four E4M3 bytes, the first
// in the low byte; the clamp keeps a quotient the scale's rounding pushed
// past 448 at the largest finite code.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
    auto cl = [](float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.f), 448.f); };
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
}

// The exact fp16 rows of one tensor of a tile store, as raw bits: K access
// `it` (8 dims of one row) in r[4 it .. 4 it + 3], or V row r's DPL dims in
// r[r] -- BS dwords either way.  load_tile_rows issues their loads,
// quantize_tile_rows does the rest, and store_tile is the two in a row.  The
// fused decode issues the loads before its streaming loop and quantizes after
// it, so that their latency hides behind the loop.
template <int BS>
struct TileRows {
    uint32_t r[BS];
    uint32_t prev;   // PREV: the pool's scale (| zero point << 16) before the store
};

// K (IS_K) or V rows of block j (physical id phys) of head g of a sequence
// whose rows before position sp sit in tail slot `slot` and whose rows sp ..
// end-1 are the new rows c0 .. c0 + end - sp - 1 of a.k / a.v.  Requires
// j * BS < end.  Every row is loaded unconditionally -- rows past the block's
// end read row 0 again and are replaced by zeros when quantized -- and the
// source is chosen arithmetically, so that all loads are in flight together.
// PREV: also the scale bits the pool held for the tile (write_stored_tile
// compares them).  Called by a whole wave.
template <int BS, int D, int CP, bool PREV, bool IS_K>
__device__ __forceinline__ TileRows<BS> load_tile_rows(const TileStoreArgs& a, int g, int slot, int c0, int sp,
                                                       int end, int j, int phys) {
    constexpr int LPR = D / 8;     // lanes per token row
    constexpr int RPI = 64 / LPR;  // rows per wave access
    constexpr int NIT = BS / RPI;  // K accesses per lane
    constexpr int DPL = D / 64;    // V: dims per lane
    constexpr int KC = CP / 4, VC = CP % 4;
    static_assert(4 * NIT <= BS, "K rows fit the raw registers");
    const int lane = threadIdx.x & 63;
    const int H = a.num_kv_heads;
    TileRows<BS> t;
    t.prev = 0u;
    const int row0 = j * BS;
    const int valid = min(BS, end - row0);   // >= 1
    const int r_in = lane / LPR;
    const int col = (lane % LPR) * 8;
    const int64_t tail_base = ((int64_t)slot * H + g) * BS * D;
    auto row_src = [&](const uint16_t* tail, const uint16_t* fresh, int r) -> const uint16_t* {
        const int rr = r < valid ? r : 0;
        const int p = row0 + rr;
        const uintptr_t tp = (uintptr_t)(tail + tail_base + rr * D);
        const uintptr_t f = (uintptr_t)(fresh + ((int64_t)(c0 + p - sp) * H + g) * D);
        const uintptr_t from_tail = (uintptr_t)0 - (uintptr_t)(p < sp);
        return (const uint16_t*)(f ^ ((tp ^ f) & from_tail));
    };
    const int64_t tile = (int64_t)phys * H + g;
    if constexpr (IS_K) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const u32x4 x = load_once<PBQ_STORE_NT_LOADS>((const u32x4*)(row_src(a.tail_k, a.k, it * RPI + r_in) + col));
#pragma unroll
            for (int c = 0; c < 4; ++c) t.r[4 * it + c] = x[c];
        }
        if constexpr (PREV) t.prev = a.k_scale[tile] | (codec_has_zp(KC) ? (uint32_t)a.k_zp[tile] << 16 : 0u);
    } else {
        if constexpr (PREV) t.prev = a.v_scale[tile] | (codec_has_zp(VC) ? (uint32_t)a.v_zp[tile] << 16 : 0u);
#pragma unroll
        for (int r = 0; r < BS; ++r) {
            const uint16_t* src = row_src(a.tail_v, a.v, r) + DPL * lane;
            t.r[r] = DPL == 2 ? load_once<PBQ_STORE_NT_LOADS>((const uint32_t*)src)
                              : (uint32_t)load_once<PBQ_STORE_NT_LOADS>(src);
        }
    }
    return t;
}

// Quantize the rows load_tile_rows loaded (same arguments; DO_K: K rows,
// else V rows): writes codes, scales, zero point, and -- when the sequence's
// last block stays partial -- its new rows to the tail slot.  With LDS set,
// the codes are also written to lds_k / lds_v in the tile layout.  Called by
// a whole wave.  One tensor per call: the store kernel and the fused decode
// give K and V to two waves, which halves the registers and the arithmetic
// on either's path.  With wr false nothing is written to the pool (only the
// LDS copy; write_stored_tile writes it later).
template <int BS, int D, int CP, bool LDS, bool DO_K, bool DO_V>
__device__ __forceinline__ TileScales quantize_tile_rows(const TileStoreArgs& a, const TileRows<BS>& rows, int g,
                                                         int slot, int sp, int end, int j, int phys,
                                                         int8_t* lds_k, uint8_t* lds_v, bool wr = true) {
    constexpr int LPR = D / 8;     // lanes per token row
    constexpr int RPI = 64 / LPR;  // rows per wave access
    constexpr int NIT = BS / RPI;  // accesses per lane per tensor
    constexpr int DPL = D / 64;    // V: dims per lane
    constexpr int KC = CP / 4, VC = CP % 4;
    constexpr bool V4 = codec_packed4(VC);
    static_assert(DO_K != DO_V, "one tensor per call");
    const int lane = threadIdx.x & 63;
    const int H = a.num_kv_heads;
    TileScales out{};
    out.prev = rows.prev;
    const int row0 = j * BS;
    const int valid = min(BS, end - row0);   // >= 1
    const int r_in = lane / LPR;
    const int col = (lane % LPR) * 8;
    const int64_t tail_base = ((int64_t)slot * H + g) * BS * D;
    const int64_t tile = (int64_t)phys * H + g;
    // rows past `valid` become zeros; V's fp16 values stay packed (dims
    // DPL*lane and DPL*lane + 1 in the low and high halves)
    f16x8 kx[DO_K ? NIT : 1];
    uint32_t vw[DO_V ? BS : 1];
    if constexpr (DO_K) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const u32x4 x = u32x4{rows.r[4 * it], rows.r[4 * it + 1], rows.r[4 * it + 2], rows.r[4 * it + 3]};
            kx[it] = it * RPI + r_in < valid ? __builtin_bit_cast(f16x8, x) : (f16x8)(_Float16)0;
        }
    }
    if constexpr (DO_V) {
#pragma unroll
        for (int r = 0; r < BS; ++r) vw[r] = r < valid ? rows.r[r] : 0u;
    }
    auto vx = [&](int k, int r) -> float {
        return bits_to_f16f((uint16_t)(k ? vw[r] >> 16 : vw[r] & 0xFFFFu));
    };

    // ---- K: FP8 E4M3 ----------------------------------------------------------
    if constexpr (DO_K && KC == KV_CODEC_FP8_E4M3) {
        uint32_t amax = 0;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const uint32_t b = absmax_bits_f16x8(kx[it]);
            amax = amax > b ? amax : b;
        }
        amax = wave_max_u32_uniform(amax);
        const float absmax = bits_to_f16f((uint16_t)amax);
        const uint16_t s16 = f32_to_f16_bits(absmax / 448.0f);
        const float sc = bits_to_f16f(s16);
        int8_t* dst = a.k_codes + tile * (BS * D);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            uint32_t w[2] = {0u, 0u};
            if (sc > 0.f) {   // uniform
                const f16x8 x = kx[it];
                w[0] = pack4_fp8((float)x[0] / sc, (float)x[1] / sc, (float)x[2] / sc, (float)x[3] / sc);
                w[1] = pack4_fp8((float)x[4] / sc, (float)x[5] / sc, (float)x[6] / sc, (float)x[7] / sc);
            }
            const int r = it * RPI + r_in;
            if (wr) store_once<PBQ_STORE_NT_WRITES>(u32x2{w[0], w[1]}, (u32x2*)(dst + r * D + col));
            if constexpr (LDS) *(u32x2*)(lds_k + r * D + col) = u32x2{w[0], w[1]};
        }
        if (wr && lane == 0) a.k_scale[tile] = s16;
        out.k_scale = s16;
    }

    // ---- K: INT8 symmetric -------------------------------------------------
    if constexpr (DO_K && KC == KV_CODEC_I8_SYM) {
        uint32_t amax = 0;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const uint32_t b = absmax_bits_f16x8(kx[it]);
            amax = amax > b ? amax : b;
        }
        amax = wave_max_u32_uniform(amax);
        const float absmax = bits_to_f16f((uint16_t)amax);
        const uint16_t s16 = f32_to_f16_bits(absmax / 127.0f);
        const Quantizer qz(bits_to_f16f(s16));
        int8_t* dst = a.k_codes + tile * (BS * D);
        // one access's 8 codes at a time (registers stay few); a tie anywhere
        // in the wave sends those codes through the exact routine
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            uint32_t w[2] = {0u, 0u};
            bool tie = false;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                w[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(qz.fast((float)kx[it][e], 128.f, 1.f, 255.f, tie), e & 3, w[e >> 2]);
            w[0] ^= 0x80808080u;   // offset-128 bytes -> two's complement codes
            w[1] ^= 0x80808080u;
            if (__builtin_amdgcn_ballot_w64(tie) != 0) {
                w[0] = w[1] = 0u;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int q = qz.exact((float)kx[it][e], 0);
                    q = q > 127 ? 127 : (q < -127 ? -127 : q);
                    w[e >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (e & 3));
                }
            }
            const int r = it * RPI + r_in;
            if (wr) store_once<PBQ_STORE_NT_WRITES>(u32x2{w[0], w[1]}, (u32x2*)(dst + r * D + col));
            if constexpr (LDS) *(u32x2*)(lds_k + r * D + col) = u32x2{w[0], w[1]};
        }
        if (wr && lane == 0) a.k_scale[tile] = s16;
        out.k_scale = s16;
    }

    // ---- K: INT4 asymmetric (token-major, two head dims per byte) -----------
    if constexpr (DO_K && KC == KV_CODEC_I4_ASYM) {
        // range widened to contain 0, over packed fp16 pairs (exact); rows
        // not held are zeros, which the widened range contains anyway
        f16x2 lo2 = f16x2{(_Float16)0, (_Float16)0}, hi2 = lo2;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f16x2 x = f16x2{kx[it][2 * e], kx[it][2 * e + 1]};
                lo2 = __builtin_elementwise_min(lo2, x);
                hi2 = __builtin_elementwise_max(hi2, x);
            }
        const float lo = wave_min_uniform(fminf((float)lo2[0], (float)lo2[1]));
        const float hi = wave_max_uniform(fmaxf((float)hi2[0], (float)hi2[1]));
        const uint16_t s16 = f32_to_f16_bits((hi - lo) / 15.0f);
        const Quantizer qz(bits_to_f16f(s16));
        int zp = 0;
        if (qz.s > 0.f) {
            const float z = __builtin_rintf(-lo / qz.s);
            zp = z > 15.f ? 15 : (z < 0.f ? 0 : (int)z);
        }
        const float zf = (float)zp;
        uint8_t* dst = (uint8_t*)a.k_codes + tile * (BS * D / 2);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {   // a lane's 8 dims of one row: 4 bytes
            uint32_t x = 0u;
            bool tie = false;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float u0 = qz.fast((float)kx[it][2 * b], zf, 0.f, 15.f, tie);
                const float u1 = qz.fast((float)kx[it][2 * b + 1], zf, 0.f, 15.f, tie);
                x = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(u1, 16.f, u0), b, x);
            }
            if (__builtin_amdgcn_ballot_w64(tie) != 0) {
                x = 0u;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    int q = qz.exact((float)kx[it][e], zp);
                    q = q > 15 ? 15 : (q < 0 ? 0 : q);
                    x |= (uint32_t)q << (4 * e);
                }
            }
            const int r = it * RPI + r_in;
            x = r < valid ? x : 0u;   // rows not held are zero bytes (their code would be zp)
            if (wr) store_once<PBQ_STORE_NT_WRITES>(x, (uint32_t*)(dst + r * (D / 2) + col / 2));
            if constexpr (LDS) *(uint32_t*)(lds_k + r * (D / 2) + col / 2) = x;
        }
        if (wr && lane == 0) {
            a.k_scale[tile] = s16;
            a.k_zp[tile] = (uint8_t)zp;
        }
        out.k_scale = (uint32_t)s16 | ((uint32_t)zp << 16);
    }

    // ---- V (dim-major tile): INT8 symmetric, FP8, INT4 or INT8 asymmetric ------
    if constexpr (DO_V && VC == KV_CODEC_FP8_E4M3) {
        uint32_t amax = 0;
#pragma unroll
        for (int k = 0; k < DPL; ++k)
#pragma unroll
            for (int r = 0; r < BS; ++r) {
                const uint32_t b = (k ? vw[r] >> 16 : vw[r]) & 0x7FFFu;
                amax = amax > b ? amax : b;
            }
        amax = wave_max_u32_uniform(amax);
        const float absmax = bits_to_f16f((uint16_t)amax);
        const uint16_t s16 = f32_to_f16_bits(absmax / 448.0f);
        const float sc = bits_to_f16f(s16);
        uint8_t* dst = a.v_codes + tile * (BS * D);
#pragma unroll
        for (int k = 0; k < DPL; ++k) {   // one dim row of codes at a time
            uint32_t w[BS / 4];
#pragma unroll
            for (int i = 0; i < BS / 4; ++i)
                w[i] = sc > 0.f ? pack4_fp8(vx(k, 4 * i) / sc, vx(k, 4 * i + 1) / sc, vx(k, 4 * i + 2) / sc,
                                            vx(k, 4 * i + 3) / sc)
                                : 0u;
            uint32_t* drow = (uint32_t*)(dst + (DPL * lane + k) * BS);
            uint32_t* lrow = LDS ? (uint32_t*)(lds_v + (DPL * lane + k) * BS) : nullptr;
#pragma unroll
            for (int i = 0; i < BS / 16; ++i) {
                const u32x4 x = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
                if (wr) store_once<PBQ_STORE_NT_WRITES>(x, (u32x4*)(drow + 4 * i));
                if constexpr (LDS) *(u32x4*)(lrow + 4 * i) = x;
            }
        }
        if (wr && lane == 0) a.v_scale[tile] = s16;
        out.v_scale = s16;
    } else if constexpr (DO_V && VC == KV_CODEC_I8_SYM) {
        uint32_t amax = 0;
#pragma unroll
        for (int k = 0; k < DPL; ++k)
#pragma unroll
            for (int r = 0; r < BS; ++r) {
                const uint32_t b = (k ? vw[r] >> 16 : vw[r]) & 0x7FFFu;
                amax = amax > b ? amax : b;
            }
        amax = wave_max_u32_uniform(amax);
        const float absmax = bits_to_f16f((uint16_t)amax);
        const uint16_t s16 = f32_to_f16_bits(absmax / 127.0f);
        const Quantizer qz(bits_to_f16f(s16));
        uint8_t* dst = a.v_codes + tile * (BS * D);
#pragma unroll
        for (int k = 0; k < DPL; ++k) {   // one dim row of codes at a time
            uint32_t w[BS / 4];
#pragma unroll
            for (int i = 0; i < BS / 4; ++i) {   // four codes, then their tie check
                uint32_t x = 0u;
                bool tie = false;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    x = __builtin_amdgcn_cvt_pk_u8_f32(qz.fast(vx(k, 4 * i + b), 128.f, 1.f, 255.f, tie), b, x);
                x ^= 0x80808080u;
                if (__builtin_amdgcn_ballot_w64(tie) != 0) {
                    x = 0u;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        int q = qz.exact(vx(k, 4 * i + b), 0);
                        q = q > 127 ? 127 : (q < -127 ? -127 : q);
                        x |= ((uint32_t)q & 0xFFu) << (8 * b);
                    }
                }
                w[i] = x;
            }
            uint32_t* drow = (uint32_t*)(dst + (DPL * lane + k) * BS);
            uint32_t* lrow = LDS ? (uint32_t*)(lds_v + (DPL * lane + k) * BS) : nullptr;
#pragma unroll
            for (int i = 0; i < BS / 16; ++i) {
                const u32x4 x = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
                if (wr) store_once<PBQ_STORE_NT_WRITES>(x, (u32x4*)(drow + 4 * i));
                if constexpr (LDS) *(u32x4*)(lrow + 4 * i) = x;
            }
        }
        if (wr && lane == 0) a.v_scale[tile] = s16;
        out.v_scale = s16;
    } else if constexpr (DO_V) {
        // INT4 or INT8 asymmetric: range widened to contain 0, over packed
        // fp16 pairs (exact)
        constexpr int QMAX = V4 ? 15 : 255;
        f16x2 lo2 = f16x2{(_Float16)0, (_Float16)0}, hi2 = lo2;
#pragma unroll
        for (int r = 0; r < BS; ++r) {
            const f16x2 x = __builtin_bit_cast(f16x2, vw[r]);
            lo2 = __builtin_elementwise_min(lo2, x);
            hi2 = __builtin_elementwise_max(hi2, x);
        }
        float lo = fminf((float)lo2[0], DPL == 2 ? (float)lo2[1] : 0.f);
        float hi = fmaxf((float)hi2[0], DPL == 2 ? (float)hi2[1] : 0.f);
        lo = wave_min_uniform(lo);
        hi = wave_max_uniform(hi);
        const uint16_t s16 = f32_to_f16_bits((hi - lo) / (float)QMAX);
        const Quantizer qz(bits_to_f16f(s16));
        int zp = 0;
        if (qz.s > 0.f) {
            const float z = __builtin_rintf(-lo / qz.s);
            zp = z > (float)QMAX ? QMAX : (z < 0.f ? 0 : (int)z);
        }
        const float zf = (float)zp;
        if constexpr (!V4) {
            // INT8 asymmetric: byte codes in dim rows, rows not yet held
            // (zero inputs, code zp) masked to zero bytes
            uint8_t* dst = a.v_codes + tile * (BS * D);
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
                uint32_t w[BS / 4];
#pragma unroll
                for (int i = 0; i < BS / 4; ++i) {   // four codes, then their tie check
                    uint32_t x = 0u;
                    bool tie = false;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        x = __builtin_amdgcn_cvt_pk_u8_f32(qz.fast(vx(k, 4 * i + b), zf, 0.f, 255.f, tie), b, x);
                    if (__builtin_amdgcn_ballot_w64(tie) != 0) {
                        x = 0u;
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            int q = qz.exact(vx(k, 4 * i + b), zp);
                            q = q > 255 ? 255 : (q < 0 ? 0 : q);
                            x |= (uint32_t)q << (8 * b);
                        }
                    }
                    const int held = min(max(valid - 4 * i, 0), 4);   // uniform
                    w[i] = held == 4 ? x : x & ((1u << (8 * held)) - 1u);
                }
                uint32_t* drow = (uint32_t*)(dst + (DPL * lane + k) * BS);
                uint32_t* lrow = LDS ? (uint32_t*)(lds_v + (DPL * lane + k) * BS) : nullptr;
#pragma unroll
                for (int i = 0; i < BS / 16; ++i) {
                    const u32x4 x = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
                    if (wr) store_once<PBQ_STORE_NT_WRITES>(x, (u32x4*)(drow + 4 * i));
                    if constexpr (LDS) *(u32x4*)(lrow + 4 * i) = x;
                }
            }
        } else {
            // two nibbles per byte (even row low): byte = u_even + 16 u_odd; rows
            // not yet held (zero inputs, code zp) are masked to zero nibbles
            uint8_t* dst = a.v_codes + tile * (BS * D / 2);
#pragma unroll
            for (int k = 0; k < DPL; ++k) {   // one dim row of codes at a time
                uint32_t w[BS / 8];
#pragma unroll
                for (int i = 0; i < BS / 8; ++i) {   // eight codes, then their tie check
                    uint32_t x = 0u;
                    bool tie = false;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int r = 8 * i + 2 * b;
                        const float u0 = qz.fast(vx(k, r), zf, 0.f, 15.f, tie);
                        const float u1 = qz.fast(vx(k, r + 1), zf, 0.f, 15.f, tie);
                        x = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(u1, 16.f, u0), b, x);
                    }
                    if (__builtin_amdgcn_ballot_w64(tie) != 0) {
                        x = 0u;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            int q = qz.exact(vx(k, 8 * i + e), zp);
                            q = q > 15 ? 15 : (q < 0 ? 0 : q);
                            x |= (uint32_t)q << (4 * e);
                        }
                    }
                    const int held = min(max(valid - 8 * i, 0), 8);   // uniform
                    w[i] = held == 8 ? x : x & ((1u << (4 * held)) - 1u);
                }
                uint32_t* drow = (uint32_t*)(dst + (DPL * lane + k) * (BS / 2));
                uint32_t* lrow = LDS ? (uint32_t*)(lds_v + (DPL * lane + k) * (BS / 2)) : nullptr;
                if constexpr (BS == 16) {
                    if (wr) store_once<PBQ_STORE_NT_WRITES>(u32x2{w[0], w[1]}, (u32x2*)drow);
                    if constexpr (LDS) *(u32x2*)lrow = u32x2{w[0], w[1]};
                } else {
#pragma unroll
                    for (int i = 0; i < BS / 32; ++i) {
                        const u32x4 x = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
                        if (wr) store_once<PBQ_STORE_NT_WRITES>(x, (u32x4*)(drow + 4 * i));
                        if constexpr (LDS) *(u32x4*)(lrow + 4 * i) = x;
                    }
                }
            }
        }
        if (wr && lane == 0) {
            a.v_scale[tile] = s16;
            a.v_zp[tile] = (uint8_t)zp;
        }
        out.v_scale = s16;
        out.v_zp = (uint32_t)zp;
    }

    // ---- tail slot: exact rows of a block that stays partial ----------------
    if (wr && end % BS != 0 && j == (end - 1) / BS) {
        if constexpr (DO_K) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int r = it * RPI + r_in;
                if (r < valid && row0 + r >= sp) *(f16x8*)(a.tail_k + tail_base + r * D + col) = kx[it];
            }
        }
#pragma unroll
        for (int r = 0; r < (DO_V ? BS : 0); ++r) {
            if (r < valid && row0 + r >= sp) {
                uint16_t* t = a.tail_v + tail_base + r * D + DPL * lane;
                if constexpr (DPL == 2) *(uint32_t*)t = vw[r];
                else *t = (uint16_t)vw[r];
            }
        }
    }
    return out;
}

// Quantize one tensor (DO_K or DO_V) of block j (physical id phys) of head
// g: load_tile_rows, then quantize_tile_rows (see both).  With LDS set,
// out.prev is the pool's scale bits before this store.
template <int BS, int D, int CP, bool LDS, bool DO_K, bool DO_V>
__device__ __forceinline__ TileScales store_tile(const TileStoreArgs& a, int g, int slot, int c0, int sp,
                                                 int end, int j, int phys, int8_t* lds_k, uint8_t* lds_v,
                                                 bool wr = true) {
    const TileRows<BS> rows = load_tile_rows<BS, D, CP, LDS, DO_K>(a, g, slot, c0, sp, end, j, phys);
    return quantize_tile_rows<BS, D, CP, LDS, DO_K, DO_V>(a, rows, g, slot, sp, end, j, phys, lds_k, lds_v, wr);
}

// Pool writes of a tile that store_tile quantized with wr false (codes left
// in LDS at lds_k / lds_v; sc: K scale (| K zero point << 16), V scale and
// zero point bits, then the K and the V `prev` of store_tile): wave 0 writes
// K, wave 1 V, each also
// the new row at position pos to the tail slot when its block stays partial.
// When the block already held rows (pos % bs > 0) and its scale (and zero
// point) did not change, the earlier rows' codes are unchanged -- the same
// exact rows under the same scale -- and only the new token's codes are
// written: its K row (D bytes, D / 2 for INT4), and its byte of every V dim
// row.  The fused
// decode calls it after its loop.  new_row is the row of a.k / a.v that holds
// position pos.
template <int BS, int D, int CP>
__device__ __forceinline__ void write_stored_tile(const TileStoreArgs& a, int w, int g, int slot, int new_row, int pos,
                                                  int phys, const uint8_t* lds_k, const uint8_t* lds_v,
                                                  const uint32_t* sc) {
    constexpr bool K4 = codec_packed4(CP / 4);
    constexpr bool KZP = codec_has_zp(CP / 4);
    constexpr int KROW = K4 ? D / 2 : D;   // K bytes per token row
    constexpr int KT = BS * KROW;
    constexpr bool V4 = codec_packed4(CP % 4);
    constexpr bool VZP = codec_has_zp(CP % 4);
    constexpr int VROW = V4 ? BS / 2 : BS;
    constexpr int VT = D * VROW;
    const int lane = threadIdx.x & 63;
    const int H = a.num_kv_heads;
    const int64_t tile = (int64_t)phys * H + g;
    const int r = pos % BS;
    const bool tail = r != BS - 1;   // the block stays partial
    const int64_t trow = (((int64_t)slot * H + g) * BS + r) * D;
    const int64_t nrow = ((int64_t)new_row * H + g) * D;
    if (w == 0) {
        if (r == 0 || sc[3] != sc[0]) {
#pragma unroll
            for (int c = 0; c < (KT + 1023) / 1024; ++c)
                if (KT % 1024 == 0 || 1024 * c + 16 * lane < KT)
                    *(u32x4*)(a.k_codes + tile * KT + 1024 * c + 16 * lane) = *(const u32x4*)(lds_k + 1024 * c + 16 * lane);
            if (lane == 0) {
                a.k_scale[tile] = (uint16_t)sc[0];
                if constexpr (KZP) a.k_zp[tile] = (uint8_t)(sc[0] >> 16);
            }
        } else if (lane < KROW / 16) {
            *(u32x4*)(a.k_codes + tile * KT + r * KROW + 16 * lane) = *(const u32x4*)(lds_k + r * KROW + 16 * lane);
        }
        if (tail && lane < D / 8) *(u32x4*)(a.tail_k + trow + 8 * lane) = *(const u32x4*)(a.k + nrow + 8 * lane);
    } else if (w == 1) {
        if (r == 0 || sc[4] != (sc[1] | (VZP ? sc[2] << 16 : 0u))) {
#pragma unroll
            for (int c = 0; c < (VT + 1023) / 1024; ++c)
                if (VT % 1024 == 0 || 1024 * c + 16 * lane < VT)
                    *(u32x4*)(a.v_codes + tile * VT + 1024 * c + 16 * lane) = *(const u32x4*)(lds_v + 1024 * c + 16 * lane);
            if (lane == 0) {
                a.v_scale[tile] = (uint16_t)sc[1];
                if constexpr (VZP) a.v_zp[tile] = (uint8_t)sc[2];
            }
        } else {
            const int b = V4 ? r / 2 : r;   // the new token's byte of each dim row
#pragma unroll
            for (int d = lane; d < D; d += 64) a.v_codes[tile * VT + d * VROW + b] = lds_v[d * VROW + b];
        }
        if (tail && lane < D / 8) *(u32x4*)(a.tail_v + trow + 8 * lane) = *(const u32x4*)(a.v + nrow + 8 * lane);
    }
}

}  // namespace pbq

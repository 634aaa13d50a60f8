// Host-only sweep of the store kernels' Quantizer (quantizer.h) against the
// codec's definition.  Built and run by tests/test_quantizer_sweep.py on
// the CPU; no GPU code.
//
// Definition checked (yunthe.com "KV-cache quantization and PagedAttention",
// "quantization principle": Q(x) = clamp(round(x / scale + zero_point), 0,
// 2^bits - 1); tbr8.org "PagedAttention + block-wise quantization against
// mobile OOM", §4 store_kv for the INT8 scale absmax / 127), with the
// readings of the oracle: the quotient is the fp32 division by the stored
// fp16 scale, correctly rounded, the zero point added in fp32, then round
// half to even and clamp.  Here that is plain IEEE fp32 host arithmetic.
//
// What the store kernels compute from it: per element u = fast(x, off, lo,
// hi, tie); when any element of a group flags a tie, the group's codes are
// redone as clamp(exact(x, zp)).  The sweep takes every element as its own
// group (the tie decision per element), and also checks exact() alone on
// every case.
//
// Modes:
//   i8   INT8 symmetric: every fp16 scale s that some positive finite fp16
//        absmax a gives (s = fp16(fp32(a) / 127), zero included) and every
//        finite fp16 x with |x| <= the largest such a; code in [-127, 127].
//   i4   INT4 asymmetric (QMAX 15), i8a INT8 asymmetric (QMAX 255): every
//        positive finite fp16 scale with the zero points of a main set, plus
//        every zero point for the scales whose bits are a multiple of a
//        stride; x is every finite fp16 value with x / s + zp in
//        [-1.5, QMAX + 1.5] and |x| >= s 2^-13 (below that every rule gives
//        zp, and the count would be dominated by tiny values), plus +-0.
//
// Output: one line "mode cases=N flagged=F true_ties=T bad_fast=B
// bad_exact=E"; exit status 1 when B or E is nonzero.

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <thread>
#include <vector>

#include "quantizer.h"

namespace {

float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
uint16_t f2h(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

struct Counts {
    std::atomic<uint64_t> cases{0}, flagged{0}, ties{0}, bad_fast{0}, bad_exact{0};
};

// One element under scale s (> 0) with offset/zero point zp and range
// [qlo, qhi] of codes, as the kernel computes it and as the definition does.
void check(const pbq::Quantizer& qz, float s, float x, int zp, int qlo, int qhi, bool symmetric, uint64_t& n,
           uint64_t& fl, uint64_t& tt, uint64_t& bf, uint64_t& be, uint16_t sb, uint16_t xb) {
    // definition (fp32, correctly rounded division; fp32 add of zp)
    const float t = x / s;
    const float u = t + (float)zp;
    float r = std::rint(u);
    r = r < (float)qlo ? (float)qlo : (r > (float)qhi ? (float)qhi : r);
    const int ref = (int)r;
    // the kernel's fast pass: symmetric codes carry an offset of 128
    bool tie = false;
    int got;
    if (symmetric) {
        const float v = qz.fast(x, 128.f, 1.f, 255.f, tie);
        got = (int)v - 128;
    } else {
        got = (int)qz.fast(x, (float)zp, (float)qlo, (float)qhi, tie);
    }
    int ex = qz.exact(x, zp);
    ex = ex < qlo ? qlo : (ex > qhi ? qhi : ex);
    if (tie) got = ex;
    ++n;
    fl += tie;
    tt += (std::fabs(u - std::floor(u) - 0.5f) == 0.f);
    if (got != ref) {
        if (bf < 5) fprintf(stderr, "fast mismatch s=0x%04x x=0x%04x zp=%d got %d ref %d\n", sb, xb, zp, got, ref);
        ++bf;
    }
    if (ex != ref) {
        if (be < 5) fprintf(stderr, "exact mismatch s=0x%04x x=0x%04x zp=%d got %d ref %d\n", sb, xb, zp, ex, ref);
        ++be;
    }
}

void run_parallel(int threads, int n_items, Counts& c,
                  void (*fn)(int item, uint64_t&, uint64_t&, uint64_t&, uint64_t&, uint64_t&, const void*),
                  const void* ctx) {
    std::atomic<int> next{0};
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t)
        pool.emplace_back([&]() {
            uint64_t n = 0, fl = 0, tt = 0, bf = 0, be = 0;
            for (int i; (i = next.fetch_add(1)) < n_items;) fn(i, n, fl, tt, bf, be, ctx);
            c.cases += n;
            c.flagged += fl;
            c.ties += tt;
            c.bad_fast += bf;
            c.bad_exact += be;
        });
    for (auto& th : pool) th.join();
}

// ---- INT8 symmetric ----------------------------------------------------------

struct SymCtx {
    std::vector<uint16_t> scales;   // distinct scale bits
    std::vector<float> amax;        // largest absmax giving each
};

void sym_item(int i, uint64_t& n, uint64_t& fl, uint64_t& tt, uint64_t& bf, uint64_t& be, const void* p) {
    const SymCtx& c = *(const SymCtx*)p;
    const uint16_t sb = c.scales[i];
    const float s = h2f(sb);
    const float am = c.amax[i];
    if (s == 0.f) {   // all-zero codes: the kernel's Quantizer(0) must give 0
        const pbq::Quantizer qz(0.f);
        for (uint32_t xb = 0; xb < 0x7C00u; ++xb)
            for (int sg = 0; sg < 2; ++sg) {
                const float x = h2f((uint16_t)(xb | (sg << 15)));
                if (std::fabs(x) > am) continue;
                bool tie = false;
                const int got = (int)qz.fast(x, 128.f, 1.f, 255.f, tie) - 128;
                ++n;
                if (got != 0 || tie) ++bf;
            }
        return;
    }
    const pbq::Quantizer qz(s);
    for (uint32_t xb = 0; xb < 0x7C00u; ++xb) {
        const float ax = h2f((uint16_t)xb);
        if (ax > am) break;   // positive fp16 bits are ordered by value
        for (int sg = 0; sg < 2; ++sg) {
            const uint16_t b = (uint16_t)(xb | (sg << 15));
            check(qz, s, h2f(b), 0, -127, 127, true, n, fl, tt, bf, be, sb, b);
        }
    }
}

// ---- asymmetric (INT4, INT8) -------------------------------------------------

struct AsymCtx {
    int qmax;
    std::vector<std::pair<uint16_t, int>> items;   // (scale bits, zero point)
};

void asym_item(int i, uint64_t& n, uint64_t& fl, uint64_t& tt, uint64_t& bf, uint64_t& be, const void* p) {
    const AsymCtx& c = *(const AsymCtx*)p;
    const uint16_t sb = c.items[i].first;
    const int zp = c.items[i].second;
    const float s = h2f(sb);
    const pbq::Quantizer qz(s);
    const float lo = (-(float)zp - 1.5f) * s, hi = ((float)(c.qmax - zp) + 1.5f) * s;
    const float tiny = s * 0x1p-13f;
    for (int sg = 0; sg < 2; ++sg) {
        check(qz, s, sg ? -0.f : 0.f, zp, 0, c.qmax, false, n, fl, tt, bf, be, sb, (uint16_t)(sg << 15));
        for (uint32_t xb = 1; xb < 0x7C00u; ++xb) {
            const uint16_t b = (uint16_t)(xb | (sg << 15));
            const float x = h2f(b);
            if (std::fabs(x) < tiny) continue;
            if (x > hi || x < lo) {
                if (std::fabs(x) > std::fmax(-lo, hi)) break;   // larger magnitudes only move further out
                continue;
            }
            check(qz, s, x, zp, 0, c.qmax, false, n, fl, tt, bf, be, sb, b);
        }
    }
}

}  // namespace

int main(int argc, char** argv) {
    if (argc < 2) {
        fprintf(stderr, "usage: %s i8|i4|i8a [threads]\n", argv[0]);
        return 2;
    }
    const char* mode = argv[1];
    int threads = argc > 2 ? atoi(argv[2]) : (int)std::thread::hardware_concurrency();
    if (threads < 1) threads = 1;
    Counts c;
    if (!strcmp(mode, "i8")) {
        SymCtx ctx;
        std::vector<float> amax_of(0x10000, -1.f);
        for (uint32_t ab = 1; ab < 0x7C00u; ++ab) {
            const float a = h2f((uint16_t)ab);
            const uint16_t sb = f2h(a / 127.0f);
            if (a > amax_of[sb]) amax_of[sb] = a;
        }
        for (uint32_t sb = 0; sb < 0x10000u; ++sb)
            if (amax_of[sb] >= 0.f) {
                ctx.scales.push_back((uint16_t)sb);
                ctx.amax.push_back(amax_of[sb]);
            }
        run_parallel(threads, (int)ctx.scales.size(), c, sym_item, &ctx);
        printf("i8 scales=%zu ", ctx.scales.size());
    } else if (!strcmp(mode, "i4") || !strcmp(mode, "i8a")) {
        const bool i4 = !strcmp(mode, "i4");
        AsymCtx ctx;
        ctx.qmax = i4 ? 15 : 255;
        const std::vector<int> main_zp = i4 ? std::vector<int>{0, 1, 7, 8, 14, 15} : std::vector<int>{0, 1, 128, 255};
        const uint32_t stride = i4 ? 16 : 256;
        for (uint32_t sb = 1; sb < 0x7C00u; ++sb) {
            if (sb % stride == 0) {
                for (int z = 0; z <= ctx.qmax; ++z) ctx.items.push_back({(uint16_t)sb, z});
            } else {
                for (int z : main_zp) ctx.items.push_back({(uint16_t)sb, z});
            }
        }
        run_parallel(threads, (int)ctx.items.size(), c, asym_item, &ctx);
        printf("%s items=%zu ", mode, ctx.items.size());
    } else {
        fprintf(stderr, "unknown mode %s\n", mode);
        return 2;
    }
    printf("cases=%llu flagged=%llu true_ties=%llu bad_fast=%llu bad_exact=%llu\n",
           (unsigned long long)c.cases.load(), (unsigned long long)c.flagged.load(),
           (unsigned long long)c.ties.load(), (unsigned long long)c.bad_fast.load(),
           (unsigned long long)c.bad_exact.load());
    return (c.bad_fast.load() || c.bad_exact.load()) ? 1 : 0;
}

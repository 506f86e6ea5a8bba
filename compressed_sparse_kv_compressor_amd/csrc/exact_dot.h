// exact_dot.h -- exact dot product of bf16 / OCP-e4m3 vectors, rounded once to fp32.
//
// Used by the top-k refinement: the indexer score is defined on the exact
// per-head dot product rounded once to fp32 ("DeepSeek-V4 技术解析" section 1.1
// names the Lightning Indexer; the pages print no score formula, so the library
// fixes a bit-reproducible one), and entries whose MFMA score lies too close to
// the selection threshold are rescored with this routine.
//
// Every bf16 / e4m3 value is an integer significand M times a power of two, so
// each product is P * 2^e exactly (P < 2^16).  Fast path: all products lie
// within 2^100 of the largest one, so the sum is an integer multiple of
// 2^(top-100) below 2^108 and two unsigned 128-bit accumulators (positive and
// negative terms) hold it exactly.  Otherwise (inputs spanning more than ~2^84
// in magnitude) a long fixed-point accumulator of 32-bit digits covering every
// product a bf16 pair can make is used.  Both end in one round-to-nearest-even.
//
// Compiles for the device (HIP) and for the host (plain C++), so the host build
// can be tested against the CPU oracle.
#pragma once
#include <stdint.h>
#include <stddef.h>

#if defined(__HIPCC__)
#define CSA_HD __host__ __device__ __forceinline__
#else
#define CSA_HD inline
#endif

namespace csa_exact {

typedef unsigned __int128 u128;

struct xv { uint32_t M; int e; uint32_t neg; };

CSA_HD xv decode_bf16(uint16_t h) {
    xv r;
    uint32_t E = (h >> 7) & 0xffu, f = h & 0x7fu;
    r.neg = h >> 15;
    if (E == 0) { r.M = f; r.e = -133; } else { r.M = 0x80u | f; r.e = (int)E - 134; }
    return r;
}

CSA_HD xv decode_e4m3(uint8_t b) {
    xv r;
    uint32_t E = (b >> 3) & 15u, f = b & 7u;
    r.neg = b >> 7;
    if (E == 0) { r.M = f; r.e = -9; } else { r.M = 8u | f; r.e = (int)E - 10; }
    return r;
}

CSA_HD int clz32(uint32_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __clz((int)x);
#else
    return __builtin_clz(x);
#endif
}

CSA_HD int msb128(u128 x) {  // x != 0
    uint64_t hi = (uint64_t)(x >> 64), lo = (uint64_t)x;
    if (hi) return 127 - __builtin_clzll(hi);
    return 63 - __builtin_clzll(lo);
}

CSA_HD float ldexp_f(float x, int n) { return __builtin_ldexpf(x, n); }

// Round X * 2^base (X > 0 exact) to fp32 with ties to even; apply the sign.
CSA_HD float round_to_f32(u128 X, int base, bool negative) {
    if (X == 0) return 0.0f;
    int P = msb128(X);
    int R = P - 23;
    if (R < -149 - base) R = -149 - base;
    uint32_t T;
    if (R <= 0) {                                  // every bit kept: X < 2^24, exact
        float v = ldexp_f((float)(uint32_t)X, base);
        return negative ? -v : v;
    }
    u128 t = X >> (unsigned)R;
    uint32_t rb = (uint32_t)((X >> (unsigned)(R - 1)) & 1u);
    bool sticky = (R >= 2) && ((X & ((((u128)1) << (unsigned)(R - 1)) - 1)) != 0);
    T = (uint32_t)t;
    if (rb && (sticky || (T & 1u))) T += 1;
    float v = ldexp_f((float)T, base + R);
    return negative ? -v : v;
}

// Long accumulator for the rare wide-span case: 32-bit digits in int64 lanes,
// digit 0 weighs 2^-300 (below the smallest bf16 x bf16 product, 2^-266).
template <int DT>
CSA_HD float exact_dot_wide(const void* a, const void* b, int n) {
    const int EMIN = -300, ND = 20;
    int64_t d[ND];
    for (int j = 0; j < ND; ++j) d[j] = 0;
    for (int i = 0; i < n; ++i) {
        xv x = DT == 0 ? decode_bf16(((const uint16_t*)a)[i]) : decode_e4m3(((const uint8_t*)a)[i]);
        xv y = DT == 0 ? decode_bf16(((const uint16_t*)b)[i]) : decode_e4m3(((const uint8_t*)b)[i]);
        uint64_t P = (uint64_t)x.M * y.M;
        if (!P) continue;
        int pos = x.e + y.e - EMIN;
        uint64_t v = P << (pos & 31);
        int64_t lo = (int64_t)(v & 0xffffffffu), hi = (int64_t)(v >> 32);
        if (x.neg ^ y.neg) { lo = -lo; hi = -hi; }
        d[pos >> 5] += lo;
        d[(pos >> 5) + 1] += hi;
    }
    for (int j = 0; j < ND - 1; ++j) { int64_t c = d[j] >> 32; d[j] -= c * 4294967296LL; d[j + 1] += c; }
    bool negative = d[ND - 1] < 0;
    if (negative) {
        for (int j = 0; j < ND; ++j) d[j] = -d[j];
        for (int j = 0; j < ND - 1; ++j) { int64_t c = d[j] >> 32; d[j] -= c * 4294967296LL; d[j + 1] += c; }
    }
    int J = -1;
    for (int j = ND - 1; j >= 0; --j) if (d[j]) { J = j; break; }
    if (J < 0) return 0.0f;
    int lo = J >= 3 ? J - 3 : 0;
    u128 X = 0;
    for (int j = J; j >= lo; --j) X = (X << 32) | (u128)(uint32_t)d[j];
    bool sticky = false;
    for (int j = lo - 1; j >= 0; --j) sticky |= d[j] != 0;
    if (sticky) X |= 1;                               // far below the rounding position
    return round_to_f32(X, EMIN + 32 * lo, negative);
}

// Exact sum_i a[i]*b[i], rounded once to fp32.  DT: 0 = bf16, 1 = e4m3.
template <int DT>
CSA_HD float exact_dot(const void* a, const void* b, int n) {
    int top = -100000;
    for (int i = 0; i < n; ++i) {
        xv x = DT == 0 ? decode_bf16(((const uint16_t*)a)[i]) : decode_e4m3(((const uint8_t*)a)[i]);
        xv y = DT == 0 ? decode_bf16(((const uint16_t*)b)[i]) : decode_e4m3(((const uint8_t*)b)[i]);
        uint32_t P = x.M * y.M;
        if (!P) continue;
        int t = x.e + y.e + 31 - clz32(P);
        top = t > top ? t : top;
    }
    if (top == -100000) return 0.0f;
    const int base = top - 100;
    u128 pos = 0, neg = 0;
    for (int i = 0; i < n; ++i) {
        xv x = DT == 0 ? decode_bf16(((const uint16_t*)a)[i]) : decode_e4m3(((const uint8_t*)a)[i]);
        xv y = DT == 0 ? decode_bf16(((const uint16_t*)b)[i]) : decode_e4m3(((const uint8_t*)b)[i]);
        uint32_t P = x.M * y.M;
        if (!P) continue;
        int sh = x.e + y.e - base;
        if (sh < 0) return exact_dot_wide<DT>(a, b, n);
        u128 v = ((u128)P) << (unsigned)sh;
        if (x.neg ^ y.neg) neg += v; else pos += v;
    }
    if (pos >= neg) return round_to_f32(pos - neg, base, false);
    return round_to_f32(neg - pos, base, true);
}

// Canonical indexer score of one entry: fma chain over heads of w_h * ReLU(exact dot).
template <int DT>
CSA_HD float exact_score(const void* q, const float* w, const void* k, int HI, int dI) {
    float S = 0.0f;
    const int es = DT == 0 ? 2 : 1;
    for (int h = 0; h < HI; ++h) {
        float d = exact_dot<DT>((const char*)q + (size_t)h * dI * es, k, dI);
        float r = d > 0.0f ? d : 0.0f;
        S = __builtin_fmaf(w[h], r, S);
    }
    return S;
}

}  // namespace csa_exact

// index_common.h -- device helpers shared by the indexer top-k paths (decode and prefill).
#pragma once

#include "common.h"
#include "exact_dot.h"

namespace csa {

// Entries visible to the query at absolute position p: entry j covers raw tokens
// [j m, min((j+1) m, L)) and is visible once its last token is at or before p.
__device__ __forceinline__ int n_visible(long long p, long long L, int m, int Nc) {
    if (p >= L - 1) return Nc;
    long long v = (p + 1) / m;
    return v < Nc ? (int)v : Nc;
}

// Variable-length batches: with seq_lens, sequence b holds seq_lens[b] raw tokens (clamped to [Tq, L]; L
// is the capacity that sizes the caches) and its Tq queries are its last Tq tokens; without seq_lens
// every sequence holds L tokens and query t sits at pos0 + t.  Returns the entries visible to query t.
__device__ __forceinline__ int row_visible(const long long* seq_lens, int b, int t, int Tq, long long L,
                                           long long pos0, int m, int Nc) {
    if (!seq_lens) return n_visible(pos0 + t, L, m, Nc);
    long long Lb = seq_lens[b];
    Lb = Lb < Tq ? Tq : (Lb > L ? L : Lb);
    return n_visible(Lb - Tq + t, Lb, m, (int)((Lb + m - 1) / m));
}

// Error model of the MFMA path:
//   |d~_h - d_h| <= E_h = C_DOT * A_h,  A_h = MFMA(|q_h|, |k|) ~ sum_i |q_hi k_i|
//   |S~ - S| <= sum_h |w_h| ( C_SUM (|d~_h| + E_h) + E_h ) (1 + 2^-10) + 2^-24 |S~| + 2^-126
// C_DOT: a bf16 x bf16 product is exact in fp32 (8 x 8 significant bits), so the only error of an
// MFMA dot over dI <= 128 elements is the rounding of its additions.  Whatever order the matrix
// core adds in, if every addition rounds to fp32 (unit roundoff u = 2^-24) each product passes
// through at most dI - 1 roundings before the result (the sequential chain is the worst order; the
// dI / K instructions of a row chain through the accumulator), so |d~ - d| <= gamma_(dI-1) sum|p|
// with gamma_n = n u / (1 - n u) < 128 u = 2^-17 for dI <= 128.  Measured on gfx950 the bf16 MFMAs
// stay far inside this: <= 2 u sum|p| (16x16x32) and <= 5.2 u sum|p| (32x32x16), and a GPU test
// checks the selected entries' scores against the full bound with an 8x margin.  C_SUM = 2^-19
// covers the fp32 rounding of the head reduction on both sides and the final RN32 of each exact dot.
#define C_DOT 7.62939453125e-06f    // 2^-17
#define C_SUM 1.9073486328125e-06f  // 2^-19

// Wave-cooperative exact score of entry s: HI head groups of LPH lanes, each
// lane EPL elements; per head, fixed-point window accumulation (as in
// exact_dot.h) reduced across the group, then the fma chain in head order.
// Fast path: every product of two bf16 (e4m3) values has at most 16 (8) significant bits and is
// exact in fp32 unless it underflows.  If the leading-bit exponents of a head's nonzero products
// span at most 45 - MB bits (MB = 15 or 7 bits below the leading bit), every partial sum of at
// most 2^7 of them is a multiple of the smallest product's last bit below 2^53 of it, so the fp64
// sum in any order is exact and one conversion gives RN32 of the exact dot product.  Otherwise
// (wide exponent span, or an fp32 product that underflows) the fixed-point window path below runs.
template <int DT>
__device__ __forceinline__ float raw_to_f32(const char* p, int i) {
    if (DT == 0) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
    const csa_exact::xv x = csa_exact::decode_e4m3(((const uint8_t*)p)[i]);
    const float v = ldexpf((float)x.M, x.e);
    return x.neg ? -v : v;
}

template <int DT, int DI, int HI>
__device__ float wave_exact_score(const void* qrow, const float* wrow, const void* krow) {
    using namespace csa_exact;
    constexpr int LPH = 64 / HI, EPL = DI / LPH, ES = DT == 0 ? 2 : 1;
    constexpr int MB = DT == 0 ? 15 : 7;
    static_assert(DI <= 128, "fast-path sum bound assumes at most 2^7 products per head");
    const int lane = lane_id(), h = lane / LPH, sub = lane % LPH;
    const char* qp = (const char*)qrow + ((size_t)h * DI + sub * EPL) * ES;
    const char* kp = (const char*)krow + (size_t)sub * EPL * ES;
    {
        double s = 0.0;
        int emin = 1000, emax = -1000, bad = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const float x = raw_to_f32<DT>(qp, i), y = raw_to_f32<DT>(kp, i);
            const float pr = x * y;
            const int e = (int)((__float_as_uint(pr) >> 23) & 0xffu);
            if (x != 0.0f && y != 0.0f) {
                bad |= e == 0 || e == 255;            // zero/subnormal product (maybe inexact) or overflow
                emin = min(emin, e);
                emax = max(emax, e);
            }
            s += (double)pr;
        }
#pragma unroll
        for (int o = 1; o < LPH; o <<= 1) {
            emin = min(emin, __shfl_xor(emin, o, 64));
            emax = max(emax, __shfl_xor(emax, o, 64));
            bad |= __shfl_xor(bad, o, 64);
        }
        const bool fast = !bad && emax - emin <= 45 - MB;     // uniform within a head's lanes
        if (__builtin_amdgcn_ballot_w64(!fast) == 0ull) {      // every head fast (the common case)
#pragma unroll
            for (int o = 1; o < LPH; o <<= 1) {
                const unsigned long long u = __double_as_longlong(s);
                const int lo = __shfl_xor((int)(uint32_t)u, o, 64), hi = __shfl_xor((int)(uint32_t)(u >> 32), o, 64);
                s += __longlong_as_double(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
            }
            const float d = (float)s;
            const float rr = d > 0.0f ? d : 0.0f;
            float Sx = 0.0f;
            for (int hh = 0; hh < HI; ++hh) {
                const float rh = __shfl(rr, hh * LPH, 64);
                Sx = __builtin_fmaf(wrow[hh], rh, Sx);
            }
            return Sx;
        }
    }
    uint32_t P[EPL];
    int ex[EPL];
    uint32_t ng[EPL];
    int top = -100000;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        xv x = DT == 0 ? decode_bf16(((const uint16_t*)qp)[i]) : decode_e4m3(((const uint8_t*)qp)[i]);
        xv y = DT == 0 ? decode_bf16(((const uint16_t*)kp)[i]) : decode_e4m3(((const uint8_t*)kp)[i]);
        P[i] = x.M * y.M;
        ex[i] = x.e + y.e;
        ng[i] = x.neg ^ y.neg;
        if (P[i]) top = max(top, ex[i] + 31 - (int)__clz((int)P[i]));
    }
#pragma unroll
    for (int o = 1; o < LPH; o <<= 1) top = max(top, __shfl_xor(top, o, 64));
    const int base = top - 100;
    u128 pos = 0, neg = 0;
    int wide = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        if (!P[i]) continue;
        const int sh = ex[i] - base;
        if (sh < 0) { wide = 1; continue; }
        const u128 v = ((u128)P[i]) << (unsigned)sh;
        if (ng[i]) neg += v; else pos += v;
    }
#pragma unroll
    for (int o = 1; o < LPH; o <<= 1) {
        wide |= __shfl_xor(wide, o, 64);
        uint32_t p0 = (uint32_t)pos, p1 = (uint32_t)(pos >> 32), p2 = (uint32_t)(pos >> 64), p3 = (uint32_t)(pos >> 96);
        uint32_t n0 = (uint32_t)neg, n1 = (uint32_t)(neg >> 32), n2 = (uint32_t)(neg >> 64), n3 = (uint32_t)(neg >> 96);
        p0 = __shfl_xor(p0, o, 64); p1 = __shfl_xor(p1, o, 64); p2 = __shfl_xor(p2, o, 64); p3 = __shfl_xor(p3, o, 64);
        n0 = __shfl_xor(n0, o, 64); n1 = __shfl_xor(n1, o, 64); n2 = __shfl_xor(n2, o, 64); n3 = __shfl_xor(n3, o, 64);
        pos += ((u128)p3 << 96) | ((u128)p2 << 64) | ((u128)p1 << 32) | p0;
        neg += ((u128)n3 << 96) | ((u128)n2 << 64) | ((u128)n1 << 32) | n0;
    }
    float d;
    if (wide) {
        d = exact_dot<DT>((const char*)qrow + (size_t)h * DI * ES, krow, DI);   // rare: long accumulator
    } else {
        d = pos >= neg ? round_to_f32(pos - neg, base, false) : round_to_f32(neg - pos, base, true);
    }
    const float rr = d > 0.0f ? d : 0.0f;
    float Sx = 0.0f;
    for (int hh = 0; hh < HI; ++hh) {
        const float rh = __shfl(rr, hh * LPH, 64);
        Sx = __builtin_fmaf(wrow[hh], rh, Sx);
    }
    return Sx;
}

// wave 0: find the bin (of 256, counting from the top) that holds the need-th
// largest element given the count already above; writes out[0] = bin,
// out[1] = count above that bin.
__device__ void wave_find_bin256(const uint32_t* h, uint32_t need, uint32_t above, uint32_t* out) {
    const int lane = lane_id();
    // lane L covers bins 255-4L .. 252-4L (descending)
    uint32_t c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = h[255 - 4 * lane - i]; s += c[i]; }
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    uint32_t acc = above + incl - s;
    if (acc < need && need <= acc + s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (acc + c[i] >= need) { out[0] = 255 - 4 * lane - i; out[1] = acc; break; }
            acc += c[i];
        }
    }
}

// Block-wide exclusive scan (any multiple of 64 threads, up to 1024); returns the exclusive prefix, *total the sum.
__device__ uint32_t block_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
    }
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    uint32_t wprefix = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const uint32_t c = scratch[w];
        if (w < wave) wprefix += c;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return wprefix + incl - v;
}

}  // namespace csa

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

// fp8 (OCP e4m3) pair -> bf16 pair, exact (gfx950 hardware conversion, scale 1).
template <bool HI_WORD>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t v) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI_WORD);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4_t e4m3x8_to_bf16x8(uint32_t x0, uint32_t x1) {
    return u32x4_t{e4m3x2_to_bf16x2<false>(x0), e4m3x2_to_bf16x2<true>(x0),
                   e4m3x2_to_bf16x2<false>(x1), e4m3x2_to_bf16x2<true>(x1)};
}

// MXFP4: the E8M0 scale byte as the float 2^(s - 127), and eight E2M1 codes (one dword, element 2i in the low
// nibble of byte i) times that scale as bf16 -- exact: every such value is a bf16 value for the scales the
// encoder produces (2^-127 .. 2^125).
__device__ __forceinline__ float e8m0_scale(uint32_t s) {
    return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}
__device__ __forceinline__ u32x4_t fp4x8_to_bf16x8(uint32_t x, float scale) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
#define CSA_FP4_PAIR(B) __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, scale, B))
    return u32x4_t{CSA_FP4_PAIR(0), CSA_FP4_PAIR(1), CSA_FP4_PAIR(2), CSA_FP4_PAIR(3)};
#undef CSA_FP4_PAIR
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

// Reduction over groups of G consecutive lanes (G a power of two): DPP lane moves within 16 lanes (two quad
// permutations, then the half-row and row mirrors, each of which pairs the two halves of the group so far)
// and shuffles beyond.
template <int G, typename Op>
__device__ __forceinline__ uint32_t grp_reduce(uint32_t v, Op op) {
    if (G >= 2) v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    if (G >= 4) v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    if (G >= 8) v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half mirror
    if (G >= 16) v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false)); // mirror
    if (G >= 32) v = op(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if (G >= 64) v = op(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}
template <int G>
__device__ __forceinline__ double grp_sum_f64(double s) {
    auto mv = [](double x, int ctl) -> double {
        const unsigned long long u = __double_as_longlong(x);
        int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
        if (ctl == 16 || ctl == 32) { lo = __shfl_xor(lo, ctl, 64); hi = __shfl_xor(hi, ctl, 64); }
        else {
            switch (ctl) {
            case 0xB1: lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);
                       hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false); break;
            case 0x4E: lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);
                       hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false); break;
            case 0x141: lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, false);
                        hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, false); break;
            default: lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, false);
                     hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, false); break;
            }
        }
        return __longlong_as_double(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
    };
    if (G >= 2) s += mv(s, 0xB1);
    if (G >= 4) s += mv(s, 0x4E);
    if (G >= 8) s += mv(s, 0x141);
    if (G >= 16) s += mv(s, 0x140);
    if (G >= 32) s += mv(s, 16);
    if (G >= 64) s += mv(s, 32);
    return s;
}

// The EPL elements of a lane as exact fp32 values (e4m3: the hardware conversion, a pair at a time, when the
// lane's bytes are whole dwords).
template <int DT, int EPL>
__device__ __forceinline__ void load_exact_f32(const char* p, float (&x)[EPL]) {
    if constexpr (DT == 0) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) x[i] = __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
    } else if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int j = 0; j < EPL / 4; ++j) {
            const uint32_t w = ((const uint32_t*)p)[j];
            const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
            const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
            x[4 * j] = lo[0]; x[4 * j + 1] = lo[1]; x[4 * j + 2] = hi[0]; x[4 * j + 3] = hi[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) x[i] = raw_to_f32<DT>(p, i);
    }
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
        float xq[EPL], xk[EPL];
        load_exact_f32<DT, EPL>(qp, xq);
        load_exact_f32<DT, EPL>(kp, xk);
        double s = 0.0;
        // leading-bit exponents of the nonzero products through their magnitudes' bit patterns (monotone)
        uint32_t mx = 0u, mn = 0xffffffffu, bad = 0u;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const float pr = xq[i] * xk[i];
            const uint32_t ab = __float_as_uint(pr) & 0x7fffffffu;
            const bool nz = xq[i] != 0.0f && xk[i] != 0.0f;
            // zero/subnormal product of nonzero factors (maybe inexact), or overflow
            bad |= (uint32_t)(nz && (ab < 0x00800000u || ab >= 0x7f800000u));
            mx = nz ? max(mx, ab) : mx;
            mn = nz ? min(mn, ab) : mn;
            s += (double)pr;
        }
        mx = grp_reduce<LPH>(mx, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
        mn = grp_reduce<LPH>(mn, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
        bad = grp_reduce<LPH>(bad, [](uint32_t a, uint32_t b) { return a | b; });
        const bool fast = !bad && (mn > mx || (int)(mx >> 23) - (int)(mn >> 23) <= 45 - MB);
        if (__builtin_amdgcn_ballot_w64(!fast) == 0ull) {      // every head fast (the common case)
            s = grp_sum_f64<LPH>(s);
            const float d = (float)s;
            const float rr = d > 0.0f ? d : 0.0f;
            float Sx = 0.0f;
#pragma unroll
            for (int hh = 0; hh < HI; ++hh) {
                const float rh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rr), hh * LPH));
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

// index_topk.hip -- Lightning-Indexer scoring and bit-exact per-query top-k on gfx950.
//
// Method: "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1:
// a light Lightning Indexer scores every compressed KV entry against the query
// and a top-k selector keeps the most relevant entries (Pro keeps 1024);
// "DeepSeek V4 详解" section "第一刀": every query looks only at its own top-k.
// The score of entry s for query row r (library definition, the pages print
// none): S = fma-chain_h w_h * ReLU(RN32(exact q_h . k_s)).
//
// GPU pipeline (all on the caller's stream, no host synchronisation):
//   k_fill      zero the per-row histograms and error maxima
//   k_score     MFMA (bf16 16x16x32) approximate scores S~ plus a per-entry
//               rigorous error bound; writes S~, a 2048-bin histogram of the
//               top 11 key bits, and the row's largest bound Dmax
//   k_refine<1> histogram of key bits 20..10 inside the threshold bin
//   k_refine<2> histogram of key bits 9..0 inside the threshold bin
//   k_classify  tau = exact k-th largest S~; entries with S~ > tau + 2 Dmax are
//               certainly selected, entries with S~ < tau - 2 Dmax certainly
//               not; the rest (the band) are rescored exactly (wave-cooperative
//               fixed-point dot products) in place; bitmaps "in" and "band"
//   k_finalize  per row: radix-select the remaining slots among the band by
//               (exact S desc, index asc), then compact the selected bitmap
//               into ascending indices.
// The selected set therefore equals the one defined on exact scores, whatever
// rounding the MFMA accumulation uses, provided its error stays inside the
// bound (checked on hardware by the parity tests).
#include "common.h"
#include "exact_dot.h"
#include "kernels.h"

namespace {

using namespace csa;

constexpr int BINS1 = 2048, BINS2 = 2048, BINS3 = 1024;
constexpr int HIST_WORDS = BINS1 + BINS2 + BINS3 + 1;   // + Dmax word
constexpr int TPB = 256;

__device__ __forceinline__ int n_visible(long long p, long long L, int m, int Nc) {
    if (p >= L - 1) return Nc;
    long long v = (p + 1) / m;
    return v < Nc ? (int)v : Nc;
}

// ---------------------------------------------------------------------------
// block-wide helpers
// ---------------------------------------------------------------------------
// Given a histogram in LDS (nb bins, nb % TPB == 0) find the bin b holding the
// need-th largest element: sum(h[b+1..]) < need <= sum(h[b..]).  Results in
// out[0] = b, out[1] = sum(h[b+1..]).  All threads must call.
__device__ void find_bin(const uint32_t* h, int nb, uint32_t need, uint32_t* out, uint32_t* scratch) {
    const int tid = threadIdx.x, per = nb / TPB;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i) s += h[tid * per + i];
    scratch[tid] = s;
    __syncthreads();
    // suffix sums over threads (TPB = 256): simple log-step scan in LDS
    for (int off = 1; off < TPB; off <<= 1) {
        uint32_t v = (tid + off < TPB) ? scratch[tid + off] : 0;
        __syncthreads();
        scratch[tid] += v;
        __syncthreads();
    }
    uint32_t incl = scratch[tid];            // sum of threads tid..TPB-1
    uint32_t above = incl - s;
    if (above < need && need <= incl) {
        uint32_t acc = above;
        for (int i = per - 1; i >= 0; --i) {
            uint32_t c = h[tid * per + i];
            if (acc + c >= need) { out[0] = tid * per + i; out[1] = acc; break; }
            acc += c;
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// k_fill
// ---------------------------------------------------------------------------
__global__ void k_fill(uint32_t* p, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

// ---------------------------------------------------------------------------
// k_score
// ---------------------------------------------------------------------------
// fp8 (OCP e4m3) pair -> bf16 pair, exact (gfx950 hardware conversion, scale 1).
template <bool HI_WORD>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t v) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI_WORD);
    return __builtin_bit_cast(uint32_t, r);
}

// Error model of the MFMA path (see DESIGN notes in the host file):
//   |d~_h - d_h| <= E_h = C_DOT * A_h,  A_h = MFMA(|q_h|, |k|) ~ sum_i |q_hi k_i|
//   |S~ - S| <= sum_h |w_h| ( C_SUM (|d~_h| + E_h) + E_h ) (1 + 2^-10) + 2^-126
// C_DOT = 2^-18 is 64 unit roundoffs (the bf16 MFMA measures <= 2 u sum|p| on
// gfx950); C_SUM = 2^-19 covers the fp32 rounding of the head reduction on both
// sides and of the final RN32 of each dot.
#define C_DOT 3.814697265625e-06f   // 2^-18
#define C_SUM 1.9073486328125e-06f  // 2^-19

template <int DT, int DI, int HI>
__global__ __launch_bounds__(TPB) void k_score(
    const void* __restrict__ q_idx, const float* __restrict__ w_idx, const void* __restrict__ k_idx,
    int Tq, int Nc, int NcP, long long L, int m, long long pos0, int keys_per_wg, int topk,
    float* __restrict__ S, uint32_t* __restrict__ hist)
{
    constexpr int STEPS = DI / 32;            // 16x16x32 MFMAs per 16-key tile
    constexpr int EPL = DI / 4;               // elements per lane per key row
    constexpr int KB = DT == 0 ? EPL * 2 : EPL;   // key bytes per lane
    constexpr int G = 16 / HI;                // query rows per column group
    constexpr int ES = DT == 0 ? 2 : 1;

    __shared__ uint32_t lh[2][BINS1];         // histogram for up to 2 rows of a group
    __shared__ uint32_t ldmax[2];

    const int b = blockIdx.y;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int key0 = blockIdx.x * keys_per_wg;
    const int NG = (Tq + G - 1) / G;

    for (int g = 0; g < NG; ++g) {
        // rows of this column group that need a selection at all
        const int t = g * G + col / HI, h = col % HI;
        const bool colv = t < Tq;
        const int nrow = min(G, Tq - g * G);
        const int nlds = min(nrow, 2);
        for (int i = threadIdx.x; i < 2 * BINS1; i += TPB) (&lh[0][0])[i] = 0;
        if (threadIdx.x < 2) ldmax[threadIdx.x] = 0;
        __syncthreads();

        // B operands: q and |q| for (t, h), permuted like the key loads
        bf16x8_t qb[STEPS], qa[STEPS];
        float w = 0.f;
        int nv = 0;
        if (colv) {
            const size_t r = (size_t)b * Tq + t;
            w = w_idx[r * HI + h];
            nv = n_visible(pos0 + t, L, m, Nc);
            const char* qp = (const char*)q_idx + (r * HI + h) * DI * ES + (size_t)grp * EPL * ES;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                u32x4_t v;
                if (DT == 0) {
                    v = *(const u32x4_t*)(qp + s * 16);
                } else {
                    uint32_t x0 = *(const uint32_t*)(qp + s * 8), x1 = *(const uint32_t*)(qp + s * 8 + 4);
                    v = u32x4_t{e4m3x2_to_bf16x2<false>(x0), e4m3x2_to_bf16x2<true>(x0),
                                e4m3x2_to_bf16x2<false>(x1), e4m3x2_to_bf16x2<true>(x1)};
                }
                qb[s] = as_bf16x8(v);
                qa[s] = as_bf16x8(v & 0x7fff7fffu);
            }
        } else {
#pragma unroll
            for (int s = 0; s < STEPS; ++s) { qb[s] = as_bf16x8(u32x4_t{0, 0, 0, 0}); qa[s] = qb[s]; }
        }
        const float aw = fabsf(w);
        // Rows whose whole visible prefix is selected need no scores.
        int nvmax = 0;
        {
            int v = (colv && nv > topk) ? nv : 0;
            for (int o = 1; o < 16; o <<= 1) v = max(v, __shfl_xor(v, o, 64));
            nvmax = v;
        }
        float dmax_loc = 0.f;

        const int tiles = keys_per_wg / 64;   // 16-key tiles per wave
        for (int tt = 0; tt < tiles; ++tt) {
            const int kbase = key0 + (tt * 4 + wave) * 16;   // waves interleave 16-key tiles
            if (kbase >= nvmax) break;
            const int krow = kbase + col;
            // A operands: key row krow, bytes [grp*KB, grp*KB + KB)
            u32x4_t kr[KB / 16 > 0 ? KB / 16 : 1];
            if (krow < Nc) {
                const char* kp = (const char*)k_idx + ((size_t)b * Nc + krow) * DI * ES + (size_t)grp * KB;
#pragma unroll
                for (int i = 0; i < (KB >= 16 ? KB / 16 : 1); ++i) {
                    if (KB >= 16) kr[i] = *(const u32x4_t*)(kp + i * 16);
                    else { uint2 x = *(const uint2*)kp; kr[i] = u32x4_t{x.x, x.y, 0, 0}; }
                }
            } else {
#pragma unroll
                for (int i = 0; i < (KB >= 16 ? KB / 16 : 1); ++i) kr[i] = u32x4_t{0, 0, 0, 0};
            }
            f32x4_t acc = {0, 0, 0, 0}, aacc = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                u32x4_t v;
                if (DT == 0) {
                    v = kr[s];
                } else {
                    // 8 fp8 bytes per step: dwords (2s, 2s+1) of the lane's bytes
                    const uint32_t x0 = kr[s / 2][(s & 1) * 2], x1 = kr[s / 2][(s & 1) * 2 + 1];
                    v = u32x4_t{e4m3x2_to_bf16x2<false>(x0), e4m3x2_to_bf16x2<true>(x0),
                                e4m3x2_to_bf16x2<false>(x1), e4m3x2_to_bf16x2<true>(x1)};
                }
                acc = mfma16_bf16(as_bf16x8(v), qb[s], acc);
                aacc = mfma16_bf16(as_bf16x8(v & 0x7fff7fffu), qa[s], aacc);
            }
            // lane holds d~ for keys kbase + 4*grp + j (j = 0..3) and column (t, h)
            float x[4], e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float d = acc[j];
                const float E = C_DOT * aacc[j];
                x[j] = w * fmaxf(d, 0.0f);
                e[j] = aw * (C_SUM * (fabsf(d) + E) + E);
            }
            // reduce over the HI lanes of one query row (adjacent columns)
#pragma unroll
            for (int o = 1; o < HI; o <<= 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) { x[j] += shfl_xor_f(x[j], o); e[j] += shfl_xor_f(e[j], o); }
            }
            if (colv && h == 0 && nv > topk) {
                const size_t r = (size_t)b * Tq + t;
                const int lrow = t - g * G;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = kbase + 4 * grp + j;
                    if (s < nv) {
                        const float sc = x[j] + 0.0f;            // canonical +0 for exact zero
                        S[r * NcP + s] = sc;
                        const uint32_t key = f32_key(sc);
                        if (lrow < nlds) atomicAdd(&lh[lrow][key >> 21], 1u);
                        else atomicAdd(&hist[r * HIST_WORDS + (key >> 21)], 1u);
                        const float ej = e[j] * 1.0009765625f + 1.1754943508222875e-38f;
                        dmax_loc = fmaxf(dmax_loc, ej + fabsf(sc) * 5.9604644775390625e-08f);
                    }
                }
            }
        }
        // row maxima of the error bound
        if (colv && h == 0 && nv > topk) {
            const int lrow = t - g * G;
            const size_t r = (size_t)b * Tq + t;
            if (lrow < nlds) atomicMax(&ldmax[lrow], __float_as_uint(dmax_loc));
            else atomicMax(&hist[r * HIST_WORDS + BINS1 + BINS2 + BINS3], __float_as_uint(dmax_loc));
        }
        __syncthreads();
        for (int lr = 0; lr < nlds; ++lr) {
            const size_t r = (size_t)b * Tq + g * G + lr;
            for (int i = threadIdx.x; i < BINS1; i += TPB)
                if (lh[lr][i]) atomicAdd(&hist[r * HIST_WORDS + i], lh[lr][i]);
            if (threadIdx.x == 0 && ldmax[lr]) atomicMax(&hist[r * HIST_WORDS + BINS1 + BINS2 + BINS3], ldmax[lr]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// k_refine: second and third radix levels of the threshold search
// ---------------------------------------------------------------------------
template <int LEVEL>
__global__ __launch_bounds__(TPB) void k_refine(const float* __restrict__ S, uint32_t* __restrict__ hist,
                                                int Tq, int Nc, int NcP, long long L, int m, long long pos0,
                                                int topk, int chunk)
{
    __shared__ uint32_t lh[BINS2];
    __shared__ uint32_t scratch[TPB];
    __shared__ uint32_t res[4];
    const int r = blockIdx.y;
    const int t = r % Tq;
    const int nv = n_visible(pos0 + t, L, m, Nc);
    if (nv <= topk) return;
    uint32_t* H = hist + (size_t)r * HIST_WORDS;
    for (int i = threadIdx.x; i < BINS1; i += TPB) lh[i] = H[i];
    __syncthreads();
    find_bin(lh, BINS1, (uint32_t)topk, res, scratch);
    const uint32_t b1 = res[0], above1 = res[1];
    uint32_t prefix, shift, mask, nb;
    if (LEVEL == 1) {
        prefix = b1; shift = 21; mask = BINS2 - 1; nb = BINS2;
    } else {
        __syncthreads();
        for (int i = threadIdx.x; i < BINS2; i += TPB) lh[i] = H[BINS1 + i];
        __syncthreads();
        find_bin(lh, BINS2, (uint32_t)topk - above1, res, scratch);
        prefix = (b1 << 11) | res[0]; shift = 10; mask = BINS3 - 1; nb = BINS3;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < (int)nb; i += TPB) lh[i] = 0;
    __syncthreads();
    const int s0 = blockIdx.x * chunk, s1 = min(nv, s0 + chunk);
    const float* Sr = S + (size_t)r * NcP;
    for (int s = s0 + threadIdx.x; s < s1; s += TPB) {
        const uint32_t key = f32_key(Sr[s]);
        if ((key >> shift) == prefix) {
            const uint32_t bin = LEVEL == 1 ? (key >> 10) & mask : key & mask;
            atomicAdd(&lh[bin], 1u);
        }
    }
    __syncthreads();
    uint32_t* dst = H + (LEVEL == 1 ? BINS1 : BINS1 + BINS2);
    for (int i = threadIdx.x; i < (int)nb; i += TPB)
        if (lh[i]) atomicAdd(&dst[i], lh[i]);
}

// ---------------------------------------------------------------------------
// k_classify: in / band bitmaps; exact rescoring of band entries
// ---------------------------------------------------------------------------
// Wave-cooperative exact score of entry s: HI head groups of LPH lanes, each
// lane EPL elements; per head, fixed-point window accumulation (as in
// exact_dot.h) reduced across the group, then the fma chain in head order.
template <int DT, int DI, int HI>
__device__ float wave_exact_score(const void* qrow, const float* wrow, const void* krow) {
    using namespace csa_exact;
    constexpr int LPH = 64 / HI, EPL = DI / LPH, ES = DT == 0 ? 2 : 1;
    const int lane = lane_id(), h = lane / LPH, sub = lane % LPH;
    const char* qp = (const char*)qrow + ((size_t)h * DI + sub * EPL) * ES;
    const char* kp = (const char*)krow + (size_t)sub * EPL * ES;
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

template <int DT, int DI, int HI>
__global__ __launch_bounds__(TPB) void k_classify(
    float* __restrict__ S, const uint32_t* __restrict__ hist, uint32_t* __restrict__ inb, uint32_t* __restrict__ bandb,
    const void* __restrict__ q_idx, const float* __restrict__ w_idx, const void* __restrict__ k_idx,
    int Tq, int Nc, int NcP, long long L, int m, long long pos0, int topk, int chunk)
{
    constexpr int ES = DT == 0 ? 2 : 1;
    __shared__ uint32_t lh[BINS2];
    __shared__ uint32_t scratch[TPB];
    __shared__ uint32_t res[4];
    const int r = blockIdx.y;
    const int b = r / Tq, t = r % Tq;
    const int nv = n_visible(pos0 + t, L, m, Nc);
    if (nv <= topk) return;
    const uint32_t* H = hist + (size_t)r * HIST_WORDS;
    for (int i = threadIdx.x; i < BINS1; i += TPB) lh[i] = H[i];
    __syncthreads();
    find_bin(lh, BINS1, (uint32_t)topk, res, scratch);
    const uint32_t b1 = res[0], a1 = res[1];
    __syncthreads();
    for (int i = threadIdx.x; i < BINS2; i += TPB) lh[i] = H[BINS1 + i];
    __syncthreads();
    find_bin(lh, BINS2, (uint32_t)topk - a1, res, scratch);
    const uint32_t b2 = res[0], a2 = res[1];
    __syncthreads();
    for (int i = threadIdx.x; i < BINS3; i += TPB) lh[i] = H[BINS1 + BINS2 + i];
    __syncthreads();
    find_bin(lh, BINS3, (uint32_t)topk - a1 - a2, res, scratch);
    const uint32_t b3 = res[0];
    const float tau = key_f32((b1 << 21) | (b2 << 10) | b3);
    const float dmax = __uint_as_float(H[BINS1 + BINS2 + BINS3]);
    const double lo = (double)tau - 2.0 * (double)dmax, hi = (double)tau + 2.0 * (double)dmax;

    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int s0 = blockIdx.x * chunk, s1 = min(NcP, s0 + chunk);     // chunk % 64 == 0
    float* Sr = S + (size_t)r * NcP;
    const char* qrow = (const char*)q_idx + (size_t)r * HI * DI * ES;
    const float* wrow = w_idx + (size_t)r * HI;
    for (int base = s0 + wave * 64; base < s1; base += TPB) {
        const int s = base + lane;
        bool isin = false, isband = false;
        if (s < nv) {
            const double v = (double)Sr[s];
            isin = v > hi;
            isband = !isin && v >= lo;
        }
        const unsigned long long bin = __ballot(isin), bband = __ballot(isband);
        if (lane == 0) {
            inb[(size_t)r * (NcP / 32) + base / 32] = (uint32_t)bin;
            inb[(size_t)r * (NcP / 32) + base / 32 + 1] = (uint32_t)(bin >> 32);
            bandb[(size_t)r * (NcP / 32) + base / 32] = (uint32_t)bband;
            bandb[(size_t)r * (NcP / 32) + base / 32 + 1] = (uint32_t)(bband >> 32);
        }
        unsigned long long todo = bband;
        while (todo) {
            const int j = __ffsll((long long)todo) - 1;
            todo &= todo - 1;
            const int e = base + j;
            const float sx = wave_exact_score<DT, DI, HI>(qrow, wrow, (const char*)k_idx + ((size_t)b * Nc + e) * DI * ES);
            if (lane == 0) Sr[e] = sx;
        }
    }
}

// ---------------------------------------------------------------------------
// k_finalize: one workgroup per query row
// ---------------------------------------------------------------------------
constexpr int FTPB = 512;

__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    // sh: FTPB words
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < FTPB; off <<= 1) {
        uint32_t x = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += x;
        __syncthreads();
    }
    const uint32_t incl = sh[tid];
    *total = sh[FTPB - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(FTPB) void k_finalize(const float* __restrict__ S, const uint32_t* __restrict__ inb,
                                                   const uint32_t* __restrict__ bandb, int Tq, int Nc, int NcP,
                                                   long long L, int m, long long pos0, int topk,
                                                   int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out)
{
    __shared__ uint32_t sh[FTPB];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t res[4];
    const int r = blockIdx.x, t = r % Tq, tid = threadIdx.x;
    const int nv = n_visible(pos0 + t, L, m, Nc);
    int32_t* out = idx_out + (size_t)r * topk;
    if (nv <= topk) {
        for (int i = tid; i < topk; i += FTPB) out[i] = i < nv ? i : -1;
        if (cnt_out && tid == 0) cnt_out[r] = nv;
        return;
    }
    const int NW = NcP / 32;
    const int per = (NW + FTPB - 1) / FTPB;
    const int w0 = min(NW, tid * per), w1 = min(NW, w0 + per);
    const uint32_t* IB = inb + (size_t)r * NW;
    const uint32_t* BB = bandb + (size_t)r * NW;
    const float* Sr = S + (size_t)r * NcP;
    uint32_t total;
    uint32_t nin = 0, nband = 0;
    for (int w = w0; w < w1; ++w) { nin += __popc(IB[w]); nband += __popc(BB[w]); }
    block_excl_scan(nin, sh, &total);
    const uint32_t n_in = total;
    block_excl_scan(nband, sh, &total);
    const uint32_t n_band = total;
    const uint32_t need = (uint32_t)topk - n_in;            // 0 <= need <= n_band by construction
    // exact threshold among band entries: need-th largest key (radix, 8 bits per pass)
    uint32_t prefix = 0, above = 0;
    bool all_band = need == n_band;
    if (need > 0 && !all_band) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int i = tid; i < 256; i += FTPB) hist[i] = 0;
            __syncthreads();
            for (int w = w0; w < w1; ++w) {
                uint32_t bits = BB[w];
                while (bits) {
                    const int j = __ffs((int)bits) - 1;
                    bits &= bits - 1;
                    const uint32_t key = f32_key(Sr[w * 32 + j]);
                    const bool match = pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8));
                    if (match) atomicAdd(&hist[(key >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t acc = above;
                for (int bin = 255; bin >= 0; --bin) {
                    if (acc + hist[bin] >= need) { res[0] = bin; res[1] = acc; break; }
                    acc += hist[bin];
                }
            }
            __syncthreads();
            prefix |= res[0] << shift;
            above = res[1];
            __syncthreads();
        }
    }
    const uint32_t need_eq = need - above;   // ties at the threshold key, taken by ascending index
    // count ties in my range, scan, then build the selected words and compact
    uint32_t nties = 0;
    if (need > 0 && !all_band) {
        for (int w = w0; w < w1; ++w) {
            uint32_t bits = BB[w];
            while (bits) {
                const int j = __ffs((int)bits) - 1;
                bits &= bits - 1;
                nties += f32_key(Sr[w * 32 + j]) == prefix;
            }
        }
    }
    uint32_t tie_rank = block_excl_scan(nties, sh, &total);
    uint32_t nsel = 0;
    // first pass: count selected in my range
    for (int pass = 0; pass < 2; ++pass) {
        uint32_t tr = tie_rank;
        uint32_t pos = 0;
        if (pass == 1) pos = block_excl_scan(nsel, sh, &total);
        for (int w = w0; w < w1; ++w) {
            uint32_t sel = IB[w];
            uint32_t bits = BB[w];
            if (need > 0) {
                if (all_band) sel |= bits;
                else {
                    while (bits) {
                        const int j = __ffs((int)bits) - 1;
                        bits &= bits - 1;
                        const uint32_t key = f32_key(Sr[w * 32 + j]);
                        if (key > prefix) sel |= 1u << j;
                        else if (key == prefix) { if (tr < need_eq) sel |= 1u << j; ++tr; }
                    }
                }
            }
            if (pass == 0) nsel += __popc(sel);
            else {
                while (sel) {
                    const int j = __ffs((int)sel) - 1;
                    sel &= sel - 1;
                    out[pos++] = w * 32 + j;
                }
            }
        }
    }
    if (cnt_out && tid == 0) cnt_out[r] = topk;
}

}  // namespace

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t index_topk_ws_bytes(int B, int Tq, int Nc) {
    const size_t R = (size_t)B * Tq;
    const size_t NcP = ((size_t)Nc + 63) / 64 * 64;
    return align256(R * NcP * 4) + align256(R * HIST_WORDS * 4) + 2 * align256(R * (NcP / 32) * 4);
}

template <int DT, int DI, int HI>
static int launch_index(const void* q_idx, const float* w_idx, const void* k_idx, int B, int Tq, int Nc,
                        long long L, int m, long long pos0, int topk, int32_t* idx_out, int32_t* cnt_out,
                        void* ws, hipStream_t st) {
    const size_t R = (size_t)B * Tq;
    const int NcP = (Nc + 63) / 64 * 64;
    char* p = (char*)ws;
    float* S = (float*)p;            p += align256(R * (size_t)NcP * 4);
    uint32_t* hist = (uint32_t*)p;   p += align256(R * HIST_WORDS * 4);
    uint32_t* inb = (uint32_t*)p;    p += align256(R * (size_t)(NcP / 32) * 4);
    uint32_t* bandb = (uint32_t*)p;
    {
        const size_t n = R * HIST_WORDS;
        int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
        CSA_LAUNCH("k_fill", k_fill, dim3(blocks), dim3(256), 0, st, hist, n);
    }
    // scoring: 1024 keys per workgroup (4 waves x 16 tiles of 16)
    const int kpw = 1024;
    dim3 g1((Nc + kpw - 1) / kpw, B);
    CSA_LAUNCH("k_score", (k_score<DT, DI, HI>), g1, dim3(TPB), 0, st,
               q_idx, w_idx, k_idx, Tq, Nc, NcP, L, m, pos0, kpw, topk, S, hist);
    const int chunk = 4096;
    dim3 g2((NcP + chunk - 1) / chunk, (unsigned)R);
    CSA_LAUNCH("k_refine1", k_refine<1>, g2, dim3(TPB), 0, st, S, hist, Tq, Nc, NcP, L, m, pos0, topk, chunk);
    CSA_LAUNCH("k_refine2", k_refine<2>, g2, dim3(TPB), 0, st, S, hist, Tq, Nc, NcP, L, m, pos0, topk, chunk);
    CSA_LAUNCH("k_classify", (k_classify<DT, DI, HI>), g2, dim3(TPB), 0, st, S, hist, inb, bandb,
               q_idx, w_idx, k_idx, Tq, Nc, NcP, L, m, pos0, topk, chunk);
    CSA_LAUNCH("k_finalize", k_finalize, dim3((unsigned)R), dim3(FTPB), 0, st, S, inb, bandb, Tq, Nc, NcP,
               L, m, pos0, topk, idx_out, cnt_out);
    return 0;
}

int index_topk_launch(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B, int Tq,
                      int HI, int dI, int Nc, long long L, int m, long long pos0, int topk,
                      int32_t* idx_out, int32_t* cnt_out, void* ws, hipStream_t st) {
#define CSA_IDX_CASE(DT, DI, HI_)                                                              \
    if (dtype == DT && dI == DI && HI == HI_)                                                  \
        return launch_index<DT, DI, HI_>(q_idx, w_idx, k_idx, B, Tq, Nc, L, m, pos0, topk,     \
                                         idx_out, cnt_out, ws, st);
#define CSA_IDX_HI(DT, DI) CSA_IDX_CASE(DT, DI, 1) CSA_IDX_CASE(DT, DI, 2) CSA_IDX_CASE(DT, DI, 4) \
                           CSA_IDX_CASE(DT, DI, 8) CSA_IDX_CASE(DT, DI, 16)
    CSA_IDX_HI(0, 64) CSA_IDX_HI(0, 128) CSA_IDX_HI(1, 64) CSA_IDX_HI(1, 128)
#undef CSA_IDX_HI
#undef CSA_IDX_CASE
    return fail(6, "index_topk: unsupported (dtype %d, dI %d, HI %d)", dtype, dI, HI);
}

__global__ void k_fp8_to_bf16(const uint32_t* in, uint32_t* out, int nwords) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nwords) {
        out[2 * i] = e4m3x2_to_bf16x2<false>(in[i]);
        out[2 * i + 1] = e4m3x2_to_bf16x2<true>(in[i]);
    }
}

int fp8_to_bf16_launch(const void* in, void* out, int n, hipStream_t st) {
    const int nw = n / 4;
    CSA_LAUNCH("k_fp8_to_bf16", k_fp8_to_bf16, dim3((nw + 255) / 256), dim3(256), 0, st,
               (const uint32_t*)in, (uint32_t*)out, nw);
    return 0;
}

}  // namespace csa_host

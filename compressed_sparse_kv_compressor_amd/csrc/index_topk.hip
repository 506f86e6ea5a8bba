// index_topk.hip -- Lightning-Indexer scoring and bit-exact per-query top-k on gfx950.
//
// Method: "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1:
// a light Lightning Indexer scores every compressed KV entry against the query
// and a top-k selector keeps the most relevant entries (Pro keeps 1024);
// "DeepSeek V4 详解" section "第一刀": every query looks only at its own top-k.
// The score of entry s for query row r (library definition; the pages print
// none): S = fma-chain_h w_h * ReLU(RN32(exact q_h . k_s)).
//
// GPU pipeline (all on the caller's stream, no host synchronisation):
//   k_fill     zero the per-row histogram, error maximum and candidate count
//   k_score    the HBM-bound pass: v_mfma_f32_16x16x32_bf16 approximate scores
//              S~ (e4m3 keys are widened to bf16 exactly in registers), a
//              rigorous per-entry error bound from a second MFMA on |q|, |k|,
//              a 4096-bin histogram of the top 12 bits of S~ and the row's
//              largest bound Dmax
//   k_collect  every entry that can still reach the top-k (S~ >= lower edge of
//              the bin holding the k-th largest, minus 2 Dmax) -> a per-row
//              candidate list of (index, S~)
//   k_select   one workgroup per row: exact k-th largest S~ (tau) from the two
//              histogram levels plus an 8-bit third level over the candidates;
//              S~ > tau + 2 Dmax is certainly selected, S~ < tau - 2 Dmax
//              certainly not; the band in between is rescored exactly
//              (wave-cooperative exact dot products) and its remaining slots go
//              by (exact S desc, index asc); the candidates are kept in index
//              order, so one prefix scan writes the k indices ascending.
// Why the classification is safe.  Let every entry satisfy |S~_s - S_s| <= D
// (D = Dmax of the row) and let tau be the k-th largest S~ (so fewer than k
// entries have S~ > tau and at least k have S~ >= tau).
//  * S~_s < tau - 2D: at least k entries t have S_t >= S~_t - D >= tau - D >
//    S~_s + D >= S_s, i.e. k entries beat s strictly, so s is not selected.
//  * S~_s > tau + 2D: any t with S_t >= S_s has S~_t >= S_t - D >= S_s - D >=
//    S~_s - 2D > tau; fewer than k entries (s included) have S~ > tau, so at most
//    k-1 entries can precede s in the order, so s is selected.
//  * entries in between (the band) get their exact score, and the slots left
//    after the certain ones go to the band by (exact S desc, index asc).
// The selected set therefore equals the one defined on exact scores whatever
// order the MFMA accumulates in, provided its error stays inside the bound.
#include "common.h"
#include "exact_dot.h"
#include "index_common.h"
#include "kernels.h"

namespace {

using namespace csa;

constexpr int BINS1 = 4096;                  // histogram of key bits 31..20
constexpr int BINS2 = 4096;                  // histogram of key bits 19..8 inside the threshold bin
constexpr int HW_DMAX = BINS1 + BINS2, HW_CNT = BINS1 + BINS2 + 1;   // row max error bound; candidate count
constexpr int HW_B1 = BINS1 + BINS2 + 2, HW_A1 = BINS1 + BINS2 + 3;    // level-1 bin of tau; count above it
constexpr int HIST_WORDS = BINS1 + BINS2 + 8;
constexpr int TPB = 256;


// Given a histogram in LDS (nb bins, nb % TPB == 0) find the bin b holding the
// need-th largest element: sum(h[b+1..]) < need <= sum(h[b..]).  Results in
// out[0] = b, out[1] = sum(h[b+1..]).  All threads of a TPB-wide block call.
__device__ void find_bin(const uint32_t* h, int nb, uint32_t need, uint32_t* out, uint32_t* scratch) {
    const int tid = threadIdx.x, per = nb / TPB, lane = tid & 63, wave = tid >> 6;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i) s += h[tid * per + i];
    uint32_t incl = s;                                  // suffix sum within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(incl, o, 64);
        if (lane + o < 64) incl += v;
    }
    if (lane == 0) scratch[wave] = incl;
    __syncthreads();
    for (int w = wave + 1; w < TPB / 64; ++w) incl += scratch[w];
    const uint32_t above = incl - s;
    if (above < need && need <= incl) {
        uint32_t acc = above;
        for (int i = per - 1; i >= 0; --i) {
            const uint32_t c = h[tid * per + i];
            if (acc + c >= need) { out[0] = tid * per + i; out[1] = acc; break; }
            acc += c;
        }
    }
    __syncthreads();
}

// find_bin for a 1024-thread block over BINS1 = 4096 bins (4 per thread).
__device__ void find_bin_wide(const uint32_t* h, uint32_t need, uint32_t* out, uint32_t* scratch) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int per = BINS1 / blockDim.x;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i) s += h[tid * per + i];
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(incl, o, 64);
        if (lane + o < 64) incl += v;
    }
    if (lane == 0) scratch[wave] = incl;
    __syncthreads();
    for (int w = wave + 1; w < nw; ++w) incl += scratch[w];
    const uint32_t above = incl - s;
    if (above < need && need <= incl) {
        uint32_t acc = above;
        for (int i = per - 1; i >= 0; --i) {
            const uint32_t c = h[tid * per + i];
            if (acc + c >= need) { out[0] = tid * per + i; out[1] = acc; break; }
            acc += c;
        }
    }
    __syncthreads();
}

__global__ void k_fill(uint32_t* p, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
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


// ---------------------------------------------------------------------------
// k_score
// ---------------------------------------------------------------------------
// MFMA roles: A = 16 query columns (row t, head h; heads padded to HP = max(HI, 4)),
// B = 16 keys, both loaded as 1/4 of a row per lane (the same k-slot order),
// so D[column][key] leaves every lane with HP/4... 4 heads of one key: the
// head reduction is mostly lane-local (one xor-16 shuffle for HP = 8).
template <int DT, int DI, int HI>
__global__ __launch_bounds__(TPB) void k_score(
    const void* __restrict__ q_idx, const float* __restrict__ w_idx, const void* __restrict__ k_idx,
    int Tq, int Nc, int NcP, long long L, int m, long long pos0, int keys_per_wg, int topk,
    float* __restrict__ S, uint32_t* __restrict__ hist)
{
    constexpr int STEPS = DI / 32;            // bf16 16x16x32 MFMAs per 16-key tile
    constexpr int EPL = DI / 4;               // key elements per lane
    constexpr int KB = DT == 0 ? EPL * 2 : EPL;   // key bytes per lane
    constexpr int NV = KB / 16;               // 16-byte loads per lane per tile
#ifndef CSA_SCORE_BATCH_BYTES
#define CSA_SCORE_BATCH_BYTES 128
#endif
    constexpr int U = CSA_SCORE_BATCH_BYTES / KB;   // tiles per load batch (bytes per lane in flight)
    constexpr int HP = HI < 4 ? 4 : HI;       // padded heads per query row
    constexpr int G = 16 / HP;                // query rows per column group
    constexpr int LPR = HP / 4;               // lanes (of one key) holding one row's heads
    constexpr int ES = DT == 0 ? 2 : 1;

    __shared__ uint32_t lh[2][BINS1];         // histograms of up to 2 rows of a group
    __shared__ uint32_t ldmax[2];

    const int b = blockIdx.y;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int key0 = blockIdx.x * keys_per_wg;
    const int NG = (Tq + G - 1) / G;
    const int tiles = keys_per_wg / 64;       // 16-key tiles per wave

    for (int g = 0; g < NG; ++g) {
        const int nrow = min(G, Tq - g * G);
        const int nlds = min(nrow, 2);
        for (int i = threadIdx.x; i < nlds * BINS1; i += TPB) (&lh[0][0])[i] = 0;
        if (threadIdx.x < 2) ldmax[threadIdx.x] = 0;
        __syncthreads();

        // A operand: query column `col` = (row ta, head ha)
        const int ta = g * G + col / HP, ha = col % HP;
        const bool av = ta < Tq && ha < HI;
        bf16x8_t qb[STEPS], qa[STEPS];
        u32x4_t qf8a[2];                      // |q| as raw e4m3 bytes (DT == 1)
        // Element order of the contraction (shared by Q and K): lane group grp takes the 16-byte chunks
        // at bytes 64 i + 16 grp of a row, so that one load instruction reads 64 contiguous bytes of
        // each of its 16 key rows.  bf16: k-step s = chunk s; e4m3: k-step s = half (s & 1) of chunk s / 2.
        if (av) {
            const size_t r = (size_t)b * Tq + ta;
            const char* qp = (const char*)q_idx + (r * HI + ha) * DI * ES + (size_t)grp * 16;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                u32x4_t v;
                if (DT == 0) v = *(const u32x4_t*)(qp + s * 64);
                else {
                    const char* c = qp + (s >> 1) * 64 + (s & 1) * 8;
                    v = e4m3x8_to_bf16x8(*(const uint32_t*)c, *(const uint32_t*)(c + 4));
                }
                qb[s] = as_bf16x8(v);
                qa[s] = as_bf16x8(v & 0x7fff7fffu);
            }
            if (DT == 1) {
                qf8a[0] = (*(const u32x4_t*)qp) & 0x7f7f7f7fu;
                qf8a[1] = DI == 128 ? (*(const u32x4_t*)(qp + 64)) & 0x7f7f7f7fu : u32x4_t{0, 0, 0, 0};
            }
        } else {
#pragma unroll
            for (int s = 0; s < STEPS; ++s) { qb[s] = as_bf16x8(u32x4_t{0, 0, 0, 0}); qa[s] = qb[s]; }
            qf8a[0] = qf8a[1] = u32x4_t{0, 0, 0, 0};
        }
        // output side: this lane's 4 columns 4*grp + j all belong to row tr
        const int tr = g * G + (4 * grp) / HP;
        const bool rv = tr < Tq;
        const size_t r = (size_t)b * Tq + (rv ? tr : 0);
        float w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hh = (4 * grp + j) % HP;
            w4[j] = (rv && hh < HI) ? w_idx[r * HI + hh] : 0.f;
        }
        const int nv = rv ? n_visible(pos0 + tr, L, m, Nc) : 0;
        const bool need_sel = rv && nv > topk;
        const bool writer = need_sel && (grp % LPR) == 0;
        int nvmax;                            // keys any row of the group needs scored
        {
            int v = need_sel ? nv : 0;
            v = max(v, __shfl_xor(v, 16, 64));
            v = max(v, __shfl_xor(v, 32, 64));
            nvmax = v;
        }
        float dmax_loc = 0.f;
        const int lrow = tr - g * G;

        // key loads are software-pipelined: batch i+1 is in flight while batch i computes
        // (rows past the end reread the last row: branch-free loads keep the wait counts exact, so the
        //  next batch stays in flight; those keys are never written)
        auto load_batch = [&](int tt0, u32x4_t (&dst)[U][NV]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int krow = min(key0 + ((tt0 + u) * 4 + wave) * 16 + col, Nc - 1);
                const char* kp = (const char*)k_idx + ((size_t)b * Nc + krow) * DI * ES + (size_t)grp * 16;
#pragma unroll
                for (int i = 0; i < NV; ++i) dst[u][i] = *(const u32x4_t*)(kp + i * 64);
            }
        };
        auto compute_batch = [&](int tt0, const u32x4_t (&cur)[U][NV]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                    // (tiles past the visible keys are computed and dropped: no branch between the
                    //  loads and their uses)
                    const int kbase = key0 + ((tt0 + u) * 4 + wave) * 16;
                    f32x4_t acc = {0, 0, 0, 0}, aacc = {0, 0, 0, 0};
#pragma unroll
                    for (int s = 0; s < STEPS; ++s) {
                        u32x4_t v;
                        if (DT == 0) v = cur[u][s];
                        else v = e4m3x8_to_bf16x8(cur[u][s / 2][(s & 1) * 2], cur[u][s / 2][(s & 1) * 2 + 1]);
                        acc = mfma16_bf16(qb[s], as_bf16x8(v), acc);
                        if (DT == 0) aacc = mfma16_bf16(qa[s], as_bf16x8(v & 0x7fff7fffu), aacc);
                    }
                    if (DT == 1) {
                        // |q|.|k| bound: one e4m3 MFMA (K = 128) on the raw bytes with the sign bits cleared
                        typedef __attribute__((ext_vector_type(8))) int i32x8_t;
                        const u32x4_t k0 = cur[u][0] & 0x7f7f7f7fu;
                        const u32x4_t k1 = NV > 1 ? cur[u][NV > 1 ? 1 : 0] & 0x7f7f7f7fu : u32x4_t{0, 0, 0, 0};
                        const i32x8_t A8 = {(int)qf8a[0][0], (int)qf8a[0][1], (int)qf8a[0][2], (int)qf8a[0][3],
                                            (int)qf8a[1][0], (int)qf8a[1][1], (int)qf8a[1][2], (int)qf8a[1][3]};
                        const i32x8_t B8 = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                                            (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
                        aacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A8, B8, aacc, 0, 0, 0, 127, 0, 127);
                    }
                    // lane: key kbase + col, columns 4*grp + j of row tr
                    float x = 0.f, e = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float d = acc[j];
                        // all-positive e4m3 MFMA sums are inflated by 2^-8 for its reduced-precision accumulation
                        const float E = C_DOT * (DT == 1 ? aacc[j] * 1.00390625f : aacc[j]);
                        x = fmaf(w4[j], fmaxf(d, 0.0f), x);
                        e = fmaf(fabsf(w4[j]), C_SUM * (fabsf(d) + E) + E, e);
                    }
                    if (LPR >= 2) { x += shfl_xor_f(x, 16); e += shfl_xor_f(e, 16); }
                    if (LPR >= 4) { x += shfl_xor_f(x, 32); e += shfl_xor_f(e, 32); }
                    const int s = kbase + col;
                    if (writer && s < nv) {
                        const float sc = x + 0.0f;                        // canonical +0
                        S[r * NcP + s] = sc;
                        const uint32_t key = f32_key(sc);
                        if (lrow < nlds) atomicAdd(&lh[lrow][key >> 20], 1u);
                        else atomicAdd(&hist[r * HIST_WORDS + (key >> 20)], 1u);
                        const float ej = e * 1.0009765625f + 1.1754943508222875e-38f;
                        dmax_loc = fmaxf(dmax_loc, ej + fabsf(sc) * 5.9604644775390625e-08f);
                    }
                }
        };
        // The loads of the next batch are issued unconditionally (past the end they reread the current
        // batch, an L2 hit), so that no branch separates loads from their uses and the compiler's wait
        // counts stay exact: the next batch stays in flight while this one computes.
        __builtin_amdgcn_s_waitcnt(0);        // the per-row loads above have landed
        u32x4_t ka[U][NV], kb[U][NV];
        if (key0 + wave * 16 < nvmax) {
            load_batch(0, ka);
            for (int tt0 = 0; tt0 < tiles; tt0 += 2 * U) {
                const bool more1 = tt0 + U < tiles && key0 + ((tt0 + U) * 4 + wave) * 16 < nvmax;
                load_batch(more1 ? tt0 + U : tt0, kb);
                compute_batch(tt0, ka);
                if (!more1) break;
                const bool more2 = tt0 + 2 * U < tiles && key0 + ((tt0 + 2 * U) * 4 + wave) * 16 < nvmax;
                load_batch(more2 ? tt0 + 2 * U : tt0 + U, ka);
                compute_batch(tt0 + U, kb);
                if (!more2) break;
            }
        }
        if (writer) {
            if (lrow < nlds) atomicMax(&ldmax[lrow], __float_as_uint(dmax_loc));
            else atomicMax(&hist[r * HIST_WORDS + HW_DMAX], __float_as_uint(dmax_loc));
        }
        __syncthreads();
        for (int lr = 0; lr < nlds; ++lr) {
            const size_t rr = (size_t)b * Tq + g * G + lr;
            for (int i = threadIdx.x; i < BINS1; i += TPB)
                if (lh[lr][i]) atomicAdd(&hist[rr * HIST_WORDS + i], lh[lr][i]);
            if (threadIdx.x == 0 && ldmax[lr]) atomicMax(&hist[rr * HIST_WORDS + HW_DMAX], ldmax[lr]);
        }
    }
}

// ---------------------------------------------------------------------------
// candidate lists, then the per-row selection
// ---------------------------------------------------------------------------
// Each k_collect workgroup filters CCHUNK entries of one row against the row's
// threshold (lower edge of the bin holding the k-th largest S~, minus 2 Dmax),
// appends (index, S~) pairs to the row's candidate list and builds the second
// radix level; k_select then selects each row with one workgroup and emits the
// chosen indices in ascending order without sorting.
constexpr int STPB = 1024;
constexpr int CCHUNK = STPB * 16;    // entries per workgroup (16 waves x 16 groups of 64)
constexpr int BAND_LDS = 1024;       // band entries ranked in LDS (larger bands: 64-bit radix in HBM)
constexpr int CAND_LDS = 8192;       // candidates kept in LDS by k_select (more: read from HBM each pass)





// k_collect: each workgroup filters CCHUNK entries of one row against the row's threshold (lower edge of
// the bin b1 holding the k-th largest S~, minus 2 Dmax), appends (index, S~) pairs to the row's candidate
// list in ascending index order (one contiguous run per workgroup, recorded in the chunk table), and
// histograms key bits 19..8 of the entries inside bin b1 (second radix level).
__global__ __launch_bounds__(STPB) void k_collect(const float* __restrict__ S, uint32_t* __restrict__ hist,
                                                  uint2* __restrict__ list, uint2* __restrict__ ctab, int Tq, int Nc,
                                                  int NcP, long long L, int m, long long pos0, int topk)
{
    constexpr int GPW = CCHUNK / (STPB / 64) / 64;   // groups of 64 entries per wave
    __shared__ uint32_t lh[BINS1];
    __shared__ uint32_t scratch[STPB / 64], res[4], wcount[STPB / 64], wbase[STPB / 64];
    const int r = blockIdx.y, t = r % Tq;
    const int nv = n_visible(pos0 + t, L, m, Nc);
    if (nv <= topk) return;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int s_w = blockIdx.x * CCHUNK + wave * (GPW * 64);
    const float* Sr = S + (size_t)r * NcP;
    // the chunk's scores first: their loads overlap the histogram scan below
    float v[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int sidx = s_w + gi * 64 + lane;
        v[gi] = sidx < nv ? Sr[sidx] : -INFINITY;
    }
    uint32_t* H = hist + (size_t)r * HIST_WORDS;
    for (int i = threadIdx.x; i < BINS1; i += STPB) lh[i] = H[i];
    __syncthreads();
    find_bin_wide(lh, (uint32_t)topk, res, scratch);
    const uint32_t b1 = res[0];
    if (blockIdx.x == 0 && threadIdx.x == 0) { H[HW_B1] = b1; H[HW_A1] = res[1]; }   // for k_select
    const double thr = (double)key_f32(b1 << 20) - 2.0 * (double)__uint_as_float(H[HW_DMAX]);
    for (int i = threadIdx.x; i < BINS2; i += STPB) lh[i] = 0;
    __syncthreads();
    unsigned long long mask[GPW];
    uint32_t cnt = 0;
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int sidx = s_w + gi * 64 + lane;
        const bool c = sidx < nv && (double)v[gi] >= thr;
        if (c) {
            const uint32_t key = f32_key(v[gi]);
            if ((key >> 20) == b1) atomicAdd(&lh[(key >> 8) & (BINS2 - 1)], 1u);
        }
        mask[gi] = __ballot(c);
        cnt += __popcll(mask[gi]);
    }
    if (lane == 0) wcount[wave] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t tot = 0;
        for (int w = 0; w < STPB / 64; ++w) tot += wcount[w];
        uint32_t base = tot ? atomicAdd(&H[HW_CNT], tot) : 0;
        ctab[(size_t)r * (NcP / CCHUNK) + blockIdx.x] = make_uint2(base, tot);
        for (int w = 0; w < STPB / 64; ++w) { wbase[w] = base; base += wcount[w]; }
    }
    __syncthreads();
    uint32_t pos = wbase[wave];
    uint2* Lr = list + (size_t)r * NcP;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int sidx = s_w + gi * 64 + lane;
        if ((mask[gi] >> lane) & 1ull)
            Lr[pos + __popcll(mask[gi] & below)] = make_uint2((uint32_t)sidx, __float_as_uint(v[gi]));
        pos += __popcll(mask[gi]);
    }
    for (int i = threadIdx.x; i < BINS2; i += STPB)
        if (lh[i]) atomicAdd(&H[BINS1 + i], lh[i]);
}

// k_select: one 1024-thread workgroup per row (see the header for the argument).  Candidates are addressed
// in ascending index order through the chunk table ("sorted position" e).
template <int DT, int DI, int HI>
__global__ __launch_bounds__(STPB) void k_select(
    const uint32_t* __restrict__ hist, const uint2* __restrict__ list, const uint2* __restrict__ ctab,
    uint2* __restrict__ band_g, unsigned long long* __restrict__ bkey_g, uint8_t* __restrict__ flag_g,
    const void* __restrict__ q_idx, const float* __restrict__ w_idx, const void* __restrict__ k_idx,
    int Tq, int Nc, int NcP, long long L, int m, long long pos0, int topk,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out)
{
    constexpr int ES = DT == 0 ? 2 : 1;
    __shared__ uint32_t lh[BINS2];
    __shared__ uint32_t scratch[STPB / 64], res[4], nband;
    __shared__ uint32_t cpre[STPB + 1], cbase[STPB];
    __shared__ unsigned long long bkey[BAND_LDS];
    __shared__ uint32_t bpos[BAND_LDS];
    __shared__ uint2 bl[BAND_LDS];                    // band entries (index, position); more go to HBM
    __shared__ uint2 cl[CAND_LDS];                    // candidates in index order (when they fit)
    __shared__ uint8_t fl[CAND_LDS];                  // their flags
    const int r = blockIdx.x, b = r / Tq, t = r % Tq, tid = threadIdx.x;
    const int lane = lane_id(), wave = tid >> 6;
    const int nv = n_visible(pos0 + t, L, m, Nc);
    int32_t* out = idx_out + (size_t)r * topk;
    if (nv <= topk) {                                 // every visible entry is selected
        for (int i = tid; i < topk; i += STPB) out[i] = i < nv ? i : -1;
        if (cnt_out && tid == 0) cnt_out[r] = nv;
        return;
    }
    const uint32_t* H = hist + (size_t)r * HIST_WORDS;
    const float dmax = __uint_as_float(H[HW_DMAX]);
    const uint2* Lr = list + (size_t)r * NcP;
    uint8_t* F = flag_g + (size_t)r * NcP;
    // chunk table -> prefix of counts in chunk (= index) order
    const int NCH = NcP / CCHUNK;                     // <= 1024
    uint32_t total;
    {
        const uint2 c = tid < NCH ? ctab[(size_t)r * NCH + tid] : make_uint2(0u, 0u);
        const uint32_t pre = block_scan(c.y, scratch, &total);
        if (tid < NCH) { cpre[tid] = pre; cbase[tid] = c.x; }
        if (tid == 0) cpre[NCH] = total;
        __syncthreads();
    }
    const uint32_t n = total;
    auto cand_g = [&](uint32_t e) -> uint2 {          // e-th candidate in index order, from HBM
        int lo_c = 0, hi_c = NCH - 1;                 // largest c with cpre[c] <= e: a non-empty chunk holding e
        while (lo_c < hi_c) {
            const int mid = (lo_c + hi_c + 1) >> 1;
            if (cpre[mid] <= e) lo_c = mid; else hi_c = mid - 1;
        }
        return Lr[cbase[lo_c] + (e - cpre[lo_c])];
    };
    const bool inl = n <= (uint32_t)CAND_LDS;        // candidates and flags live in LDS (uniform)
    auto cand = [&](uint32_t e) -> uint2 { return inl ? cl[e] : cand_g(e); };
    auto fget = [&](uint32_t e) -> uint8_t { return inl ? fl[e] : F[e]; };
    auto fset = [&](uint32_t e, uint8_t f) { if (inl) fl[e] = f; else F[e] = f; };

    // 1. tau: the bin b1 (level 1, found by k_collect), then b2 (level 2, built by k_collect), then the
    //    last 8 bits.  The candidates are read once into LDS in the same pass as the level-2 histogram.
    const uint32_t b1 = H[HW_B1], a1 = H[HW_A1];
    for (int i = tid; i < BINS2; i += STPB) lh[i] = H[BINS1 + i];
    if (inl)
        for (uint32_t e = tid; e < n; e += STPB) cl[e] = cand_g(e);
    __syncthreads();
    find_bin_wide(lh, (uint32_t)topk - a1, res, scratch);
    const uint32_t b2 = res[0], a2 = res[1];
    __syncthreads();
    const uint32_t pfx = (b1 << 12) | b2;
    for (int i = tid; i < 256; i += STPB) lh[i] = 0;
    __syncthreads();
    for (uint32_t e = tid; e < n; e += STPB) {
        const uint32_t key = f32_key(__uint_as_float(cand(e).y));
        if ((key >> 8) == pfx) atomicAdd(&lh[key & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) wave_find_bin256(lh, (uint32_t)topk - a1 - a2, 0u, res);
    __syncthreads();
    const float tau = key_f32((pfx << 8) | res[0]);
    const double lo = (double)tau - 2.0 * (double)dmax, hi = (double)tau + 2.0 * (double)dmax;

    // 2. classify: flag 1 = certainly in, 2 = band (listed with its position), 0 = out
    if (tid == 0) nband = 0;
    __syncthreads();
    uint2* Bg = band_g + (size_t)r * NcP;
    uint32_t my_in = 0;
    for (uint32_t e = tid; e < n; e += STPB) {
        const uint2 c = cand(e);
        const double v = (double)__uint_as_float(c.y);
        uint8_t f = 0;
        if (v > hi) { f = 1; ++my_in; }
        else if (v >= lo) {
            f = 2;
            const uint32_t slot = atomicAdd(&nband, 1u);
            if (slot < (uint32_t)BAND_LDS) bl[slot] = make_uint2(c.x, e);
            else Bg[slot] = make_uint2(c.x, e);
        }
        fset(e, f);
    }
    uint32_t n_in;
    block_scan(my_in, scratch, &n_in);
    __syncthreads();
    const uint32_t nb = nband;
    const uint32_t need = (uint32_t)topk - n_in;       // 0 <= need <= nb by construction
    auto band = [&](uint32_t i) -> uint2 { return i < (uint32_t)BAND_LDS ? bl[i] : Bg[i]; };

    // 3. exact rescoring of the band (one wave per entry); composite keys (exact score key,
    //    inverted index): larger composite = earlier in the order
    unsigned long long* Kg = bkey_g + (size_t)r * NcP;
    const char* qrow = (const char*)q_idx + (size_t)r * HI * DI * ES;
    const float* wrow = w_idx + (size_t)r * HI;
    if (need > 0 && need < nb) {
        for (uint32_t i = wave; i < nb; i += STPB / 64) {
            const uint2 be = band(i);
            const float sx = wave_exact_score<DT, DI, HI>(qrow, wrow, (const char*)k_idx + ((size_t)b * Nc + be.x) * DI * ES);
            if (lane == 0) {
                const unsigned long long ck = ((unsigned long long)f32_key(sx) << 32) | (0xffffffffu - be.x);
                if (nb > (uint32_t)BAND_LDS) Kg[i] = ck;       // the radix path reads every key from HBM
                if (i < BAND_LDS) { bkey[i] = ck; bpos[i] = be.y; }
            }
        }
    }
    __syncthreads();

    // 4. the `need` largest composite keys among the band get flag 1
    if (need > 0 && need == nb) {
        for (uint32_t i = tid; i < nb; i += STPB) fset(band(i).y, 1);
    } else if (need > 0 && nb <= BAND_LDS) {
        for (uint32_t i = tid; i < nb; i += STPB) {          // rank by counting (keys are distinct)
            const unsigned long long ki = bkey[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < nb; ++j) rank += bkey[j] > ki;
            if (rank < need) fset(bpos[i], 1);
        }
    } else if (need > 0) {
        unsigned long long kp = 0;
        uint32_t ab = 0;
        for (int pass = 0; pass < 8; ++pass) {
            const int shift = 56 - 8 * pass;
            for (int i = tid; i < 256; i += STPB) lh[i] = 0;
            __syncthreads();
            for (uint32_t i = tid; i < nb; i += STPB) {
                const unsigned long long key = Kg[i];
                if (pass == 0 || (key >> (shift + 8)) == (kp >> (shift + 8))) atomicAdd(&lh[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (wave == 0) wave_find_bin256(lh, need, ab, res);
            __syncthreads();
            kp |= (unsigned long long)res[0] << shift;
            ab = res[1];
            __syncthreads();
        }
        for (uint32_t i = tid; i < nb; i += STPB)
            if (Kg[i] >= kp) fset(band(i).y, 1);
    }
    __threadfence_block();
    __syncthreads();

    // 5. compaction in index order: thread tid owns positions [tid*per, (tid+1)*per)
    const uint32_t per = (n + STPB - 1) / STPB;
    const uint32_t e0 = min(n, tid * per), e1 = min(n, e0 + per);
    uint32_t mine = 0;
    for (uint32_t e = e0; e < e1; ++e) mine += fget(e) == 1;
    uint32_t tot2;
    uint32_t o = block_scan(mine, scratch, &tot2);
    for (uint32_t e = e0; e < e1; ++e)
        if (fget(e) == 1 && o < (uint32_t)topk) out[o++] = (int32_t)cand(e).x;
    if (cnt_out && tid == 0) cnt_out[r] = topk;
}

}  // namespace

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// S~ [R][NcP] f32 | hist [R][HIST_WORDS] | list [R][NcP] (index, S~) | chunk table [R][NcP/CCHUNK] |
// band [R][NcP] (index, position) | band keys [R][NcP] u64 | flags [R][NcP] u8
static size_t decode_index_ws_bytes(int B, int Tq, int Nc) {
    const size_t R = (size_t)B * Tq;
    const size_t NcP = ((size_t)Nc + CCHUNK - 1) / CCHUNK * CCHUNK;
    return align256(R * NcP * 4) + align256(R * HIST_WORDS * 4) + align256(R * NcP * 8) +
           align256(R * (NcP / CCHUNK) * 8) + align256(R * NcP * 8) + align256(R * NcP * 8) + align256(R * NcP);
}

template <int DT, int DI, int HI>
static int launch_index(const void* q_idx, const float* w_idx, const void* k_idx, int B, int Tq, int Nc,
                        long long L, int m, long long pos0, int topk, int32_t* idx_out, int32_t* cnt_out,
                        void* ws, hipStream_t st) {
    const size_t R = (size_t)B * Tq;
    const int NcP = (Nc + CCHUNK - 1) / CCHUNK * CCHUNK;
    char* p = (char*)ws;
    float* S = (float*)p;                       p += align256(R * (size_t)NcP * 4);
    uint32_t* hist = (uint32_t*)p;              p += align256(R * HIST_WORDS * 4);
    uint2* list = (uint2*)p;                    p += align256(R * (size_t)NcP * 8);
    uint2* ctab = (uint2*)p;                    p += align256(R * (size_t)(NcP / CCHUNK) * 8);
    uint2* band = (uint2*)p;                    p += align256(R * (size_t)NcP * 8);
    unsigned long long* bkey = (unsigned long long*)p; p += align256(R * (size_t)NcP * 8);
    uint8_t* flags = (uint8_t*)p;
    {
        const size_t n = R * HIST_WORDS;
        const int blocks = (int)std::min<size_t>((n + 255) / 256, 2048);
        CSA_LAUNCH("k_fill", k_fill, dim3(blocks), dim3(256), 0, st, hist, n);
    }
    // keys per scoring workgroup (4 waves x tiles of 16): the largest of 4096/2048/1024 that still
    // gives >= 512 workgroups (two per CU), so the grid runs in one round without a tail
#ifndef CSA_SCORE_KPW
    int kpw = 4096;
    while (kpw > 1024 && (size_t)((Nc + kpw - 1) / kpw) * B < 512) kpw >>= 1;
#else
    const int kpw = CSA_SCORE_KPW;
#endif
    CSA_LAUNCH("k_score", (k_score<DT, DI, HI>), dim3((Nc + kpw - 1) / kpw, B), dim3(TPB), 0, st,
               q_idx, w_idx, k_idx, Tq, Nc, NcP, L, m, pos0, kpw, topk, S, hist);
    CSA_LAUNCH("k_collect", k_collect, dim3(NcP / CCHUNK, (unsigned)R), dim3(STPB), 0, st, S, hist, list, ctab, Tq,
               Nc, NcP, L, m, pos0, topk);
    CSA_LAUNCH("k_select", (k_select<DT, DI, HI>), dim3((unsigned)R), dim3(STPB), 0, st, hist, list, ctab, band,
               bkey, flags, q_idx, w_idx, k_idx, Tq, Nc, NcP, L, m, pos0, topk, idx_out, cnt_out);
    return 0;
}

size_t index_topk_ws_bytes(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk) {
    if (prefill_index_applicable(dtype, HI, dI, B, Tq, Nc, topk)) return prefill_index_ws_bytes(B, Tq, Nc);
    return decode_index_ws_bytes(B, Tq, Nc);
}

int index_topk_launch(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B, int Tq,
                      int HI, int dI, int Nc, long long L, int m, long long pos0, int topk,
                      int32_t* idx_out, int32_t* cnt_out, void* ws, hipStream_t st) {
    if (prefill_index_applicable(dtype, HI, dI, B, Tq, Nc, topk))
        return prefill_index_launch(q_idx, w_idx, k_idx, B, Tq, Nc, L, m, pos0, topk, idx_out, cnt_out, ws, st);
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

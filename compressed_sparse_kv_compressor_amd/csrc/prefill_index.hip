// prefill_index.hip -- Lightning-Indexer scores and bit-exact per-query top-k for
// many queries at once (chunked prefill) on gfx950.
//
// Method: "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1
// (the indexer scores every compressed entry for each query; a top-k selector keeps
// the most relevant ones) and "DeepSeek V4 详解", section "第一刀" (each query looks
// only at its own top-k).  The score and the order are those of the decode path:
// S = fma-chain_h w_h ReLU(RN32(exact q_h . k_s)), first k under (S desc, index asc).
//
// With thousands of queries the score matrix (Tq x Nc fp32: 2 GiB at 8192 x 65536)
// must not be written.  Pipeline, all on the caller's stream:
//   k_pnorm     per-row bound inputs: Wq = sum_h |w_h| ||q_h||_2 (rounded up) and the
//               largest key norm Kmax of the sequence
//   k_pscore<0> approximate scores S~ of every 16th entry only (MFMA, 1/16 of the work),
//               stored as the top 16 bits of their order key
//   k_pthresh   per row: thr = lower edge of the key bin of the j-th largest sampled
//               S~ (j = k/8 + 16), i.e. about 2k + O(sqrt k) entries lie above it
//   k_pscore<1> the dense contraction [queries x heads] x [entries] on MFMA with the
//               ReLU-weighted head reduction fused; entries with S~ >= thr are
//               appended to per-(row, key split) lists in ascending index order
//   k_pselect   per row: exact k-th largest S~ (tau) of the list; with the row bound
//               D (below) entries above tau + 2D are in, those in the band are
//               rescored exactly and ranked; the chosen indices are written in
//               ascending order
//   k_pfallback rows whose list could be incomplete (fewer than k entries above thr,
//               thr above tau - 2D, a list or band over its capacity): exact scores
//               of every visible entry and a 64-bit radix select on (S, index)
// Row bound.  With N_h = ||q_h|| ||k||, the MFMA error model of the decode path
// (|d~_h - d_h| <= C_DOT sum_i |q_hi k_i| <= C_DOT N_h by Cauchy-Schwarz, and
// |d~_h| <= N_h (1 + C_DOT)) gives
//   |S~ - S| <= sum_h |w_h| N_h [(C_SUM (1 + 2 C_DOT) + C_DOT)(1 + 2^-10)
//               + 2^-24 (1 + C_DOT)(1 + 2^-21)] + 2^-126 <= Wq Kmax 2^-17 + 2^-126,
// since the bracket is below 5.8e-6 < 2^-17.  The classification argument is the
// decode path's; the list holds every entry with S~ >= thr, so when thr <= tau - 2D
// it holds every entry that is in or in the band.
#include "common.h"
#include "exact_dot.h"
#include "index_common.h"
#include "kernels.h"

namespace {

using namespace csa;

constexpr int P_HI = 8, P_DI = 128;           // indexer heads and dim served by this path
constexpr int P_ROW_B = P_DI * 2;             // bytes per key row (bf16)
constexpr int P_TK = 64;                      // entries per LDS tile
constexpr int P_NA = 4;                       // 16-row MFMA blocks per wave (2 queries x 8 heads each)
constexpr int P_QPW = 2 * P_NA;               // queries per wave
constexpr int P_NW = 4;                       // waves per workgroup
constexpr int P_QPG = P_QPW * P_NW;           // queries per workgroup
constexpr int P_TPB = 64 * P_NW;
constexpr int P_DMA = 16 / P_NW;              // 1 KiB tile loads per wave per tile
constexpr int SAMPLE = 16;                    // the sampling pass scores entries 0, 16, 32, ...
constexpr int MAX_SPLIT = 8;                  // key splits per query block
constexpr int CAND_P = 4096;                  // list entries per row the select holds (in registers)
constexpr int BAND_P = 256;                   // band entries ranked in LDS
constexpr int SEL_TPB = 256, SEL_CPT = CAND_P / SEL_TPB;
constexpr int FB_TPB = 1024, FB_SLOTS = 64;

__device__ __forceinline__ int sample_rank(int topk) { return topk / 8 + 16; }

// Raw buffer resource (stride 0, byte offsets) over [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt immediate: vmcnt(n) with expcnt and lgkmcnt left free
__device__ __forceinline__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Smallest float >= x (x >= 0 finite).
__device__ __forceinline__ float round_up_f32(double x) {
    float f = (float)x;
    if ((double)f < x) f = __uint_as_float(__float_as_uint(f) + 1u);
    return f;
}

// ---------------------------------------------------------------------------
// k_pnorm: Kmax per sequence (atomic max of non-negative float bits) and Wq per row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pnorm(const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
                                                const uint16_t* __restrict__ k_idx, int B, int Nc, int R,
                                                float* __restrict__ wq, uint32_t* __restrict__ kmax)
{
    const long long nk = (long long)B * Nc, kblocks = (nk + 255) / 256;
    const long long i = (long long)blockIdx.x < kblocks ? (long long)blockIdx.x * 256 + threadIdx.x
                                                         : nk + ((long long)blockIdx.x - kblocks) * 256 + threadIdx.x;
    auto norm = [](const uint16_t* v) -> double {   // ||v||_2 of P_DI bf16, rounded up a little
        double s = 0.0;
        for (int e = 0; e < P_DI; e += 8) {
            const u32x4_t x = *(const u32x4_t*)(v + e);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double lo = (double)__uint_as_float(x[j] << 16), hi = (double)__uint_as_float(x[j] & 0xffff0000u);
                s = fma(lo, lo, s);
                s = fma(hi, hi, s);
            }
        }
        return sqrt(s) * (1.0 + 1.0e-12);
    };
    if (i < nk) {
        const uint32_t f = __float_as_uint(round_up_f32(norm(k_idx + (size_t)i * P_DI)));
        const int bi = (int)(i / Nc);
        if (__all(bi == __shfl(bi, 0, 64))) {          // one sequence in this wave: one atomic
            uint32_t u = f;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) u = max(u, (uint32_t)__shfl_xor((int)u, o, 64));
            if ((threadIdx.x & 63) == 0) atomicMax(&kmax[bi], u);
        } else {
            atomicMax(&kmax[bi], f);
        }
    } else if (i >= nk && i < nk + R) {
        const size_t r = (size_t)(i - nk);
        double s = 0.0;
        for (int h = 0; h < P_HI; ++h) s += fabs((double)w_idx[r * P_HI + h]) * norm(q_idx + (r * P_HI + h) * P_DI);
        wq[r] = round_up_f32(s * (1.0 + 1.0e-12));
    }
}

// ---------------------------------------------------------------------------
// k_pscore: the contraction.  A workgroup owns P_QPG queries and one key split;
// wave w owns queries q0 + 8w .. +7 as P_NA A blocks (16 rows = 2 queries x 8 heads,
// row = 8 query + head) held in registers for the whole sweep.  Key tiles of 64
// entries stream through four LDS buffers by buffer-load DMA (issued three tiles
// ahead); per 16-entry sub-tile and block: 4 v_mfma_f32_16x16x32_bf16.
// Element order of the contraction: k-step s, lane group g takes the 16-byte
// chunk 4s + g of a row (the same for Q and K).  LDS rows are 256 B with chunk c
// of row r stored at chunk c ^ (r & 15): the 16 rows one read instruction touches
// at one chunk fall on 16 distinct 16-byte bank groups.
// Epilogue per pair of blocks: D lane (g, c) holds rows 4g..4g+3 = heads 4(g&1)..+3
// of query 2a + g/2 at key c; the 4-term w-weighted ReLU sums of two blocks are
// combined by one v_permlane16_swap, after which lane row g holds the full S~ of
// query 4p + 2(g & 1) + (g >> 1) at key c.
// MODE 0: sample indices (key 16 i) and the top 16 key bits of S~ stored per row.
// MODE 1: entries; S~ >= thr (and visible) appended to the row's list of this split.
// ---------------------------------------------------------------------------
struct PScoreArgs {
    const uint16_t* q_idx;
    const float* w_idx;
    const uint16_t* k_idx;
    int Tq, Nc;
    long long L;
    int m;
    long long pos0;
    int topk, nqb, nsplit, span;
    const float* thr;            // MODE 1
    uint16_t* samp;              // MODE 0: [R][NSP]
    int NSP;
    uint2* cand;                 // MODE 1: [R][nsplit][caps] (index, S~ bits)
    uint32_t* cnt;               // MODE 1: [R][nsplit] entries with S~ >= thr (may exceed caps)
    int caps;
};

template <int MODE>
__device__ __forceinline__ void pscore_body(uint16_t* bufA, uint16_t* bufB, uint16_t* bufC, uint16_t* bufD,
                                            const PScoreArgs& A)
{
    const int bid = blockIdx.x;
    const int qb = bid % A.nqb, rest = bid / A.nqb, split = rest % A.nsplit, b = rest / A.nsplit;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int Tq = A.Tq, Nc = A.Nc;
    const int q0 = qb * P_QPG, qw = q0 + w * P_QPW;
    const int NKS = MODE == 0 ? (Nc + SAMPLE - 1) / SAMPLE : Nc;     // key space of this mode
    const int kb = split * A.span;
    const int tlast = min(q0 + P_QPG, Tq) - 1;
    const int nvl = n_visible(A.pos0 + tlast, A.L, A.m, Nc);         // the block's largest visible count
    int ke = min(NKS, kb + A.span);
    ke = min(ke, MODE == 0 ? (nvl + SAMPLE - 1) / SAMPLE : nvl);
    int ntiles = ke > kb ? (ke - kb + P_TK - 1) / P_TK : 0;
    if (MODE == 1 && nvl <= A.topk) ntiles = 0;                       // no row of the block selects

    // ---- A operands and head weights ----
    bf16x8_t qa[P_NA][4];
    float wv[P_NA][4];
#pragma unroll
    for (int a = 0; a < P_NA; ++a) {
        const int t = qw + 2 * a + (c >> 3), h = c & 7;
        const bool v = t < Tq;
        const uint16_t* qp = A.q_idx + (((size_t)b * Tq + (v ? t : 0)) * P_HI + h) * P_DI + 8 * g;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qa[a][s] = as_bf16x8(v ? *(const u32x4_t*)(qp + 32 * s) : u32x4_t{0u, 0u, 0u, 0u});
        const int tw = qw + 2 * a + (g >> 1);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wv[a][r] = tw < Tq ? A.w_idx[((size_t)b * Tq + tw) * P_HI + 4 * (g & 1) + r] : 0.f;
    }
    // ---- per-lane output rows: pair p holds query qw + 4p + 2(g & 1) + (g >> 1) ----
    int rowt[2];
    float thr_l[2];
    int nv_l[2];
    uint32_t cn[2] = {0u, 0u};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int t = qw + 4 * p + 2 * (g & 1) + (g >> 1);
        rowt[p] = t;
        thr_l[p] = INFINITY;
        nv_l[p] = 0;
        if (MODE == 1 && t < Tq) {
            thr_l[p] = A.thr[(size_t)b * Tq + t];
            nv_l[p] = n_visible(A.pos0 + t, A.L, A.m, Nc);
        }
    }
    const uint32_t below = (1u << c) - 1u;
    uint2* crow[2];                           // this split's list of the lane's rows (MODE 1)
#pragma unroll
    for (int p = 0; p < 2; ++p)
        crow[p] = A.cand + (((size_t)b * Tq + min(rowt[p], Tq - 1)) * A.nsplit + split) * A.caps;

    // ---- tile loads: instruction i of wave w covers tile rows 4 (w + P_NW i) .. +3 ----
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(A.k_idx + (size_t)b * Nc * P_DI, (uint32_t)((size_t)Nc * P_ROW_B));
    const int drow = lane >> 4, dpc = lane & 15;
    auto issue = [&](uint16_t* buf, int tile) {
        const int base = kb + tile * P_TK;
#pragma unroll
        for (int i = 0; i < P_DMA; ++i) {
            const int I = w + P_NW * i;
            const int row = 4 * I + drow;
            int key = base + row;
            if (MODE == 0) key *= SAMPLE;
            key = min(key, Nc - 1);
            const uint32_t voff = (uint32_t)key * P_ROW_B + 16u * (uint32_t)(dpc ^ (row & 15));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (CSA_LDS void*)((CSA_LDS char*)buf + 1024 * I), 16,
                                                     (int)voff, 0, 0, 0);
        }
    };
    // this lane's B read at k-step s of sub-tile j: (boff ^ 64 s) + 4096 j
    const uint32_t boff = (uint32_t)c * P_ROW_B + 64u * (uint32_t)(c >> 2) + 16u * (uint32_t)(g ^ (c & 3));

    auto epilogue = [&](const f32x4_t (&acc)[P_NA], int kk) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // ReLU as a signed-integer max on the bit pattern (negative floats, -0 included, are negative
            // integers): one VALU op, with no NaN canonicalisation
            auto relu = [](float x) { return __int_as_float(max(__float_as_int(x), 0)); };
            float x0 = 0.f, x1 = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x0 = fmaf(wv[2 * p][r], relu(acc[2 * p][r]), x0);
                x1 = fmaf(wv[2 * p + 1][r], relu(acc[2 * p + 1][r]), x1);
            }
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
            const float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if constexpr (MODE == 0) {
                if (rowt[p] < Tq)
                    A.samp[((size_t)b * Tq + rowt[p]) * A.NSP + kk] = (uint16_t)(f32_key(v) >> 16);
            } else {
                const bool cd = kk < nv_l[p] && v >= thr_l[p];
                const unsigned long long mask = __builtin_amdgcn_ballot_w64(cd);
                const uint32_t seg = (uint32_t)(mask >> (16 * g)) & 0xffffu;
                // past the capacity the last slot is overwritten: the count then exceeds it and the
                // select hands the row to the exact path
                const uint32_t pos = min(cn[p] + __popc(seg & below), (uint32_t)A.caps - 1u);
                if (cd) crow[p][pos] = make_uint2((uint32_t)kk, __float_as_uint(v));
                cn[p] += __popc(seg);
            }
        }
    };
    auto compute = [&](const uint16_t* buf, int tile) {
        const CSA_LDS char* lb = (const CSA_LDS char*)buf;
        const int k0 = kb + tile * P_TK + c;
#pragma unroll
        for (int j = 0; j < P_TK / 16; ++j) {
            u32x4_t bv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) bv[s] = *(const CSA_LDS u32x4_t*)(lb + ((boff ^ (64u * s)) + 4096u * j));
            f32x4_t acc[P_NA];
#pragma unroll
            for (int a = 0; a < P_NA; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int a = 0; a < P_NA; ++a) acc[a] = mfma16_bf16(qa[a][s], as_bf16x8(bv[s]), acc[a]);
            epilogue(acc, k0 + 16 * j);
        }
    };

    // ---- the tile pipeline: tile t in buffer t % 4, loads issued three tiles ahead ----
    // Before the barrier of tile t each wave waits for its own loads of tile t; at least the
    // loads of tiles t+1 and t+2 were issued after them (candidate stores in between only make
    // the wait longer), hence vmcnt(2 P_DMA).  After the barrier buffer (t+3) % 4 = (t-1) % 4 is
    // free everywhere; it takes tile t+3 once tile t is done.  Loads past the last tile reread
    // clamped rows, so every step issues the same number of loads.
    if (ntiles > 0) {
        issue(bufA, 0);
        issue(bufB, 1);
        issue(bufC, 2);
        for (int t = 0; t < ntiles; t += 4) {
#define CSA_PSTEP(CUR, K, NXT)                                         \
            {                                                          \
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * P_DMA));      \
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
                compute(CUR, t + K);                                   \
                issue(NXT, t + K + 3);                                 \
            }
            CSA_PSTEP(bufA, 0, bufD)
            if (t + 1 >= ntiles) break;
            CSA_PSTEP(bufB, 1, bufA)
            if (t + 2 >= ntiles) break;
            CSA_PSTEP(bufC, 2, bufB)
            if (t + 3 >= ntiles) break;
            CSA_PSTEP(bufD, 3, bufC)
#undef CSA_PSTEP
        }
        __builtin_amdgcn_s_waitcnt(0);        // no tile load may still target this workgroup's LDS
    }
    if constexpr (MODE == 1) {
        if (c == 0) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
                if (rowt[p] < Tq) A.cnt[((size_t)b * Tq + rowt[p]) * A.nsplit + split] = cn[p];
        }
    }
}

// Four tile buffers (distinct objects: the compiler tells a read of one from the loads in
// flight into another).
template <int MODE>
__global__ __launch_bounds__(P_TPB, 2) void k_pscore(PScoreArgs A)
{
    __shared__ __attribute__((aligned(1024))) uint16_t bufA[P_TK * P_DI];
    __shared__ __attribute__((aligned(1024))) uint16_t bufB[P_TK * P_DI];
    __shared__ __attribute__((aligned(1024))) uint16_t bufC[P_TK * P_DI];
    __shared__ __attribute__((aligned(1024))) uint16_t bufD[P_TK * P_DI];
    pscore_body<MODE>(bufA, bufB, bufC, bufD, A);
}

// ---------------------------------------------------------------------------
// k_pthresh: one wave per row; 16-bit radix select of the j-th largest sample key
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_pthresh(const uint16_t* __restrict__ samp, int NSP, int Tq, int Nc, long long L,
                                                 int m, long long pos0, int topk, float* __restrict__ thr)
{
    __shared__ uint32_t h[256];
    __shared__ uint32_t res[2];
    const int r = blockIdx.x, t = r % Tq, lane = lane_id();
    const int nv = n_visible(pos0 + t, L, m, Nc);
    if (nv <= topk) {                                  // every visible entry is selected
        if (lane == 0) thr[r] = INFINITY;
        return;
    }
    const int ns = (nv + SAMPLE - 1) / SAMPLE, j = sample_rank(topk);
    if (ns < j) {                                      // too few samples: every visible entry is a candidate
        if (lane == 0) thr[r] = -INFINITY;
        return;
    }
    const uint16_t* sp = samp + (size_t)r * NSP;
    for (int i = lane; i < 256; i += 64) h[i] = 0;
    __syncthreads();
    for (int i = lane; i < ns; i += 64) atomicAdd(&h[sp[i] >> 8], 1u);
    __syncthreads();
    wave_find_bin256(h, (uint32_t)j, 0u, res);
    __syncthreads();
    const uint32_t b1 = res[0], a1 = res[1];
    __syncthreads();
    for (int i = lane; i < 256; i += 64) h[i] = 0;
    __syncthreads();
    for (int i = lane; i < ns; i += 64) {
        const uint32_t v = sp[i];
        if ((v >> 8) == b1) atomicAdd(&h[v & 255u], 1u);
    }
    __syncthreads();
    wave_find_bin256(h, (uint32_t)j - a1, 0u, res);
    __syncthreads();
    if (lane == 0) thr[r] = key_f32(((b1 << 8) | res[0]) << 16);
}

// ---------------------------------------------------------------------------
// k_pselect: one 256-thread workgroup per row; thread i holds list positions
// 16 i .. 16 i + 15 (the list is in ascending index order across the splits)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(SEL_TPB) void k_pselect(
    const uint2* __restrict__ cand, const uint32_t* __restrict__ cnt, const float* __restrict__ thr,
    const float* __restrict__ wq, const uint32_t* __restrict__ kmax, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const uint16_t* __restrict__ k_idx, int Tq, int Nc, long long L, int m,
    long long pos0, int topk, int nsplit, int caps, int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out,
    uint32_t* __restrict__ fail)
{
    __shared__ uint32_t spre[MAX_SPLIT + 1];
    __shared__ uint32_t hist[256], res[4], scratch[SEL_TPB / 64], nband, bad;
    __shared__ unsigned long long bkey[BAND_P];
    __shared__ uint32_t bpos[BAND_P], bidx[BAND_P];
    __shared__ uint32_t chosen[CAND_P / 32];
    const int r = blockIdx.x, b = r / Tq, t = r % Tq, tid = threadIdx.x;
    const int lane = lane_id(), wave = tid >> 6;
    const int nv = n_visible(pos0 + t, L, m, Nc);
    int32_t* out = idx_out + (size_t)r * topk;
    if (nv <= topk) {
        for (int i = tid; i < topk; i += SEL_TPB) out[i] = i < nv ? i : -1;
        if (cnt_out && tid == 0) cnt_out[r] = nv;
        return;
    }
    auto give_up = [&]() {                              // uniform: the exact fallback takes the row
        if (tid == 0) fail[1 + atomicAdd(&fail[0], 1u)] = (uint32_t)r;
    };
    if (tid == 0) {
        uint32_t s = 0, over = 0;
        for (int i = 0; i < nsplit; ++i) {
            const uint32_t ci = cnt[(size_t)r * nsplit + i];
            spre[i] = s;
            over |= ci > (uint32_t)caps;
            s += ci;
        }
        spre[nsplit] = s;
        bad = over || s < (uint32_t)topk || s > (uint32_t)CAND_P;
        nband = 0;
    }
    for (int i = tid; i < CAND_P / 32; i += SEL_TPB) chosen[i] = 0;
    __syncthreads();
    if (bad) { give_up(); return; }
    const uint32_t n = spre[nsplit];
    const uint32_t e0 = (uint32_t)tid * SEL_CPT;
    uint32_t key[SEL_CPT], cid[SEL_CPT];
    {
        int seg = 0;
        while (seg + 1 < nsplit && e0 >= spre[seg + 1]) ++seg;
#pragma unroll
        for (int i = 0; i < SEL_CPT; ++i) {
            const uint32_t e = e0 + i;
            key[i] = 0u;
            cid[i] = 0u;
            if (e < n) {
                while (e >= spre[seg + 1]) ++seg;
                const uint2 cv = cand[((size_t)r * nsplit + seg) * caps + (e - spre[seg])];
                key[i] = f32_key(__uint_as_float(cv.y));
                cid[i] = cv.x;
            }
        }
    }
    // 1. tau = k-th largest S~ of the list (four 8-bit radix passes)
    uint32_t pref = 0, need = (uint32_t)topk;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SEL_CPT; ++i)
            if (e0 + i < n && (pass == 0 || (key[i] >> (shift + 8)) == (pref >> (shift + 8))))
                atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
        __syncthreads();
        if (wave == 0) wave_find_bin256(hist, need, 0u, res);
        __syncthreads();
        pref |= res[0] << shift;
        need -= res[1];
        __syncthreads();
    }
    const float tau = key_f32(pref);
    const double D = (double)wq[r] * (double)__uint_as_float(kmax[b]) * 7.62939453125e-06 * (1.0 + 1.0 / 512) +
                     1.1754943508222875e-38;
    const double lo = (double)tau - 2.0 * D, hi = (double)tau + 2.0 * D;
    if (!((double)thr[r] <= lo)) { give_up(); return; }       // the list might miss band entries

    // 2. classify: in (above hi), band (listed), out
    uint32_t in_m = 0, band_m = 0, my_in = 0;
#pragma unroll
    for (int i = 0; i < SEL_CPT; ++i) {
        if (e0 + i >= n) continue;
        const double v = (double)key_f32(key[i]);
        if (v > hi) { in_m |= 1u << i; ++my_in; }
        else if (v >= lo) {
            band_m |= 1u << i;
            const uint32_t slot = atomicAdd(&nband, 1u);
            if (slot < (uint32_t)BAND_P) { bidx[slot] = cid[i]; bpos[slot] = e0 + i; }
        }
    }
    uint32_t n_in;
    block_scan(my_in, scratch, &n_in);
    __syncthreads();
    const uint32_t nb = nband;
    if (nb > (uint32_t)BAND_P || n_in > (uint32_t)topk || (uint32_t)topk - n_in > nb) { give_up(); return; }
    const uint32_t needb = (uint32_t)topk - n_in;

    // 3. exact scores of the band, composite keys (score key, inverted index), rank, choose
    if (needb > 0 && needb < nb) {
        const uint16_t* qrow = q_idx + (size_t)r * P_HI * P_DI;
        const float* wrow = w_idx + (size_t)r * P_HI;
        for (uint32_t i = wave; i < nb; i += SEL_TPB / 64) {
            const float sx = wave_exact_score<0, P_DI, P_HI>(qrow, wrow, k_idx + ((size_t)b * Nc + bidx[i]) * P_DI);
            if (lane == 0) bkey[i] = ((unsigned long long)f32_key(sx) << 32) | (0xffffffffu - bidx[i]);
        }
        __syncthreads();
        for (uint32_t i = tid; i < nb; i += SEL_TPB) {
            const unsigned long long ki = bkey[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < nb; ++j) rank += bkey[j] > ki;
            if (rank < needb) atomicOr(&chosen[bpos[i] >> 5], 1u << (bpos[i] & 31));
        }
    } else if (needb == nb) {
        for (uint32_t i = tid; i < nb; i += SEL_TPB) atomicOr(&chosen[bpos[i] >> 5], 1u << (bpos[i] & 31));
    }
    __syncthreads();

    // 4. the chosen indices in ascending order
    uint32_t sel = in_m;
#pragma unroll
    for (int i = 0; i < SEL_CPT; ++i) {
        const uint32_t e = e0 + i;
        if (((band_m >> i) & 1u) && ((chosen[e >> 5] >> (e & 31)) & 1u)) sel |= 1u << i;
    }
    uint32_t tot;
    uint32_t o = block_scan(__popc(sel), scratch, &tot);
    if (tot != (uint32_t)topk) { give_up(); return; }          // inconsistent: leave it to the exact path
#pragma unroll
    for (int i = 0; i < SEL_CPT; ++i)
        if ((sel >> i) & 1u) out[o++] = (int32_t)cid[i];
    if (cnt_out && tid == 0) cnt_out[r] = topk;
}

// ---------------------------------------------------------------------------
// k_pfallback: exact scores of every visible entry of each failed row, then a
// 64-bit radix select on (score key, inverted index); FB_SLOTS rows at a time
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(FB_TPB) void k_pfallback(
    const uint32_t* __restrict__ fail, const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, int Tq, int Nc, long long L, int m, long long pos0, int topk,
    unsigned long long* __restrict__ keys, size_t NcP, int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out)
{
    __shared__ uint32_t hist[256], res[4], scratch[FB_TPB / 64];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const uint32_t nf = fail[0];
    unsigned long long* K = keys + (size_t)blockIdx.x * NcP;
    for (uint32_t fi = blockIdx.x; fi < nf; fi += gridDim.x) {
        const int r = (int)fail[1 + fi], b = r / Tq, t = r % Tq;
        const int nv = n_visible(pos0 + t, L, m, Nc);
        const uint16_t* qrow = q_idx + (size_t)r * P_HI * P_DI;
        const float* wrow = w_idx + (size_t)r * P_HI;
        for (int s = wave; s < nv; s += FB_TPB / 64) {
            const float sx = wave_exact_score<0, P_DI, P_HI>(qrow, wrow, k_idx + ((size_t)b * Nc + s) * P_DI);
            if (lane == 0) K[s] = ((unsigned long long)f32_key(sx) << 32) | (0xffffffffu - (uint32_t)s);
        }
        __threadfence_block();
        __syncthreads();
        unsigned long long kp = 0;
        uint32_t above = 0;
        for (int pass = 0; pass < 8; ++pass) {
            const int shift = 56 - 8 * pass;
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int s = tid; s < nv; s += FB_TPB) {
                const unsigned long long k = K[s];
                if (pass == 0 || (k >> (shift + 8)) == (kp >> (shift + 8))) atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (wave == 0) wave_find_bin256(hist, (uint32_t)topk, above, res);
            __syncthreads();
            kp |= (unsigned long long)res[0] << shift;
            above = res[1];
            __syncthreads();
        }
        // keys are distinct: exactly topk of them are >= kp
        const int per = (nv + FB_TPB - 1) / FB_TPB;
        const int s0 = min(nv, tid * per), s1 = min(nv, s0 + per);
        uint32_t mine = 0;
        for (int s = s0; s < s1; ++s) mine += K[s] >= kp;
        uint32_t tot;
        uint32_t o = block_scan(mine, scratch, &tot);
        int32_t* out = idx_out + (size_t)r * topk;
        for (int s = s0; s < s1; ++s)
            if (K[s] >= kp && o < (uint32_t)topk) out[o++] = s;
        if (cnt_out && tid == 0) cnt_out[r] = topk;
        __syncthreads();                               // K and hist are reused by the next row
    }
}

__global__ void k_pzero(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PrefillPlan {
    int nqb, nsplit0, span0, nsplit1, span1, NSP, caps;
    size_t R, NcP;
};

static PrefillPlan prefill_plan(int B, int Tq, int Nc) {
    PrefillPlan P;
    P.R = (size_t)B * Tq;
    P.nqb = (Tq + P_QPG - 1) / P_QPG;
    auto splits = [&](int nks, int& nsplit, int& span) {
        const int units = B * P.nqb;
        int ns = (1024 + units - 1) / units;
        ns = std::max(1, std::min(ns, MAX_SPLIT));
        ns = std::min(ns, std::max(1, (nks + 1023) / 1024));
        span = ((nks + ns - 1) / ns + P_TK - 1) / P_TK * P_TK;
        nsplit = (nks + span - 1) / span;
        if (nsplit < 1) nsplit = 1;
    };
    const int NS = (Nc + SAMPLE - 1) / SAMPLE;
    splits(NS, P.nsplit0, P.span0);
    splits(Nc, P.nsplit1, P.span1);
    P.NSP = (NS + P_TK - 1) / P_TK * P_TK;
    // per-split capacity: twice an even share of the row's limit (a row whose list crowds into one
    // split past that goes to the exact path)
    P.caps = std::min(CAND_P, std::max(1024, 2 * CAND_P / P.nsplit1));
    P.NcP = ((size_t)Nc + 63) / 64 * 64;
    return P;
}

bool prefill_index_applicable(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk) {
    return dtype == 0 && HI == P_HI && dI == P_DI && Tq >= 64 && topk <= 1024 && Nc >= 1 &&
           (size_t)Nc * P_ROW_B < ((size_t)1 << 31) && (size_t)B * Tq <= ((size_t)1 << 24);
}

// kmax [B] | fail [1 + R] | wq [R] | thr [R] | samp [R][NSP] u16 | cnt [R][nsplit1] | cand [R][nsplit1][caps]
// | fallback keys [FB_SLOTS][NcP] u64
size_t prefill_index_ws_bytes(int B, int Tq, int Nc) {
    const PrefillPlan P = prefill_plan(B, Tq, Nc);
    return align256((size_t)B * 4) + align256((P.R + 1) * 4) + align256(P.R * 4) + align256(P.R * 4) +
           align256(P.R * P.NSP * 2) + align256(P.R * P.nsplit1 * 4) + align256(P.R * P.nsplit1 * P.caps * 8) +
           align256((size_t)FB_SLOTS * P.NcP * 8);
}

int prefill_index_launch(const void* q_idx, const float* w_idx, const void* k_idx, int B, int Tq, int Nc,
                         long long L, int m, long long pos0, int topk, int32_t* idx_out, int32_t* cnt_out, void* ws,
                         hipStream_t st) {
    const PrefillPlan P = prefill_plan(B, Tq, Nc);
    char* p = (char*)ws;
    uint32_t* kmax = (uint32_t*)p;          p += align256((size_t)B * 4);
    uint32_t* fail = (uint32_t*)p;          p += align256((P.R + 1) * 4);
    float* wq = (float*)p;                  p += align256(P.R * 4);
    float* thr = (float*)p;                 p += align256(P.R * 4);
    uint16_t* samp = (uint16_t*)p;          p += align256(P.R * P.NSP * 2);
    uint32_t* cnt = (uint32_t*)p;           p += align256(P.R * P.nsplit1 * 4);
    uint2* cand = (uint2*)p;                p += align256(P.R * P.nsplit1 * P.caps * 8);
    unsigned long long* fbk = (unsigned long long*)p;
    const uint16_t* q = (const uint16_t*)q_idx;
    const uint16_t* k = (const uint16_t*)k_idx;

    CSA_LAUNCH("k_pzero", k_pzero, dim3((B + 255) / 256), dim3(256), 0, st, kmax, B);
    CSA_LAUNCH("k_pzero", k_pzero, dim3(1), dim3(64), 0, st, fail, 1);
    {
        const long long nb = ((long long)B * Nc + 255) / 256 + ((long long)P.R + 255) / 256;
        CSA_LAUNCH("k_pnorm", k_pnorm, dim3((unsigned)nb), dim3(256), 0, st, q, w_idx, k, B, Nc,
                   (int)P.R, wq, kmax);
    }
    PScoreArgs A;
    A.q_idx = q; A.w_idx = w_idx; A.k_idx = k;
    A.Tq = Tq; A.Nc = Nc; A.L = L; A.m = m; A.pos0 = pos0; A.topk = topk; A.nqb = P.nqb;
    A.thr = thr; A.samp = samp; A.NSP = P.NSP; A.cand = cand; A.cnt = cnt; A.caps = P.caps;
    A.nsplit = P.nsplit0; A.span = P.span0;
    CSA_LAUNCH("k_pscore_sample", k_pscore<0>, dim3((unsigned)(B * P.nqb * P.nsplit0)), dim3(P_TPB), 0, st, A);
    CSA_LAUNCH("k_pthresh", k_pthresh, dim3((unsigned)P.R), dim3(64), 0, st, samp, P.NSP, Tq, Nc, L, m, pos0, topk,
               thr);
    A.nsplit = P.nsplit1; A.span = P.span1;
    CSA_LAUNCH("k_pscore", k_pscore<1>, dim3((unsigned)(B * P.nqb * P.nsplit1)), dim3(P_TPB), 0, st, A);
    CSA_LAUNCH("k_pselect", k_pselect, dim3((unsigned)P.R), dim3(SEL_TPB), 0, st, cand, cnt, thr, wq, kmax, q, w_idx,
               k, Tq, Nc, L, m, pos0, topk, P.nsplit1, P.caps, idx_out, cnt_out, fail);
    CSA_LAUNCH("k_pfallback", k_pfallback, dim3(FB_SLOTS), dim3(FB_TPB), 0, st, fail, q, w_idx, k, Tq, Nc, L, m,
               pos0, topk, fbk, P.NcP, idx_out, cnt_out);
    return 0;
}

}  // namespace csa_host

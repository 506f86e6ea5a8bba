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
//               S~ (j = 3k/32 + 16), i.e. about 1.5k + 256 +- 16 sqrt(j) entries lie above it
//   k_pscore<1> the dense contraction [queries x heads] x [entries] on MFMA with the
//               ReLU-weighted head reduction fused; entries with S~ >= thr are
//               appended to per-(row, key split) lists in ascending index order
//   k_pselect   per row: exact k-th largest S~ (tau) of the list; with the row bound
//               D (below) entries above tau + 2D are in, those in the band are
//               rescored exactly and ranked; the chosen indices are written in
//               ascending order
//   k_pfb_score, k_pfb_rows  rows whose list could be incomplete (fewer than k
//               entries above thr, thr above tau - 2D, a list or band over its
//               capacity): exact scores of every visible entry, then a radix select
//               on the exact score keys (ties by index)
// Other operand formats (e4m3 or MXFP4 rows, HI = 1, 2 or 4 heads, dI = 64) run the same kernels on
// operands widened once into the workspace by k_pwiden: 8 heads x 128 bf16 dims per row.  Nothing the
// method computes changes: every e4m3 value and every scaled E2M1 value is a bf16 value, a padded dim
// is zero in query and key (an exact zero term of every dot and norm), and a padded head has weight +0
// (each adds fmaf(+0, ReLU(d), S) = S to the fma chain, whose partial sums are never -0), so exact and
// approximate scores, the bound and the selection are those of the original operands.
// Row bound.  With N_h = ||q_h|| ||k||, the MFMA error model of the decode path
// (|d~_h - d_h| <= C_DOT sum_i |q_hi k_i| <= C_DOT N_h by Cauchy-Schwarz, and
// |d~_h| <= N_h (1 + C_DOT)) gives
//   |S~ - S| <= sum_h |w_h| N_h [(C_SUM (1 + 2 C_DOT) + C_DOT)(1 + 2^-10)
//               + 2^-24 (1 + C_DOT)(1 + 2^-21)] + 2^-126 <= Wq Kmax 2^-16 + 2^-126,
// since with C_DOT = 2^-17 and C_SUM = 2^-19 the bracket is below 9.7e-6 < 2^-16.  The
// 32x32x16 MFMA's dot over 128 elements chains 8 instructions of 16 products through the
// accumulator, which the decode path's order-free model covers.  The classification argument is the
// decode path's; the list holds every entry with S~ >= thr, so when thr <= tau - 2D
// it holds every entry that is in or in the band.
#include "common.h"
#include "exact_dot.h"
#include "index_common.h"
#include "kernels.h"

#include <type_traits>

namespace {

using namespace csa;

constexpr int P_HI = 8, P_DI = 128;           // indexer heads and dim served by this path
constexpr int P_ROW_B = P_DI * 2;             // bytes per key row (bf16)
constexpr int P_TK = 64;                      // entries per LDS tile
constexpr int P_NA = 2;                       // 32-row MFMA blocks per wave (4 queries x 8 heads each)
constexpr int P_QPW = 4 * P_NA;               // queries per wave
constexpr int P_UNITS = 1024;                 // target workgroups of the contraction
constexpr int P_VPM1 = 8;                     // VALU instructions scheduled after each MFMA of a tile's first half
constexpr int P_VPM2 = 5;                     // ... and of its second half
constexpr int P_NBUF = 5;                     // LDS tile buffers (loads run P_NBUF - 1 tiles ahead)
static_assert(P_NBUF >= 3 && P_NBUF <= 8, "tile buffers");
static_assert(P_TK == 64, "the tile pipeline handles two 32-entry sub-tiles per tile");
constexpr int P_NW = 4;                       // waves per workgroup
constexpr int P_QPG = P_QPW * P_NW;           // queries per workgroup
constexpr int P_TPB = 64 * P_NW;
constexpr int P_DMA = 16 / P_NW;              // 1 KiB tile loads per wave per tile
constexpr int SAMPLE = 16;                    // the sampling pass scores entries 0, 16, 32, ...
constexpr int MAX_SPLIT = 8;                  // key splits per query block
constexpr int CAND_P = 4096;                  // list capacity scale (per-split capacities derive from it)
constexpr int FB_TPB = 1024, FB_SLOTS = 64;

__device__ __forceinline__ int sample_rank(int topk) { return topk * 3 / 32 + 16; }

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
// k_pnorm: Kmax per sequence (atomic max of non-negative float bits) and Wq per row.
// Key blocks: 16 lanes per key (16 bytes each), four keys per wave at a time.  Row
// blocks: one wave per row, 8 lanes per head.  Squares and sums in fp64 (each square
// of a bf16 is exact); the results are rounded up to fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double sumsq8(u32x4_t x) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double lo = (double)__uint_as_float(x[j] << 16), hi = (double)__uint_as_float(x[j] & 0xffff0000u);
        s = fma(lo, lo, s);
        s = fma(hi, hi, s);
    }
    return s;
}
__device__ __forceinline__ double shfl_xor_d(double v, int o) {
    const unsigned long long u = __double_as_longlong(v);
    const int lo = __shfl_xor((int)(uint32_t)u, o, 64), hi = __shfl_xor((int)(uint32_t)(u >> 32), o, 64);
    return __longlong_as_double(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

constexpr int NORM_KEYS_PER_BLOCK = 64;     // 4 waves x 4 keys x 4 rounds

__global__ __launch_bounds__(256) void k_pnorm(const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
                                                const uint16_t* __restrict__ k_idx, int B, int Nc, int R,
                                                float* __restrict__ wq, uint32_t* __restrict__ kmax)
{
    const long long nk = (long long)B * Nc;
    const long long kblocks = (nk + NORM_KEYS_PER_BLOCK - 1) / NORM_KEYS_PER_BLOCK;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    if ((long long)blockIdx.x < kblocks) {
        __shared__ uint32_t wmax[4];
        const long long k0 = (long long)blockIdx.x * NORM_KEYS_PER_BLOCK;
        const long long k1 = min(nk, k0 + NORM_KEYS_PER_BLOCK) - 1;
        const bool one_seq = k0 / Nc == k1 / Nc;        // uniform: the block's keys share a sequence
        uint32_t mx = 0;
#pragma unroll
        for (int rd = 0; rd < 4; ++rd) {
            const long long key = k0 + rd * 16 + wave * 4 + (lane >> 4);
            double ss = 0.0;
            if (key < nk) ss = sumsq8(*(const u32x4_t*)(k_idx + (size_t)key * P_DI + 8 * (lane & 15)));
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) ss += shfl_xor_d(ss, o);
            if (key < nk) {
                const uint32_t f = __float_as_uint(round_up_f32(sqrt(ss) * (1.0 + 1.0e-12)));
                if (one_seq) mx = max(mx, f);
                else if ((lane & 15) == 0) atomicMax(&kmax[(int)(key / Nc)], f);
            }
        }
        if (one_seq) {                                  // one atomic per block
#pragma unroll
            for (int o = 16; o < 64; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
            if (lane == 0) wmax[wave] = mx;
            __syncthreads();
            if (threadIdx.x == 0)
                atomicMax(&kmax[(int)(k0 / Nc)], max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
        }
    } else {
        const long long r = ((long long)blockIdx.x - kblocks) * 4 + wave;
        if (r >= R) return;
        const int h = lane >> 3, part = lane & 7;     // 8 lanes per head, 16 elements each
        const uint16_t* qp = q_idx + ((size_t)r * P_HI + h) * P_DI + 16 * part;
        double ss = sumsq8(*(const u32x4_t*)qp) + sumsq8(*(const u32x4_t*)(qp + 8));
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) ss += shfl_xor_d(ss, o);
        double t = fabs((double)w_idx[(size_t)r * P_HI + h]) * (sqrt(ss) * (1.0 + 1.0e-12));
#pragma unroll
        for (int o = 8; o < 64; o <<= 1) t += shfl_xor_d(t, o);
        if (lane == 0) wq[r] = round_up_f32(t * (1.0 + 1.0e-12));
    }
}

// ---------------------------------------------------------------------------
// k_pscore: the contraction.  A workgroup owns P_QPG queries and one key split;
// wave w owns queries qw = q0 + 8w .. +7 as P_NA A blocks of 32 rows (4 queries x
// 8 heads, row = 8 query + head) held in registers for the whole sweep.  Key tiles
// of 64 entries stream through four LDS buffers by buffer-load DMA (issued three
// tiles ahead); per 32-entry sub-tile and block: 8 v_mfma_f32_32x32x16_bf16.
// The 32x32x16 shape leaves the most VALU issue room beside the matrix pipe
// (about six VALU instructions per MFMA at no cost), which the fused epilogue needs.
// Element order of the contraction: k-step s, lane half g2 takes the 16-byte chunk
// 2s + g2 of a row (the same for Q and K).  LDS rows are 256 B with chunk c of row r
// stored at chunk c ^ (r & 15): the rows one read instruction touches at one chunk
// fall on distinct 16-byte bank groups.
// Epilogue: D lane (g2, c) register r holds row 8 (r/4) + 4 g2 + r%4, i.e. head
// 4 g2 + r%4 of query r/4 at key c.  Four-term w-weighted ReLU sums per query, then
// one v_permlane32_swap per query pair adds the two head halves: lane half g2 holds
// S~ of query 2 g2 (first register) and 2 g2 + 1 (second).  After the two sub-tiles
// of a tile one more permlane32 swap per register pair leaves one register per
// query with its 64 keys in lane order, so that the threshold, the count and the
// list offset of every store are wave-uniform.
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
__device__ __forceinline__ void pscore_body(uint16_t* const (&bufs)[P_NBUF], const PScoreArgs& A)
{
    const int bid = blockIdx.x;
    const int qb = bid % A.nqb, rest = bid / A.nqb, split = rest % A.nsplit, b = rest / A.nsplit;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, g2 = lane >> 5;
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
    // Row 8 j + 4 g + i of block a (j, i = 0..3, g = 0, 1) is head 4 (j % 2) + i of query qw + 4a + 2g + j/2,
    // so that accumulator register r = 4 j + i of a lane in half g (which holds row 8 j + 4 g + i) covers
    // all eight heads of queries 4a + 2g (registers 0-7) and 4a + 2g + 1 (registers 8-15): the head sum
    // stays within the lane.
    bf16x8_t qa[P_NA][8];
    float wv[P_NA][16];                       // register r of block a: query qw + 4a + 2 g2 + r/8, head 4 (r/4 % 2) + r%4
#pragma unroll
    for (int a = 0; a < P_NA; ++a) {
        const int t = qw + 4 * a + 2 * ((r32 >> 2) & 1) + (r32 >> 4), h = 4 * ((r32 >> 3) & 1) + (r32 & 3);
        const bool v = t < Tq;
        const uint16_t* qp = A.q_idx + (((size_t)b * Tq + (v ? t : 0)) * P_HI + h) * P_DI + 8 * g2;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qa[a][s] = as_bf16x8(v ? *(const u32x4_t*)(qp + 16 * s) : u32x4_t{0u, 0u, 0u, 0u});
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tw = qw + 4 * a + 2 * g2 + r / 8;
            wv[a][r] = tw < Tq ? A.w_idx[((size_t)b * Tq + tw) * P_HI + 4 * ((r / 4) % 2) + r % 4] : 0.f;
        }
    }
    // ---- per-query state (wave-uniform): local query lq = 0..7 is query qw + lq ----
    float thr_q[P_QPW];
    int nv_q[P_QPW];
    uint32_t C[P_QPW];                        // list entries so far (MODE 1)
#pragma unroll
    for (int lq = 0; lq < P_QPW; ++lq) {
        const int t = qw + lq;
        thr_q[lq] = INFINITY;
        nv_q[lq] = 0;
        C[lq] = 0u;
        if (MODE == 1 && t < Tq) {
            thr_q[lq] = A.thr[(size_t)b * Tq + t];
            nv_q[lq] = n_visible(A.pos0 + t, A.L, A.m, Nc);
        }
    }
    // list stores go through a buffer resource over this workgroup's rows of this split; a
    // non-candidate lane stores at an offset past its end, which the hardware drops (no branch).
    // (the pieces go through readfirstlane so that the resource is built in scalar registers)
    const int nrow_wg = max(0, min(P_QPG, Tq - q0));
    const uint32_t seg_bytes = (uint32_t)A.caps * 8u;
    const uint64_t cbase = MODE == 1 ? (uint64_t)(A.cand + (((size_t)b * Tq + q0) * A.nsplit + split) * A.caps) : 0u;
    const uint32_t cb_lo = __builtin_amdgcn_readfirstlane((uint32_t)cbase);
    const uint32_t cb_hi = __builtin_amdgcn_readfirstlane((uint32_t)(cbase >> 32));
    const uint32_t cb_n = __builtin_amdgcn_readfirstlane(MODE == 1 ? (uint32_t)nrow_wg * (uint32_t)A.nsplit * seg_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const void*)(((uint64_t)cb_hi << 32) | cb_lo), cb_n);
    const uint32_t drop = __builtin_amdgcn_readfirstlane(0x80000000u | cb_n);   // an offset past the resource
    // MODE 0: the sample rows of this workgroup, same scheme
    const uint64_t sbase64 = MODE == 0 ? (uint64_t)(A.samp + ((size_t)b * Tq + q0) * A.NSP) : 0u;
    const uint32_t sb_lo = __builtin_amdgcn_readfirstlane((uint32_t)sbase64);
    const uint32_t sb_hi = __builtin_amdgcn_readfirstlane((uint32_t)(sbase64 >> 32));
    const uint32_t sb_n = __builtin_amdgcn_readfirstlane(MODE == 0 ? (uint32_t)nrow_wg * (uint32_t)A.NSP * 2u : 0u);
    const __amdgpu_buffer_rsrc_t rsmp = make_rsrc((const void*)(((uint64_t)sb_hi << 32) | sb_lo), sb_n);

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
    // this lane's B read at k-step s of sub-tile j: (boff ^ 32 s) + 8192 j (key 32 j + r32, chunk 2 s + g2)
    const uint32_t boff = (uint32_t)r32 * P_ROW_B + 32u * (uint32_t)((r32 & 15) >> 1) + 16u * (uint32_t)(g2 ^ (r32 & 1));

    // ReLU as a signed-integer max on the bit pattern (negative floats, -0 included, are negative
    // integers): one VALU op, with no NaN canonicalisation
    auto relu = [](float x) { return __int_as_float(max(__float_as_int(x), 0)); };
    // S~ of one block: va = query 4a (lanes 0-31) / 4a + 2 (lanes 32-63), vb = 4a + 1 / 4a + 3, at key r32
    auto block_scores = [&](const f32x16_t& acc, const float (&wb)[16], float& va, float& vb) {
        float x = 0.f, y = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            x = fmaf(wb[r], relu(acc[r]), x);
            y = fmaf(wb[8 + r], relu(acc[8 + r]), y);
        }
        va = x;
        vb = y;
    };
    // one query's 64 keys (lane = key - kbase): sample store or list append
    auto emit = [&](float v, int lq, int kk, bool live, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;     // every key of the tile visible to every query
        if constexpr (MODE == 0) {
            // every lane stores (a missing row's offset lies past the resource): the number of memory
            // operations per tile is fixed, which the tile wait below counts on
            const uint32_t off = live && qw + lq < Tq
                                     ? ((uint32_t)(w * P_QPW + lq) * (uint32_t)A.NSP + (uint32_t)kk) * 2u
                                     : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(f32_key(v) >> 16), rsmp, (int)off, 0, 0);
        } else {
            const bool cd = live && (FULL ? v >= thr_q[lq] : (kk < nv_q[lq] && v >= thr_q[lq]));
            const unsigned long long mask = __builtin_amdgcn_ballot_w64(cd);
            // slot base of this query's stores (scalar); once fewer than 64 slots remain the stores
            // go to the last 64 (the count then exceeds caps - 64 and the select hands the row to the
            // exact path)
            const uint32_t sbase = (uint32_t)((w * P_QPW + lq) * A.nsplit) * seg_bytes +
                                   8u * min(C[lq], (uint32_t)A.caps - 64u);
            const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
            // (the select is written as one v_cndmask on the ballot so that the compiler does not turn it
            // into an exec-masked branch, which would blur its count of memory operations per step)
            uint32_t off;
            asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(off) : "v"(drop), "v"(sbase + 8u * rank), "s"(mask));
            typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{(uint32_t)kk, __float_as_uint(v)}, rc, (int)off, 0, 0);
            C[lq] += (uint32_t)__popcll(mask);
        }
    };
    auto tile_out = [&](const float (&VA)[P_NA][2], const float (&VB)[P_NA][2], int tile, bool live, auto full_tag) {
        const int kk = kb + tile * P_TK + lane;
#pragma unroll
        for (int a = 0; a < P_NA; ++a) {
            const auto tA = __builtin_amdgcn_permlane32_swap(__float_as_uint(VA[a][0]), __float_as_uint(VA[a][1]), false, false);
            const auto tB = __builtin_amdgcn_permlane32_swap(__float_as_uint(VB[a][0]), __float_as_uint(VB[a][1]), false, false);
            emit(__uint_as_float(tA[0]), 4 * a + 0, kk, live, full_tag);
            emit(__uint_as_float(tB[0]), 4 * a + 1, kk, live, full_tag);
            emit(__uint_as_float(tA[1]), 4 * a + 2, kk, live, full_tag);
            emit(__uint_as_float(tB[1]), 4 * a + 3, kk, live, full_tag);
        }
    };
    // Software pipeline across tiles: the MFMAs of a tile's first sub-tile run beside the epilogue of
    // the previous tile's second sub-tile and that tile's list stores, and the MFMAs of the second
    // sub-tile beside the epilogue of the first, so that the VALU work always has MFMAs to hide
    // behind.  Carried from one tile to the next: the accumulators of the second sub-tile and the
    // scores of the first.  (At the first tile the carried state is empty and its stores are dropped,
    // which keeps the number of stores per step fixed.)
    f32x16_t pacc[P_NA];
    float pVA[P_NA], pVB[P_NA];
#pragma unroll
    for (int a = 0; a < P_NA; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[a][r] = 0.f;
        pVA[a] = pVB[a] = 0.f;
    }
    auto finish_prev = [&](int tile, bool live) {             // epilogue + stores of tile `tile`
        float qVA[P_NA][2], qVB[P_NA][2];
#pragma unroll
        for (int a = 0; a < P_NA; ++a) {
            qVA[a][0] = pVA[a];
            qVB[a][0] = pVB[a];
            block_scores(pacc[a], wv[a], qVA[a][1], qVB[a][1]);
        }
        // (one code path: a branch between variants would leave the compiler unsure of the number of
        // stores per step, and it would then add waits of its own before the tile reads)
        tile_out(qVA, qVB, tile, live, std::false_type{});
    };
    auto compute = [&](const uint16_t* buf, int tile) {
        const CSA_LDS char* lb = (const CSA_LDS char*)buf;
        // all B fragments of the tile are read up front (16 reads in flight): the MFMAs of the first
        // sub-tile wait for the first eight only, and LDS latency is paid once per tile
        u32x4_t bt[P_TK / 32][8];
#pragma unroll
        for (int j = 0; j < P_TK / 32; ++j)
#pragma unroll
            for (int s = 0; s < 8; ++s) bt[j][s] = *(const CSA_LDS u32x4_t*)(lb + ((boff ^ (32u * s)) + 8192u * j));
        __builtin_amdgcn_sched_barrier(0);
        f32x16_t acc0[P_NA], acc1[P_NA];
#pragma unroll
        for (int a = 0; a < P_NA; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc0[a][r] = 0.f; acc1[a][r] = 0.f; }
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int a = 0; a < P_NA; ++a) acc0[a] = mfma32_bf16(qa[a][s], as_bf16x8(bt[0][s]), acc0[a]);
        finish_prev(tile - 1, tile > 0);
        // one MFMA, then a share of the VALU work (the 32x32x16 MFMA leaves room for about six VALU
        // instructions beside it)
#pragma unroll
        for (int i = 0; i < 8 * P_NA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, P_VPM1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int a = 0; a < P_NA; ++a) acc1[a] = mfma32_bf16(qa[a][s], as_bf16x8(bt[1][s]), acc1[a]);
#pragma unroll
        for (int a = 0; a < P_NA; ++a) {
            block_scores(acc0[a], wv[a], pVA[a], pVB[a]);
            pacc[a] = acc1[a];
        }
#pragma unroll
        for (int i = 0; i < 8 * P_NA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x002, P_VPM2, 1);
        }
    };

    // ---- the tile pipeline: tile t in buffer t % NB, loads issued NB - 1 tiles ahead ----
    // Vector memory operations complete in issue order as far as vmcnt is concerned.  Step t
    // waits, passes the barrier, issues exactly P_DMA loads (tile t+NB-1, into buffer (t-1) % NB,
    // which every wave has finished reading once it is past this barrier) and then exactly P_QPW
    // stores (tile t's scores), with no branch around them.  Before the barrier of tile t each wave
    // waits for its own loads of tile t: issued after them are the loads of tiles t+1 .. t+NB-2 and
    // the stores of the min(t, NB-1) steps before, hence vmcnt((NB-2) P_DMA + min(t, NB-1) P_QPW).
    // Loads past the last tile reread clamped rows.
    constexpr int NB = P_NBUF;
    static_assert((NB - 2) * P_DMA + (NB - 1) * P_QPW < 64, "vmcnt field");
    auto wait_tile = [&](int t) {
        switch (min(t, NB - 1)) {
#define CSA_PWAIT(I) case I: if constexpr (I < NB) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 2) * P_DMA + I * P_QPW)); break;
            CSA_PWAIT(0) CSA_PWAIT(1) CSA_PWAIT(2) CSA_PWAIT(3) CSA_PWAIT(4) CSA_PWAIT(5) CSA_PWAIT(6) CSA_PWAIT(7)
#undef CSA_PWAIT
        }
    };
    auto step = [&](auto kc, int t) {
        constexpr int K = decltype(kc)::value;
        wait_tile(t + K);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(bufs[(K + NB - 1) % NB], t + K + NB - 1);
        compute(bufs[K], t + K);
    };
    if (ntiles > 0) {
#pragma unroll
        for (int i = 0; i < NB - 1; ++i) issue(bufs[i], i);
        for (int t = 0; t < ntiles; t += NB) {
#define CSA_PSTEP(K) if constexpr (K < NB) { if (t + K >= ntiles) break; step(std::integral_constant<int, K>{}, t); }
            CSA_PSTEP(0) CSA_PSTEP(1) CSA_PSTEP(2) CSA_PSTEP(3) CSA_PSTEP(4) CSA_PSTEP(5) CSA_PSTEP(6) CSA_PSTEP(7)
#undef CSA_PSTEP
        }
        finish_prev(ntiles - 1, true);         // the last tile's second sub-tile and stores
        __builtin_amdgcn_s_waitcnt(0);        // no tile load may still target this workgroup's LDS
    }
    if constexpr (MODE == 1) {
        if (lane < P_QPW) {
            uint32_t cv = 0;
#pragma unroll
            for (int lq = 0; lq < P_QPW; ++lq) cv = lane == lq ? C[lq] : cv;
            if (qw + lane < Tq) A.cnt[((size_t)b * Tq + qw + lane) * A.nsplit + split] = cv;
        }
    }
}

// P_NBUF tile buffers (distinct objects: the compiler tells a read of one from the loads in
// flight into another).
template <int MODE>
__global__ __launch_bounds__(P_TPB, 8 / P_NW) void k_pscore(PScoreArgs A)
{
#define CSA_PBUF(I) __shared__ __attribute__((aligned(1024))) uint16_t buf##I[I < P_NBUF ? P_TK * P_DI : 1];
    CSA_PBUF(0) CSA_PBUF(1) CSA_PBUF(2) CSA_PBUF(3) CSA_PBUF(4) CSA_PBUF(5) CSA_PBUF(6) CSA_PBUF(7)
#undef CSA_PBUF
    uint16_t* const all[8] = {buf0, buf1, buf2, buf3, buf4, buf5, buf6, buf7};
    uint16_t* bufs[P_NBUF];
#pragma unroll
    for (int i = 0; i < P_NBUF; ++i) bufs[i] = all[i];
    pscore_body<MODE>(bufs, A);
}

// ---------------------------------------------------------------------------
// k_pthresh: one wave per row.  The j-th largest sample key (16 bits) by a radix
// select over bins of the key range present in the row (min .. max), so that the
// few values most samples share do not pile their LDS atomics onto one bin.
// ---------------------------------------------------------------------------
// wave: the bin (of 1024, counted from the top) holding the need-th largest; returns {bin, count above it}.
// Lane L reads bins 1008 - 16 L .. 1023 - 16 L once (four 16-byte reads) and locates from registers.
__device__ __forceinline__ uint2 wave_find_bin1024(const uint32_t* h, uint32_t need) {
    const int lane = lane_id();
    const u32x4_t* hp = (const u32x4_t*)(h + 1008 - 16 * lane);
    uint32_t c[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const u32x4_t v = hp[q4];
        c[4 * q4] = v[0]; c[4 * q4 + 1] = v[1]; c[4 * q4 + 2] = v[2]; c[4 * q4 + 3] = v[3];
    }
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[i];
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    const uint32_t acc0 = incl - s;
    const bool found = acc0 < need && need <= incl;
    uint32_t bin = 0, above = 0, a = acc0;
    bool done = !found;
#pragma unroll
    for (int i = 15; i >= 0; --i) {                    // descending bins
        if (!done && a + c[i] >= need) { bin = 1008u - 16u * lane + i; above = a; done = true; }
        if (!done) a += c[i];
    }
    const unsigned long long fm = __builtin_amdgcn_ballot_w64(found);
    const int fl = fm ? (int)__builtin_ctzll(fm) : 0;
    return make_uint2((uint32_t)__builtin_amdgcn_readlane((int)bin, fl), (uint32_t)__builtin_amdgcn_readlane((int)above, fl));
}

__global__ __launch_bounds__(64) void k_pthresh(const uint16_t* __restrict__ samp, int NSP, int Tq, int Nc, long long L,
                                                 int m, long long pos0, int topk, float* __restrict__ thr)
{
    __shared__ __attribute__((aligned(16))) uint32_t h[1024];
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
    const uint16_t* sp = samp + (size_t)r * NSP;      // rows are 128-byte aligned (NSP % 64 == 0)
    const int nvec = (ns + 7) / 8;
    // visit every sample (8 per 16-byte load), f(x)
    // (chunks of 8 loads per lane, all issued before any is used)
    auto for_samples = [&](auto f) {
        for (int c0 = 0; c0 < nvec; c0 += 512) {
            u32x4_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {             // unconditional (clamped) loads: all in flight at once
                const int i = c0 + 64 * u + lane;
                v[u] = *(const u32x4_t*)(sp + 8 * min(i, nvec - 1));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = c0 + 64 * u + lane;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (8 * i + e < ns) f((v[u][e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
        }
    };
    uint32_t mn = 0xffffu, mx = 0u;
    for_samples([&](uint32_t x) { mn = min(mn, x); mx = max(mx, x); });
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
    }
    uint32_t base = mn, need = (uint32_t)j;
    int shift = max(0, 32 - (int)__clz((int)(mx - mn)) - 10), pshift = 32;
    for (;;) {
        for (int i = lane; i < 1024; i += 64) h[i] = 0;
        __syncthreads();
        for_samples([&](uint32_t x) {
            const uint32_t d = x - base;               // wraps for x < base: outside the range
            if (pshift >= 32 || d < (1u << pshift)) atomicAdd(&h[d >> shift], 1u);
        });
        __syncthreads();
        const uint2 fb = wave_find_bin1024(h, need);
        __syncthreads();
        base += fb.x << shift;
        need -= fb.y;
        if (shift == 0) break;
        pshift = shift;
        shift = max(0, shift - 10);
        __syncthreads();
    }
    if (lane == 0) thr[r] = key_f32(base << 16);
}

// ---------------------------------------------------------------------------
// k_pselect: one wave per row (SW_ROWS rows per workgroup, no workgroup barrier).
// The row's list segments are read in 64-entry slots: slot k of the wave holds, in
// lane L, entry 64 (k - first slot of its segment) + L of that segment, so that slot
// order and lane order follow the ascending index order (a segment's last slot is
// partly empty).  Keys and indices stay in registers; every step is wave-level.
// ---------------------------------------------------------------------------
constexpr int SW_SLOTS = 48;                  // 64-entry slots per row (3072 list entries minus padding)
constexpr int SW_BAND = 128;                  // band entries per row ranked in LDS
constexpr int SW_ROWS = 4;                    // rows (waves) per workgroup

// order-preserving LDS code motion fence within a wave (the LDS executes a wave's operations in order)
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Reductions over aligned groups of 8 lanes with DPP moves: swap neighbours, swap pairs, then
// mirror the two halves of the group (every lane ends with the group's result).
template <int CTRL> __device__ __forceinline__ int dpp8(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141;
__device__ __forceinline__ int g8_min(int v) {
    v = min(v, dpp8<DPP_XOR1>(v)); v = min(v, dpp8<DPP_XOR2>(v)); return min(v, dpp8<DPP_HALF_MIRROR>(v));
}
__device__ __forceinline__ int g8_max(int v) {
    v = max(v, dpp8<DPP_XOR1>(v)); v = max(v, dpp8<DPP_XOR2>(v)); return max(v, dpp8<DPP_HALF_MIRROR>(v));
}
template <int CTRL> __device__ __forceinline__ double dpp8_d(double v) {
    const unsigned long long u = __double_as_longlong(v);
    const int lo = dpp8<CTRL>((int)(uint32_t)u), hi = dpp8<CTRL>((int)(uint32_t)(u >> 32));
    return __longlong_as_double(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double g8_sum(double v) {     // exact here: every partial sum is representable
    v += dpp8_d<DPP_XOR1>(v); v += dpp8_d<DPP_XOR2>(v); return v + dpp8_d<DPP_HALF_MIRROR>(v);
}

// The bf16 pair c of a fragment word as two fp32 values.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// The exact score of one key row whose fragments sit in registers (lane L: head L / 8, elements
// 16 (L % 8) .. + 15 of q and k, bf16 pairs).  A bf16 product is an fp32 value with a 16-bit
// significand; when a head's products are normal and their exponents span at most 30, their fp64
// sum is exact (30 + 16 + 7 < 53 bits for 128 terms), and rounding it once to fp32 gives the
// correctly rounded head dot.  A span of up to 61 is split at 30 below the top exponent into two
// such exact sums, added with an error-free transformation and rounded once (a tie of the rounded
// sum is broken by the sign of the error).  Returns false (uniformly) outside these cases.
__device__ __forceinline__ bool band_score_frag(const u32x4_t (&qf)[2], const u32x4_t (&kf)[2], const float (&w)[P_HI],
                                                float& score) {
    double s = 0.0;
    int emin = 1000, emax = -1000, bad = 0;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const float x = hf ? bf_hi(qf[v][c]) : bf_lo(qf[v][c]);
                const float y = hf ? bf_hi(kf[v][c]) : bf_lo(kf[v][c]);
                const float pr = x * y;
                const int e = (int)((__float_as_uint(pr) >> 23) & 0xffu);
                if (x != 0.0f && y != 0.0f) {
                    bad |= e == 0 || e == 255;
                    emin = min(emin, e);
                    emax = max(emax, e);
                }
                s += (double)pr;
            }
    emin = g8_min(emin);
    emax = g8_max(emax);
    bad = g8_max(bad);
    float d;
    if (__builtin_amdgcn_ballot_w64(bad || emax - emin > 30) == 0ull) {
        d = (float)g8_sum(s);
    } else {
        if (__builtin_amdgcn_ballot_w64(bad || emax - emin > 61) != 0ull) return false;
        const int T = emax - emin > 30 ? emax - 30 : -1000;   // products below T form the low sum
        double hi = 0.0, lo = 0.0;
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float pr = (hf ? bf_hi(qf[v][c]) : bf_lo(qf[v][c])) * (hf ? bf_hi(kf[v][c]) : bf_lo(kf[v][c]));
                    const int e = (int)((__float_as_uint(pr) >> 23) & 0xffu);
                    if (e >= T) hi += (double)pr; else lo += (double)pr;
                }
        hi = g8_sum(hi);
        lo = g8_sum(lo);
        const double sm = hi + lo, bv = sm - hi;
        const double er = (hi - (sm - bv)) + (lo - bv);           // hi + lo = sm + er exactly
        d = (float)sm;
        if (er != 0.0 && sm > 0.0) {                               // only positive dots survive the relu
            if (sm < 0x1p-125 || sm > 0x1p+127) return false;      // (uniform: rare, outside the fp32 normal range)
            const unsigned long long bits = __double_as_longlong(sm);
            if ((bits & 0x1fffffffull) == 0x10000000ull) {        // sm is halfway between two floats
                if (er > 0.0 && (double)d < sm) d = __uint_as_float(__float_as_uint(d) + 1u);
                if (er < 0.0 && (double)d > sm) d = __uint_as_float(__float_as_uint(d) - 1u);
            }
        }
    }
    const float rr = d > 0.0f ? d : 0.0f;
    float sx = 0.0f;
#pragma unroll
    for (int hh = 0; hh < P_HI; ++hh)
        sx = __builtin_fmaf(w[hh], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rr), 8 * hh)), sx);
    score = sx;
    return true;
}

constexpr int SW_BG = 4;                      // band rows fetched together

__global__ __launch_bounds__(64 * SW_ROWS) void k_pselect(
    const uint2* __restrict__ cand, const uint32_t* __restrict__ cnt, const float* __restrict__ thr,
    const float* __restrict__ wq, const uint32_t* __restrict__ kmax, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const uint16_t* __restrict__ k_idx, int Tq, int Nc, long long L, int m,
    long long pos0, int topk, int nsplit, int caps, int R, int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out,
    float* __restrict__ score_out, uint32_t* __restrict__ fail)
{
    __shared__ uint32_t hist_all[SW_ROWS][1024];
    __shared__ unsigned long long bkey_all[SW_ROWS][SW_BAND];
    __shared__ uint32_t bpos_all[SW_ROWS][SW_BAND], bidx_all[SW_ROWS][SW_BAND];
    __shared__ unsigned long long chosen_all[SW_ROWS][SW_SLOTS];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
    const int r = blockIdx.x * SW_ROWS + wv;
    if (r >= R) return;                               // wave-uniform; nothing below synchronises waves
    uint32_t* h = hist_all[wv];
    unsigned long long* bkey = bkey_all[wv];
    uint32_t* bpos = bpos_all[wv];
    uint32_t* bidx = bidx_all[wv];
    unsigned long long* chosen = chosen_all[wv];
    const int b = r / Tq, t = r % Tq;
    const int nv = n_visible(pos0 + t, L, m, Nc);
    int32_t* out = idx_out + (size_t)r * topk;
    if (nv <= topk) {                                 // every visible entry is selected (no score is formed)
        for (int i = lane; i < topk; i += 64) {
            out[i] = i < nv ? i : -1;
            if (score_out) score_out[(size_t)r * topk + i] = __builtin_nanf("");
        }
        if (cnt_out && lane == 0) cnt_out[r] = nv;
        return;
    }
    auto give_up = [&]() {                            // the exact fallback takes the row
        if (lane == 0) fail[1 + atomicAdd(&fail[0], 1u)] = (uint32_t)r;
    };
    // segment counts (lane s holds segment s), slots per segment and their prefix
    const uint32_t mc = lane < nsplit ? cnt[(size_t)r * nsplit + lane] : 0u;
    const uint32_t msl = (mc + 63u) / 64u;
    uint32_t send = msl;                              // inclusive prefix of slot counts
#pragma unroll
    for (int o = 1; o < MAX_SPLIT; o <<= 1) {
        const uint32_t x = __shfl_up(send, o, 64);
        if (lane >= o) send += x;
    }
    uint32_t n = mc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) n += __shfl_xor(n, o, 64);
    n = (uint32_t)__builtin_amdgcn_readfirstlane((int)n);                 // uniform: kept in scalar registers
    const uint32_t nslots = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl((int)send, nsplit - 1, 64));
    const bool over = __builtin_amdgcn_ballot_w64(lane < nsplit && mc > (uint32_t)caps - 64u) != 0;
    if (over || n < (uint32_t)topk || nslots > (uint32_t)SW_SLOTS) { give_up(); return; }

    // ---- load: slot k belongs to segment seg(k) = #{s : send[s] <= k} ----
    // lane k works out slot k's first storage entry (seg caps + 64 (k - first slot of seg)) and its
    // number of entries; each slot then fetches both with a lane permute (kept in vector registers:
    // one scalar copy per slot would exhaust the scalar file)
    uint32_t soff = 0u, sval = 0u;
    {
        uint32_t seg = 0u;
#pragma unroll
        for (int s2 = 0; s2 < MAX_SPLIT; ++s2) {
            const uint32_t e = (uint32_t)__shfl((int)send, s2, 64);
            if (s2 < nsplit && e <= (uint32_t)lane) seg = (uint32_t)s2 + 1u;
        }
        const uint32_t sg = min(seg, (uint32_t)MAX_SPLIT - 1u);
        const uint32_t sbeg = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(4u * sg), (int)(send - msl));
        const uint32_t scnt = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(4u * sg), (int)mc);
        if ((uint32_t)lane < nslots && seg < (uint32_t)nsplit) {
            const uint32_t first = 64u * ((uint32_t)lane - sbeg);
            soff = seg * (uint32_t)caps + first;
            sval = min(64u, scnt - first);
        }
    }
    // every slot loads unconditionally (empty lanes reread the row's first entry), so that all the
    // loads are in flight before the first result is used; empty lanes are masked afterwards
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(cand + (size_t)r * nsplit * caps, (uint32_t)(nsplit * caps * 8));
    uint32_t key[SW_SLOTS], cid[SW_SLOTS];
#pragma unroll
    for (int k = 0; k < SW_SLOTS; ++k) {
        const uint32_t so = (uint32_t)__builtin_amdgcn_readlane((int)soff, k);
        const uint32_t sv = (uint32_t)__builtin_amdgcn_readlane((int)sval, k);
        const bool ok = (uint32_t)lane < sv;        // sval is 0 in lanes >= nslots
        const auto e = __builtin_amdgcn_raw_buffer_load_b64(crs, ok ? 8u * (so + (uint32_t)lane) : 0u, 0, 0);
        key[k] = e[1];
        cid[k] = e[0];
    }
    // the per-slot validity is derived again from an opaque copy of the slot sizes, so that the
    // compiler does not hold 48 lane masks in scalar registers across the loads
    uint32_t sval2 = sval;
    asm volatile("" : "+v"(sval2));
#pragma unroll
    for (int k = 0; k < SW_SLOTS; ++k) {              // 0 = empty (no finite score has order key 0)
        const uint32_t sv = (uint32_t)__builtin_amdgcn_readlane((int)sval2, k);
        key[k] = (uint32_t)lane < sv ? f32_key(__uint_as_float(key[k])) : 0u;
        asm volatile("" : "+v"(key[k]));
    }
    // ---- tau: radix select over 1024 bins of the key range present, then inside the chosen bin ----
    // (empty keys are 0: below every key, so they are excluded by "key >= base" tests below, and
    // kmn is the minimum of key - 1 + 1, where an empty key wraps to the top)
    uint32_t kmn = 0xffffffffu, kmx = 0u;
#pragma unroll
    for (int k = 0; k < SW_SLOTS; ++k) { kmn = min(kmn, key[k] - 1u); kmx = max(kmx, key[k]); }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, o, 64));
        kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, o, 64));
    }
    kmn += 1u;
    uint32_t base = kmn, need = (uint32_t)topk;
    {
        int shift = max(0, 32 - (int)__clz((int)(kmx - kmn)) - 10);
        uint32_t lim = 0xffffffffu;                   // the current bin spans keys base .. base + lim
        for (;;) {
#pragma unroll
            for (int i = 0; i < 4; ++i) *(u32x4_t*)(h + 4 * (lane + 64 * i)) = u32x4_t{0u, 0u, 0u, 0u};
            wave_lds_fence();
#pragma unroll
            for (int k = 0; k < SW_SLOTS; ++k) {
                const uint32_t d = key[k] - base;
                if (key[k] >= base && d <= lim) atomicAdd(&h[d >> shift], 1u);
            }
            wave_lds_fence();
            const uint2 fb = wave_find_bin1024(h, need);
            const uint32_t nbin = h[fb.x];
            wave_lds_fence();
            base += fb.x << shift;
            need -= fb.y;
            if (shift == 0) break;
            if (nbin <= 64u) {
                // few keys left in the bin: gather them into one register (lane j holds the j-th key met,
                // through the histogram's LDS, which is no longer needed) and take the need-th largest by
                // counting, instead of more histogram levels
                const uint32_t width = 1u << shift;
                uint32_t got = 0u;
#pragma unroll
                for (int k = 0; k < SW_SLOTS; ++k) {
                    const bool inb = key[k] >= base && key[k] - base < width;
                    const unsigned long long mb = __builtin_amdgcn_ballot_w64(inb);
                    if (mb) {                          // uniform
                        const uint32_t pos = got + __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u));
                        if (inb) h[pos] = key[k];
                        got += (uint32_t)__popcll(mb);
                    }
                }
                wave_lds_fence();
                const uint32_t mine = (uint32_t)lane < got ? h[lane] : 0u;
                uint32_t gt = 0u, ge = 0u;
                for (uint32_t i = 0; i < got; ++i) {
                    const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)mine, (int)i);
                    gt += y > mine;
                    ge += y >= mine;
                }
                const bool ok = (uint32_t)lane < got && gt < need && need <= ge;
                const unsigned long long om = __builtin_amdgcn_ballot_w64(ok);
                base = (uint32_t)__builtin_amdgcn_readlane((int)mine, om ? (int)__builtin_ctzll(om) : 0);
                break;
            }
            lim = (1u << shift) - 1u;
            shift = max(0, shift - 10);
        }
    }
    const float tau = key_f32(base);
    const double D = (double)wq[r] * (double)__uint_as_float(kmax[b]) * 1.52587890625e-05 * (1.0 + 1.0 / 512) +
                     1.1754943508222875e-38;
    const double lo = (double)tau - 2.0 * D, hi = (double)tau + 2.0 * D;
    if (!((double)thr[r] <= lo)) { give_up(); return; }       // the list might miss band entries

    // ---- classify: in (above hi) / band (listed in LDS with its slot position) / out ----
    // In the key domain with the bounds rounded outward to fp32: an entry just above hi may be
    // ranked with the band and one just below lo may join it, which changes nothing (the band
    // is ranked exactly, and the certain classes stay certain).
    uint32_t khi = f32_key((float)hi), klo = f32_key((float)lo);
    if ((double)key_f32(khi) < hi) khi += 1u;         // key of the smallest float >= hi
    if ((double)key_f32(klo) > lo) klo -= 1u;         // key of the largest float <= lo
    klo = max(klo, 1u);                               // empty keys (0) belong to no class
    // the class is kept in the two top bits of the entry's index (bit 31: in, bit 30: band)
    uint32_t n_in = 0, nb = 0;
#pragma unroll
    for (int k = 0; k < SW_SLOTS; ++k) {
        const bool f_in = key[k] > khi;
        const bool f_band = key[k] <= khi && key[k] >= klo;
        const unsigned long long mi = __builtin_amdgcn_ballot_w64(f_in), mb = __builtin_amdgcn_ballot_w64(f_band);
        if (mb) {                                     // uniform
            const uint32_t slot = nb + __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u));
            if (f_band && slot < (uint32_t)SW_BAND) { bidx[slot] = cid[k]; bpos[slot] = 64u * k + lane; }
        }
        cid[k] |= (f_in ? 0x80000000u : 0u) | (f_band ? 0x40000000u : 0u);
        asm volatile("" : "+v"(cid[k]));              // tag now: no lane masks carried to the output scan
        n_in += (uint32_t)__popcll(mi);
        nb += (uint32_t)__popcll(mb);
    }
    if (nb > (uint32_t)SW_BAND || n_in > (uint32_t)topk || (uint32_t)topk - n_in > nb) { give_up(); return; }
    const uint32_t needb = (uint32_t)topk - n_in;
    if (lane < SW_SLOTS) chosen[lane] = 0ull;
    wave_lds_fence();

    // ---- exact scores of the band, composite keys (score key, inverted index), rank, choose ----
    if (needb > 0 && needb < nb) {
        const uint16_t* qrow = q_idx + (size_t)r * P_HI * P_DI;
        const float* wrow = w_idx + (size_t)r * P_HI;
        const int sub = lane & 7;
        u32x4_t qf[2];
        qf[0] = *(const u32x4_t*)(qrow + (lane >> 3) * P_DI + 16 * sub);
        qf[1] = *(const u32x4_t*)(qrow + (lane >> 3) * P_DI + 16 * sub + 8);
        float w[P_HI];
#pragma unroll
        for (int hh = 0; hh < P_HI; ++hh) w[hh] = wrow[hh];
        const uint16_t* kseq = k_idx + (size_t)b * Nc * P_DI + 16 * sub;
        for (uint32_t i0 = 0; i0 < nb; i0 += SW_BG) {
            // the group's key rows are fetched together (a short group rereads its last row)
            u32x4_t kf[SW_BG][2];
            uint32_t gi[SW_BG];
#pragma unroll
            for (int g = 0; g < SW_BG; ++g) {
                gi[g] = bidx[min(i0 + (uint32_t)g, nb - 1u)];
                const uint16_t* kp = kseq + (size_t)gi[g] * P_DI;
                kf[g][0] = *(const u32x4_t*)kp;
                kf[g][1] = *(const u32x4_t*)(kp + 8);
            }
#pragma unroll
            for (int g = 0; g < SW_BG; ++g) {
                if (i0 + (uint32_t)g < nb) {
                    float sx;
                    // outside the fp64 case (rare) the exact fallback takes the row
                    if (!band_score_frag(qf, kf[g], w, sx)) { give_up(); return; }
                    if (lane == 0) bkey[i0 + g] = ((unsigned long long)f32_key(sx) << 32) | (0xffffffffu - gi[g]);
                }
            }
        }
        wave_lds_fence();
        for (uint32_t i = lane; i < nb; i += 64) {
            const unsigned long long ki = bkey[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < nb; ++j) rank += bkey[j] > ki;
            if (rank < needb) atomicOr(&chosen[bpos[i] >> 6], 1ull << (bpos[i] & 63));
        }
    } else if (needb == nb) {
        for (uint32_t i = lane; i < nb; i += 64) atomicOr(&chosen[bpos[i] >> 6], 1ull << (bpos[i] & 63));
    }
    wave_lds_fence();

    // ---- the chosen indices in ascending order: a ballot scan over the slots ----
    // lane k holds the chosen-band mask of slot k; each slot reads it with lane reads
    const unsigned long long cm = lane < SW_SLOTS ? chosen[lane] : 0ull;
    const uint32_t cm_lo = (uint32_t)cm, cm_hi = (uint32_t)(cm >> 32);
    uint32_t o = 0;
#pragma unroll
    for (int k = 0; k < SW_SLOTS; ++k) {
        if ((uint32_t)k < nslots) {
            const uint32_t clo = (uint32_t)__builtin_amdgcn_readlane((int)cm_lo, k);
            const uint32_t chi = (uint32_t)__builtin_amdgcn_readlane((int)cm_hi, k);
            const uint32_t cw = lane < 32 ? clo : chi;
            const bool sel = (cid[k] >> 31) || (((cid[k] >> 30) & 1u) && ((cw >> (lane & 31)) & 1u));
            const unsigned long long ms = __builtin_amdgcn_ballot_w64(sel);
            const uint32_t pos = o + __builtin_amdgcn_mbcnt_hi((uint32_t)(ms >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ms, 0u));
            if (sel && pos < (uint32_t)topk) {
                out[pos] = (int32_t)(cid[k] & 0x3fffffffu);
                if (score_out) {                      // the approximate score it was ranked by, from the list
                    const uint32_t so = (uint32_t)__builtin_amdgcn_readlane((int)soff, k);
                    score_out[(size_t)r * topk + pos] =
                        __uint_as_float(cand[(size_t)r * nsplit * caps + so + (uint32_t)lane].y);
                }
            }
            o += (uint32_t)__popcll(ms);
        }
    }
    if (cnt_out && lane == 0) cnt_out[r] = topk;
}

// ---------------------------------------------------------------------------
// Exact fallback for the rows the certified path gave up on.  The first FB_SLOTS
// failed rows: k_pfb_score spreads the exact scores of their visible entries over
// the whole grid (a score key per entry), then k_pfb_rows selects each row's
// top-k from its stored keys with one workgroup.  Rows beyond FB_SLOTS (only when
// more than FB_SLOTS rows fail) are scored and selected by the same workgroups
// afterwards, one row at a time.
// ---------------------------------------------------------------------------
constexpr int FB_CH = 512;                    // workgroups of k_pfb_score (4 waves each)
constexpr int FB_G = 8;                       // key rows fetched together per wave

// exact score keys K[s] of entries s = s0, s0 + step, .. < nv of row r (one wave)
__device__ __forceinline__ void fb_score_entries(int r, int b, int nv, int s0, int step,
                                                 const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
                                                 const uint16_t* __restrict__ k_idx, int Nc, uint32_t* K) {
    const int lane = lane_id(), sub = lane & 7;
    const uint16_t* qrow = q_idx + (size_t)r * P_HI * P_DI;
    const float* wrow = w_idx + (size_t)r * P_HI;
    u32x4_t qf[2];
    qf[0] = *(const u32x4_t*)(qrow + (lane >> 3) * P_DI + 16 * sub);
    qf[1] = *(const u32x4_t*)(qrow + (lane >> 3) * P_DI + 16 * sub + 8);
    float w[P_HI];
#pragma unroll
    for (int hh = 0; hh < P_HI; ++hh) w[hh] = wrow[hh];
    const uint16_t* kseq = k_idx + (size_t)b * Nc * P_DI;
    for (int s = s0; s < nv; s += FB_G * step) {
        u32x4_t kf[FB_G][2];
#pragma unroll
        for (int g = 0; g < FB_G; ++g) {
            const uint16_t* kp = kseq + (size_t)min(s + g * step, nv - 1) * P_DI + 16 * sub;
            kf[g][0] = *(const u32x4_t*)kp;
            kf[g][1] = *(const u32x4_t*)(kp + 8);
        }
#pragma unroll
        for (int g = 0; g < FB_G; ++g) {
            const int e = s + g * step;
            if (e < nv) {
                float sx;
                if (!band_score_frag(qf, kf[g], w, sx))
                    sx = wave_exact_score<0, P_DI, P_HI>(qrow, wrow, kseq + (size_t)e * P_DI);
                if (lane == 0) K[e] = f32_key(sx);
            }
        }
    }
}

// top-k of one row from its exact score keys K[0, nv) (a 1024-thread workgroup): the
// topk-th largest key tau by radix levels over 1024 bins of the key range present,
// then every entry above tau and the lowest-indexed entries equal to tau, ascending.
// Thread t owns the contiguous entries [t per, (t + 1) per), per a multiple of 64, read
// 64 at a time with 16-byte loads (K holds a multiple of 64 keys).
__device__ __forceinline__ void fb_select_row(const uint32_t* K, int nv, int topk, int32_t* out, float* sout, uint32_t* h,
                                              uint32_t* red) {
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int per = ((nv + FB_TPB - 1) / FB_TPB + 63) & ~63;
    const int s0 = min(nv, tid * per), s1 = min(nv, s0 + per);
    auto for_any = [&](auto&& f) {                    // every key once, in any order (coalesced)
        for (int c = 4 * tid; c < nv; c += 32 * FB_TPB) {
            u32x4_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = *(const u32x4_t*)(K + min(c + 4 * FB_TPB * j, (nv - 1) & ~3));
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c + 4 * FB_TPB * j + e < nv) f(v[j][e]);
        }
    };
    auto for_keys = [&](auto&& f) {                   // this thread's keys in ascending order
        for (int c = s0; c < s1; c += 64) {
            u32x4_t v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = *(const u32x4_t*)(K + c + 4 * j);
#pragma unroll
            for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c + 4 * j + e < s1) f(c + 4 * j + e, v[j][e]);
        }
    };
    uint32_t mn = 0xffffffffu, mx = 0u;
    for_any([&](uint32_t x) { mn = min(mn, x); mx = max(mx, x); });
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
    }
    if (lane == 0) { red[2 * wave] = mn; red[2 * wave + 1] = mx; }
    __syncthreads();
    mn = 0xffffffffu; mx = 0u;
    for (int w2 = 0; w2 < FB_TPB / 64; ++w2) { mn = min(mn, red[2 * w2]); mx = max(mx, red[2 * w2 + 1]); }
    __syncthreads();
    uint32_t base = mn, need = (uint32_t)topk, lim = 0xffffffffu;
    int shift = max(0, 32 - (int)__clz((int)(mx - mn)) - 10);
    for (;;) {
        for (int i = tid; i < 1024; i += FB_TPB) h[i] = 0;
        __syncthreads();
        for_any([&](uint32_t x) {
            const uint32_t d = x - base;
            if (x >= base && d <= lim) atomicAdd(&h[d >> shift], 1u);
        });
        __syncthreads();
        if (wave == 0) {
            const uint2 fb = wave_find_bin1024(h, need);
            if (lane == 0) { red[0] = fb.x; red[1] = fb.y; }
        }
        __syncthreads();
        base += red[0] << shift;
        need -= red[1];
        __syncthreads();
        if (shift == 0) break;
        lim = (1u << shift) - 1u;
        shift = max(0, shift - 10);
    }
    // tau = base; need entries equal to tau are taken, the lowest indices first
    uint32_t gt = 0, eq = 0;
    for_keys([&](int, uint32_t x) { gt += x > base; eq += x == base; });
    uint32_t tot;
    const uint32_t eq0 = block_scan(eq, red, &tot);
    const uint32_t mine = gt + min(eq, need > eq0 ? need - eq0 : 0u);
    uint32_t o = block_scan(mine, red, &tot);
    uint32_t e = eq0;
    for_keys([&](int s, uint32_t x) {
        const bool sel = x > base || (x == base && (e++) < need);
        if (sel && o < (uint32_t)topk) {
            if (sout) sout[o] = key_f32(x);           // the exact score
            out[o++] = s;
        }
    });
}

__global__ __launch_bounds__(256) void k_pfb_score(
    const uint32_t* __restrict__ fail, const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, int Tq, int Nc, long long L, int m, long long pos0, uint32_t* __restrict__ keys,
    size_t NcP)
{
    const uint32_t nf = min(fail[0], (uint32_t)FB_SLOTS);
    const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = gridDim.x * 4;
    for (uint32_t fi = 0; fi < nf; ++fi) {
        const int r = (int)fail[1 + fi], b = r / Tq, t = r % Tq;
        const int nv = n_visible(pos0 + t, L, m, Nc);
        fb_score_entries(r, b, nv, gw, nw, q_idx, w_idx, k_idx, Nc, keys + (size_t)fi * NcP);
    }
}

// One workgroup per fallback slot x: first the top-k of failed row x (x < FB_SLOTS) from the score keys
// k_pfb_score stored in region x, then (only when more than FB_SLOTS rows failed) rows FB_SLOTS + x,
// FB_SLOTS + x + gridDim.x, .., each scored by this workgroup itself into the same region and selected.
__global__ __launch_bounds__(FB_TPB) void k_pfb_rows(
    const uint32_t* __restrict__ fail, const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, int Tq, int Nc, long long L, int m, long long pos0, int topk,
    uint32_t* __restrict__ keys, size_t NcP, int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out,
    float* __restrict__ score_out)
{
    __shared__ __align__(16) uint32_t h[1024];
    __shared__ uint32_t red[2 * (FB_TPB / 64)];
    const uint32_t nf = fail[0];
    if (blockIdx.x >= nf) return;                      // (uniform) nothing failed for this slot
    uint32_t* K = keys + (size_t)blockIdx.x * NcP;
    {
        const int r = (int)fail[1 + blockIdx.x], t = r % Tq;
        const int nv = n_visible(pos0 + t, L, m, Nc);
        fb_select_row(K, nv, topk, idx_out + (size_t)r * topk, score_out ? score_out + (size_t)r * topk : nullptr,
                      h, red);
        if (cnt_out && threadIdx.x == 0) cnt_out[r] = topk;
        __syncthreads();                               // K is reused below
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (uint32_t fi = FB_SLOTS + blockIdx.x; fi < nf; fi += gridDim.x) {
        const int r = (int)fail[1 + fi], b = r / Tq, t = r % Tq;
        const int nv = n_visible(pos0 + t, L, m, Nc);
        fb_score_entries(r, b, nv, wave, FB_TPB / 64, q_idx, w_idx, k_idx, Nc, K);
        __threadfence_block();
        __syncthreads();
        fb_select_row(K, nv, topk, idx_out + (size_t)r * topk, score_out ? score_out + (size_t)r * topk : nullptr,
                      h, red);
        if (cnt_out && threadIdx.x == 0) cnt_out[r] = topk;
        __syncthreads();                               // K is reused by the next row
    }
}

// k_pwiden: rows of the many-query layout (P_HI heads x P_DI bf16) from rows of hin heads x dI elements
// in format dtype (0 bf16, 1 e4m3, 2 MXFP4 with one E8M0 scale per 32 elements); output row o is head
// o % P_HI (or the key row o when hin = 1 and hout = 1) of group o / hout.  One thread per 16-byte
// output chunk (grid-stride); heads past hin and dims past dI are zero.
__global__ __launch_bounds__(256) void k_pwiden(const void* __restrict__ src, const uint8_t* __restrict__ scale,
                                                int dtype, long long nout, int hout, int hin, int dI,
                                                uint16_t* __restrict__ dst)
{
    constexpr int CPR = P_DI / 8;                      // 16-byte chunks per output row
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nout * CPR;
         i += (long long)gridDim.x * blockDim.x) {
        const long long o = i / CPR;
        const int c = (int)(i % CPR), h = (int)(o % hout);
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (h < hin && 8 * c < dI) {
            const long long r = o / hout * hin + h;         // source row
            if (dtype == 0) {
                v = *(const u32x4_t*)((const uint16_t*)src + r * dI + 8 * c);
            } else if (dtype == 1) {
                const uint2 x = *(const uint2*)((const uint8_t*)src + r * dI + 8 * c);
                v = e4m3x8_to_bf16x8(x.x, x.y);
            } else {
                const uint32_t x = *(const uint32_t*)((const uint8_t*)src + r * (dI / 2) + 4 * c);
                v = fp4x8_to_bf16x8(x, e8m0_scale(scale[r * (dI / 32) + c / 4]));
            }
        }
        *(u32x4_t*)(dst + o * P_DI + 8 * c) = v;
    }
}

// head weights of the many-query layout: P_HI per row, +0 past hin
__global__ __launch_bounds__(256) void k_pwiden_w(const float* __restrict__ w, long long R, int hin, float* __restrict__ dst)
{
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < R * P_HI;
         i += (long long)gridDim.x * blockDim.x) {
        const int h = (int)(i % P_HI);
        dst[i] = h < hin ? w[i / P_HI * hin + h] : 0.0f;
    }
}

// clears the Kmax accumulators [n] and the fallback row count
__global__ void k_pzero(uint32_t* p, int n, uint32_t* fail) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
    if (i == 0) fail[0] = 0;
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
        int ns = (P_UNITS + units - 1) / units;
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

// operands the kernels read as they are (others are widened first)
static bool prefill_direct(int dtype, int HI, int dI) { return dtype == 0 && HI == P_HI && dI == P_DI; }

bool prefill_index_applicable(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk) {
    const bool fmt = (dtype == 0 || dtype == 1) ? (dI == 64 || dI == P_DI) : (dtype == 2 && dI == P_DI);
    return fmt && (HI == 1 || HI == 2 || HI == 4 || HI == P_HI) && Tq >= 64 && topk <= 1024 && Nc >= 1 &&
           (size_t)Nc * P_ROW_B < ((size_t)1 << 31) && (size_t)B * Tq <= ((size_t)1 << 24);
}

// widened operands at the start of the workspace: keys [B][Nc][P_DI] bf16 | queries [R][P_HI][P_DI] bf16 |
// head weights [R][P_HI] f32
static size_t prefill_widen_bytes(int dtype, int HI, int dI, int B, int Tq, int Nc) {
    if (prefill_direct(dtype, HI, dI)) return 0;
    const size_t R = (size_t)B * Tq;
    return align256((size_t)B * Nc * P_ROW_B) + align256(R * P_HI * P_ROW_B) + align256(R * P_HI * 4);
}

// kmax [B] | fail [1 + R] | wq [R] | thr [R] | samp [R][NSP] u16 | cnt [R][nsplit1] | cand [R][nsplit1][caps]
// | fallback score keys [FB_SLOTS][NcP] u32
size_t prefill_index_ws_bytes(int dtype, int HI, int dI, int B, int Tq, int Nc) {
    const PrefillPlan P = prefill_plan(B, Tq, Nc);
    return prefill_widen_bytes(dtype, HI, dI, B, Tq, Nc) + align256((size_t)B * 4) + align256((P.R + 1) * 4) + align256(P.R * 4) + align256(P.R * 4) +
           align256(P.R * P.NSP * 2) + align256(P.R * P.nsplit1 * 4) + align256(P.R * P.nsplit1 * P.caps * 8) +
           align256((size_t)FB_SLOTS * P.NcP * 4);
}

int prefill_index_launch(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int HI, int dI, int B,
                         int Tq, int Nc, long long L, int m, long long pos0, int topk, int32_t* idx_out,
                         int32_t* cnt_out, float* score_out, const uint8_t* q_scale, const uint8_t* k_scale, void* ws,
                         hipStream_t st) {
    const PrefillPlan P = prefill_plan(B, Tq, Nc);
    char* p = (char*)ws;
    if (!prefill_direct(dtype, HI, dI)) {
        uint16_t* kw = (uint16_t*)p;        p += align256((size_t)B * Nc * P_ROW_B);
        uint16_t* qw = (uint16_t*)p;        p += align256(P.R * P_HI * P_ROW_B);
        float* ww = (float*)p;              p += align256(P.R * P_HI * 4);
        const long long nk = (long long)B * Nc, nq = (long long)P.R * P_HI, cpr = P_DI / 8;
        auto blocks = [](long long n) { return dim3((unsigned)std::min<long long>((n + 255) / 256, 65536)); };
        CSA_LAUNCH("k_pwiden", k_pwiden, blocks(nk * cpr), dim3(256), 0, st, k_idx, k_scale, dtype, nk, 1, 1, dI, kw);
        CSA_LAUNCH("k_pwiden", k_pwiden, blocks(nq * cpr), dim3(256), 0, st, q_idx, q_scale, dtype, nq, P_HI, HI, dI,
                   qw);
        CSA_LAUNCH("k_pwiden", k_pwiden_w, blocks(nq), dim3(256), 0, st, w_idx, (long long)P.R, HI, ww);
        k_idx = kw;
        q_idx = qw;
        w_idx = ww;
    }
    uint32_t* kmax = (uint32_t*)p;          p += align256((size_t)B * 4);
    uint32_t* fail = (uint32_t*)p;          p += align256((P.R + 1) * 4);
    float* wq = (float*)p;                  p += align256(P.R * 4);
    float* thr = (float*)p;                 p += align256(P.R * 4);
    uint16_t* samp = (uint16_t*)p;          p += align256(P.R * P.NSP * 2);
    uint32_t* cnt = (uint32_t*)p;           p += align256(P.R * P.nsplit1 * 4);
    uint2* cand = (uint2*)p;                p += align256(P.R * P.nsplit1 * P.caps * 8);
    uint32_t* fbk = (uint32_t*)p;
    const uint16_t* q = (const uint16_t*)q_idx;
    const uint16_t* k = (const uint16_t*)k_idx;

    CSA_LAUNCH("k_pzero", k_pzero, dim3((B + 255) / 256), dim3(256), 0, st, kmax, B, fail);
    {
        const long long nb = ((long long)B * Nc + NORM_KEYS_PER_BLOCK - 1) / NORM_KEYS_PER_BLOCK + ((long long)P.R + 3) / 4;
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
    CSA_LAUNCH("k_pselect", k_pselect, dim3((unsigned)((P.R + SW_ROWS - 1) / SW_ROWS)), dim3(64 * SW_ROWS), 0, st, cand,
               cnt, thr, wq, kmax, q, w_idx, k, Tq, Nc, L, m, pos0, topk, P.nsplit1, P.caps, (int)P.R, idx_out, cnt_out,
               score_out, fail);
    CSA_LAUNCH("k_pfb_score", k_pfb_score, dim3(FB_CH), dim3(256), 0, st, fail, q, w_idx, k, Tq, Nc, L, m, pos0, fbk,
               P.NcP);
    CSA_LAUNCH("k_pfb_rows", k_pfb_rows, dim3(FB_SLOTS), dim3(FB_TPB), 0, st, fail, q, w_idx, k, Tq, Nc, L, m, pos0,
               topk, fbk, P.NcP, idx_out, cnt_out, score_out);
    return 0;
}

}  // namespace csa_host

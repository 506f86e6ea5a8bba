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
//   k_fill     zero the per-row histogram and error maximum
//   k_score    the HBM-bound pass: v_mfma_f32_16x16x32_bf16 approximate scores
//              S~ (e4m3 keys are widened to bf16 exactly in registers), a
//              rigorous per-entry error bound from a second MFMA on |q|, |k|,
//              a 4096-bin histogram of the top 12 bits of S~ and the row's
//              largest bound Dmax
//   k_collect  every entry that can still reach the top-k (S~ >= lower edge of
//              the bin holding the k-th largest, minus 2 Dmax) -> a per-row
//              candidate list of (index, S~), one region per workgroup
//   k_select   one workgroup per row: exact k-th largest S~ (tau) from the
//              level-1 bin plus a 12-bit and an 8-bit level over the
//              candidates; S~ > tau + 2 Dmax is certainly selected,
//              S~ < tau - 2 Dmax certainly not; the band in between is rescored
//              exactly (wave-cooperative exact dot products) and its remaining
//              slots go by (exact S desc, index asc); the candidates are kept in
//              index order, so one prefix scan writes the k indices ascending.
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
constexpr int BINS2 = 4096;                  // (k_select, in LDS) key bits 19..8 inside the threshold bin
constexpr int HW_DMAX = BINS1;               // per row: the largest error bound
constexpr int HW_B1 = BINS1 + 2, HW_A1 = BINS1 + 3;    // level-1 bin of tau; count above it
constexpr int HIST_WORDS = BINS1 + 8;
constexpr int TPB = 256;
constexpr int KPW_MAX = 4096;               // keys per scoring workgroup, at most


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



// LDS accesses of the ring sweep in k_score, in asm: the compiler cannot tell the ring (written by loads to
// LDS) from the other LDS arrays, so it would hold every LDS access of the sweep until all loads in flight had
// landed, draining the ring at each tile.  A read block waits for its own results.
__device__ __forceinline__ uint32_t lds_addr(const CSA_LDS void* p) { return (uint32_t)(size_t)p; }
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(size_t)(const CSA_LDS void*)p; }
template <int N>
__device__ __forceinline__ void lds_read_b128(u32x4_t (&v)[N], uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 reads");
    if constexpr (N == 1)
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a0) : "memory");
    else if constexpr (N == 2)
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]) : "v"(a0), "v"(a1) : "memory");
    else
        asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(a0), "v"(a1), "v"(a2), "v"(a3) : "memory");
}
__device__ __forceinline__ uint32_t lds_read_b32(uint32_t a) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
    return v;
}
__device__ __forceinline__ void lds_write_b32(uint32_t a, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_add_u32(uint32_t a, uint32_t v) {
    asm volatile("ds_add_u32 %0, %1" ::"v"(a), "v"(v) : "memory");
}

// ---------------------------------------------------------------------------
// k_score
// ---------------------------------------------------------------------------
// MFMA roles: A = 16 query columns (row t, head h; heads padded to HP = max(HI, 4)),
// B = 16 keys, both loaded as 1/4 of a row per lane (the same k-slot order),
// so D[column][key] leaves every lane with HP/4... 4 heads of one key: the
// head reduction is mostly lane-local (one xor-16 shuffle for HP = 8).
template <int DT, int DI, int HI, bool PAGED, bool RING>
__global__ __launch_bounds__(TPB) void k_score(
    const void* __restrict__ q_idx, const float* __restrict__ w_idx, const void* __restrict__ k_idx,
    int Tq, int Nc, int NcP, long long L, int m, long long pos0, int keys_per_wg, int topk,
    float* __restrict__ S, uint32_t* __restrict__ hist, const long long* __restrict__ seq_lens, PageMap pm,
    const uint8_t* __restrict__ q_scale, const uint8_t* __restrict__ k_scale)
{
    constexpr int STEPS = DI / 32;            // bf16 16x16x32 MFMAs per 16-key tile
    constexpr int EPL = DI / 4;               // key elements per lane
    constexpr int KB = DT == 0 ? EPL * 2 : (DT == 1 ? EPL : EPL / 2);   // key bytes per lane
    constexpr int NV = KB / 16;               // 16-byte loads per lane per tile
    constexpr int U = 128 / KB;                // tiles per load batch (bytes per lane in flight)
    constexpr int HP = HI < 4 ? 4 : HI;       // padded heads per query row
    constexpr int G = 16 / HP;                // query rows per column group
    constexpr int LPR = HP / 4;               // lanes (of one key) holding one row's heads
    constexpr int RB = DT == 0 ? DI * 2 : (DT == 1 ? DI : DI / 2);     // bytes per key / query-head row
    static_assert(DT != 2 || DI == 128, "MXFP4 rows: one 32-element scale block per lane group");
    // RING: the keys stream through a per-wave ring of NS 16-key tiles in LDS, filled by loads to LDS in
    // which each 64-lane instruction moves 1 KiB of contiguous rows (the register loads below read 16 rows
    // x 64 bytes per instruction); only for groups whose rows all keep their histogram in LDS (NL = 1),
    // so that the sweep issues no other vector-memory instruction and the load counts stay exact.
    static_assert(!RING || (DT != 2 && G >= 1), "ring sweep: bf16 / e4m3 keys");
    constexpr int NL = RING ? 1 : 2;          // rows of a group with LDS histograms
    constexpr int TILEB = 16 * RB;            // bytes of one 16-key tile
    constexpr int NS = RING ? (32768 / 4) / TILEB : 1;   // ring slots per wave (32 KiB per workgroup)
    static_assert(!RING || (NS >= 2 && TILEB % 1024 == 0), "ring: >= 2 slots of whole 1 KiB loads");

    __shared__ uint32_t lh[NL][BINS1];        // histograms of up to NL rows of a group
    __shared__ uint32_t ldmax[NL];
    // the same rows' scores, written out in 16-byte stores after the key sweep (scattered 4-byte stores
    // between the key loads cost the stream ~9% of its rate)
    __shared__ __attribute__((aligned(16))) float lsc[NL][KPW_MAX];
    __shared__ __attribute__((aligned(16))) uint8_t ring[RING ? 4 * NS * TILEB : 16];
    // paged keys: the pool page of every page the workgroup's key range touches, read once here, so that a
    // key load waits on no table load (a table load between two key batches made the wait for it wait for
    // the batch in flight as well).  Sized for pages of >= 2 entries, which keeps two workgroups per CU;
    // pages of one entry read the table per key.
    constexpr int PG_CAP = KPW_MAX / 2 + 1;
    __shared__ uint32_t lpg[PAGED ? PG_CAP : 1];

    const int b = blockIdx.y;
    const int lane = lane_id(), wave = RING ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int key0 = blockIdx.x * keys_per_wg;
    const int NG = (Tq + G - 1) / G;
    const int tiles = keys_per_wg / 64;       // 16-key tiles per wave
    const int pg0 = PAGED ? key0 >> pm.eshift : 0;
    const bool pg_lds = PAGED && pm.eshift > 0;        // (uniform)
    if (pg_lds) {
        const int np = ((key0 + keys_per_wg - 1) >> pm.eshift) - pg0 + 1;     // <= keys_per_wg / 2 + 1
        for (int i = threadIdx.x; i < np; i += TPB) {
            const int pi = pg0 + i;
            uint32_t blk = pi < pm.max_blocks ? (uint32_t)pm.table[(size_t)b * pm.max_blocks + pi] : 0u;
            lpg[i] = blk < (uint32_t)pm.nblocks ? blk : (uint32_t)pm.nblocks - 1u;   // clamped like entry_row
        }
        // (the barrier at the top of the row-group loop publishes lpg)
    }

    for (int g = 0; g < NG; ++g) {
        const int nrow = min(G, Tq - g * G);
        const int nlds = min(nrow, NL);
        for (int i = threadIdx.x; i < nlds * BINS1; i += TPB) (&lh[0][0])[i] = 0;
        if (threadIdx.x < NL) ldmax[threadIdx.x] = 0;
        __syncthreads();

        // A operand: query column `col` = (row ta, head ha)
        const int ta = g * G + col / HP, ha = col % HP;
        const bool av = ta < Tq && ha < HI;
        bf16x8_t qb[STEPS], qa[STEPS];
        u32x4_t qf8a[2];                      // |q| as raw e4m3 bytes (DT == 1)
        // Element order of the contraction (shared by Q and K): lane group grp takes the 16-byte chunks
        // at bytes 64 i + 16 grp of a row, so that one load instruction reads 64 contiguous bytes of
        // each of its 16 key rows.  bf16: k-step s = chunk s; e4m3: k-step s = half (s & 1) of chunk s / 2;
        // MXFP4: the lane group's one chunk holds elements 32 grp .. 32 grp + 31 (one scale block), and
        // k-step s takes its dword s.
        if (av) {
            const size_t r = (size_t)b * Tq + ta;
            const char* qp = (const char*)q_idx + (r * HI + ha) * RB + (size_t)grp * 16;
            float qsc = 1.f;
            u32x4_t qw = u32x4_t{0, 0, 0, 0};
            if (DT == 2) {
                qsc = e8m0_scale(q_scale[(r * HI + ha) * (DI / 32) + grp]);
                qw = *(const u32x4_t*)qp;
            }
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                u32x4_t v;
                if (DT == 0) v = *(const u32x4_t*)(qp + s * 64);
                else if (DT == 2) v = fp4x8_to_bf16x8(qw[s], qsc);
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
        const int nv = rv ? row_visible(seq_lens, b, tr, Tq, L, pos0, m, Nc) : 0;
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
        // (rows past the last visible entry reread it: branch-free loads keep the wait counts exact, so
        //  the next batch stays in flight; those keys are never written)
        auto load_batch = [&](int tt0, u32x4_t (&dst)[U][NV], uint32_t (&dsc)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int krow = min(key0 + ((tt0 + u) * 4 + wave) * 16 + col, nvmax - 1);
                const size_t prow = !PAGED ? (size_t)b * Nc + krow
                                  : pg_lds ? ((size_t)lpg[(krow >> pm.eshift) - pg0] << pm.eshift) |
                                                 (size_t)(krow & ((1 << pm.eshift) - 1))
                                           : entry_row(pm, b, Nc, krow);
                const char* kp = (const char*)k_idx + prow * RB + (size_t)grp * 16;
#pragma unroll
                for (int i = 0; i < NV; ++i) dst[u][i] = *(const u32x4_t*)(kp + i * 64);
                if (DT == 2) dsc[u] = k_scale[prow * (DI / 32) + grp];
            }
        };
        // one 16-key tile: kv = this lane's NV chunks of key kbase + col, sc its MXFP4 scale byte
        auto compute_tile = [&](int kbase, const u32x4_t (&kv)[NV], uint32_t sc_b) {
                    // (tiles past the visible keys are computed and dropped: no branch between the
                    //  loads and their uses)
                    f32x4_t acc = {0, 0, 0, 0}, aacc = {0, 0, 0, 0};
#pragma unroll
                    for (int s = 0; s < STEPS; ++s) {
                        u32x4_t v;
                        if (DT == 0) v = kv[s];
                        else if (DT == 2) v = fp4x8_to_bf16x8(kv[0][s], e8m0_scale(sc_b));
                        else v = e4m3x8_to_bf16x8(kv[s / 2][(s & 1) * 2], kv[s / 2][(s & 1) * 2 + 1]);
                        acc = mfma16_bf16(qb[s], as_bf16x8(v), acc);
                        if (DT != 1) aacc = mfma16_bf16(qa[s], as_bf16x8(v & 0x7fff7fffu), aacc);
                    }
                    if (DT == 1) {
                        // |q|.|k| bound: one e4m3 MFMA (K = 128) on the raw bytes with the sign bits cleared
                        typedef __attribute__((ext_vector_type(8))) int i32x8_t;
                        const u32x4_t k0 = kv[0] & 0x7f7f7f7fu;
                        const u32x4_t k1 = NV > 1 ? kv[NV > 1 ? 1 : 0] & 0x7f7f7f7fu : u32x4_t{0, 0, 0, 0};
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
                        const uint32_t key = f32_key(sc);
                        if constexpr (RING) {
                            lds_write_b32(lds_addr(&lsc[0][s - key0]), __float_as_uint(sc));
                            lds_add_u32(lds_addr(&lh[0][key >> 20]), 1u);
                        } else if (lrow < nlds) {
                            lsc[lrow][s - key0] = sc;
                            atomicAdd(&lh[lrow][key >> 20], 1u);
                        } else {
                            S[r * NcP + s] = sc;
                            atomicAdd(&hist[r * HIST_WORDS + (key >> 20)], 1u);
                        }
                        const float ej = e * 1.0009765625f + 1.1754943508222875e-38f;
                        dmax_loc = fmaxf(dmax_loc, ej + fabsf(sc) * 5.9604644775390625e-08f);
                    }
        };
        auto compute_batch = [&](int tt0, const u32x4_t (&cur)[U][NV], const uint32_t (&csc)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) compute_tile(key0 + ((tt0 + u) * 4 + wave) * 16, cur[u], csc[u]);
        };
        // The loads of the next batch are issued unconditionally (past the end they reread the current
        // batch, an L2 hit), so that no branch separates loads from their uses and the compiler's wait
        // counts stay exact: the next batch stays in flight while this one computes.
        __builtin_amdgcn_s_waitcnt(0);        // the per-row loads above have landed
        if constexpr (RING) {
            // Ring sweep.  Load j of a tile moves its rows j RPI .. j RPI + RPI - 1: lane l fetches 16 bytes of
            // row j RPI + l / CPR into slot bytes 1024 j + 16 l.  Chunk c of tile row kr sits at chunk
            // c ^ swz(kr) of its slot row, so the 16 lanes of one LDS read phase (16 keys, one chunk) fall on
            // distinct bank groups.  Tile t goes to slot t mod NS; it is read into registers once its loads have
            // landed (this wave's loads complete in order: the count of loads still in flight says which), and
            // the freed slot takes tile t + NS before tile t computes.  Tiles past the wave's last visible
            // tile reread that tile (an L2 hit), so every step issues the same loads and the counts stay exact.
            constexpr int CPR = RB / 16;          // 16-byte chunks per key row
            constexpr int RPI = 1024 / RB;        // key rows per load
            constexpr int NI = TILEB / 1024;      // loads per tile
            auto swz = [](int kr) { return (kr / (16 / CPR)) % CPR; };
            CSA_LDS uint8_t* wr = (CSA_LDS uint8_t*)ring + wave * (NS * TILEB);
            const int first = key0 + wave * 16;
            const int ntw = __builtin_amdgcn_readfirstlane(first < nvmax ? min(tiles, (nvmax - first + 63) / 64) : 0);
            const int lr_i = lane / CPR, lc = lane % CPR;
            auto issue = [&](int t, int slot) {
                const int tb = key0 + (min(t, ntw - 1) * 4 + wave) * 16;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int kr = i * RPI + lr_i;
                    const int krow = min(tb + kr, nvmax - 1);
                    size_t prow = (size_t)b * Nc + krow;
                    if constexpr (PAGED)
                        prow = ((size_t)lds_read_b32(lds_addr(&lpg[(krow >> pm.eshift) - pg0])) << pm.eshift) |
                               (size_t)(krow & ((1 << pm.eshift) - 1));
                    const char* src = (const char*)k_idx + prow * RB + 16 * (lc ^ swz(kr));
                    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                                     (CSA_LDS void*)(wr + slot * TILEB + i * 1024), 16, 0, 0);
                }
            };
            if (ntw > 0) {
#pragma unroll
                for (int j = 0; j < NS; ++j) issue(j, j);
                for (int t0 = 0; t0 < ntw; t0 += NS) {
#pragma unroll
                    for (int j = 0; j < NS; ++j) {
                        const int t = t0 + j;
                        if (t >= ntw) break;
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI * (NS - 1)) : "memory");   // tile t landed
                        const uint32_t sl = lds_addr(wr + j * TILEB + col * RB);
                        u32x4_t kv[NV];
                        lds_read_b128<NV>(kv, sl + 16 * ((grp + 0) ^ swz(col)), sl + 16 * ((grp + 4) ^ swz(col)),
                                          sl + 16 * ((grp + 8) ^ swz(col)), sl + 16 * ((grp + 12) ^ swz(col)));
                        issue(t + NS, j);
                        compute_tile(key0 + (t * 4 + wave) * 16, kv, 0u);
                    }
                }
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // the reread loads; the asm LDS ops
            }
        } else {
        u32x4_t ka[U][NV], kb[U][NV];
        uint32_t sa[U], sb[U];                // MXFP4 scale bytes of the batch's key rows (DT == 2)
        if (key0 + wave * 16 < nvmax) {
            load_batch(0, ka, sa);
            for (int tt0 = 0; tt0 < tiles; tt0 += 2 * U) {
                const bool more1 = tt0 + U < tiles && key0 + ((tt0 + U) * 4 + wave) * 16 < nvmax;
                load_batch(more1 ? tt0 + U : tt0, kb, sb);
                compute_batch(tt0, ka, sa);
                if (!more1) break;
                const bool more2 = tt0 + 2 * U < tiles && key0 + ((tt0 + 2 * U) * 4 + wave) * 16 < nvmax;
                load_batch(more2 ? tt0 + 2 * U : tt0 + U, ka, sa);
                compute_batch(tt0 + U, kb, sb);
                if (!more2) break;
            }
        }
        }
        if (writer) {
            if (lrow < nlds) atomicMax(&ldmax[lrow], __float_as_uint(dmax_loc));
            else atomicMax(&hist[r * HIST_WORDS + HW_DMAX], __float_as_uint(dmax_loc));
        }
        __syncthreads();
        for (int lr = 0; lr < nlds; ++lr) {
            const int nvr = row_visible(seq_lens, b, g * G + lr, Tq, L, pos0, m, Nc);
            const int nk = nvr > topk ? min(keys_per_wg, nvr - key0) : 0;     // (key0 and NcP are multiples of 4)
            float* Sr = S + ((size_t)b * Tq + g * G + lr) * NcP + key0;
            for (int i = threadIdx.x; i < nk / 4; i += TPB) ((f32x4_t*)Sr)[i] = ((const f32x4_t*)lsc[lr])[i];
            for (int i = (nk / 4) * 4 + threadIdx.x; i < nk; i += TPB) Sr[i] = lsc[lr][i];
        }
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
// threshold (lower edge of the bin holding the k-th largest S~, minus 2 Dmax) and
// writes its (index, S~) candidates in index order to its own region of the
// row's list; k_select then selects each row with one workgroup and emits the
// chosen indices in ascending order without sorting.
constexpr int STPB = 1024;
constexpr int CCHUNK = STPB * 16;    // entries per workgroup (16 waves x 16 groups of 64)
constexpr int BAND_LDS = 1024;       // band entries ranked in LDS (larger bands: 64-bit radix in HBM)
constexpr int CAND_LDS = 8192;       // candidates kept in LDS by k_select (more: read from HBM each pass)
constexpr int PF_MAX = 64;           // key rows near tau that k_select fetches into LDS ahead of the band
constexpr int SEL_TPB = 512;         // k_select threads (256 VGPRs each: the exact rescoring does not spill)

// k_collect: each workgroup filters CCHUNK entries of one row against the row's threshold (lower edge of
// the bin b1 holding the k-th largest S~, minus 2 Dmax) and writes its candidates (index, S~) in ascending
// index order at the start of its chunk's region of the row's list (chunk c at c * CCHUNK), with their count
// in the chunk table.  Workgroup 0 of the row publishes b1 and the count above it.
__global__ __launch_bounds__(STPB) void k_collect(const float* __restrict__ S, uint32_t* __restrict__ hist,
                                                  uint2* __restrict__ list, uint32_t* __restrict__ ctab, int Tq,
                                                  int Nc, int NcP, long long L, int m, long long pos0, int topk,
                                                  const long long* __restrict__ seq_lens)
{
    constexpr int GPW = CCHUNK / (STPB / 64) / 64;   // groups of 64 entries per wave
    __shared__ uint32_t lh[BINS1];
    __shared__ uint32_t scratch[STPB / 64], res[4], wcount[STPB / 64];
    const int r = blockIdx.y, t = r % Tq;
    const int nv = row_visible(seq_lens, r / Tq, t, Tq, L, pos0, m, Nc);
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
    const float dmax = __uint_as_float(H[HW_DMAX]);
    __syncthreads();
    find_bin_wide(lh, (uint32_t)topk, res, scratch);
    const uint32_t b1 = res[0];
    if (blockIdx.x == 0 && threadIdx.x == 0) { H[HW_B1] = b1; H[HW_A1] = res[1]; }   // for k_select
    const double thr = (double)key_f32(b1 << 20) - 2.0 * (double)dmax;
    unsigned long long mask[GPW];
    uint32_t cnt = 0;
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int sidx = s_w + gi * 64 + lane;
        mask[gi] = __ballot(sidx < nv && (double)v[gi] >= thr);
        cnt += __popcll(mask[gi]);
    }
    if (lane == 0) wcount[wave] = cnt;
    __syncthreads();
    uint32_t pos = blockIdx.x * CCHUNK;
    for (int w = 0; w < wave; ++w) pos += wcount[w];
    if (threadIdx.x == 0) {
        uint32_t tot = 0;
        for (int w = 0; w < STPB / 64; ++w) tot += wcount[w];
        ctab[(size_t)r * gridDim.x + blockIdx.x] = tot;
    }
    uint2* Lr = list + (size_t)r * NcP;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int sidx = s_w + gi * 64 + lane;
        if ((mask[gi] >> lane) & 1ull)
            Lr[pos + __popcll(mask[gi] & below)] = make_uint2((uint32_t)sidx, __float_as_uint(v[gi]));
        pos += __popcll(mask[gi]);
    }
}

// k_select: one 512-thread workgroup per row (see the header for the argument).  Candidates are addressed
// in ascending index order through the chunk counts ("sorted position" e).  The query row and its head
// weights are staged in LDS at the start, and the key rows of the candidates that can fall in the band
// are fetched into LDS as soon as tau is known to 12 + 12 bits, so that their loads overlap the rest of
// the search and the classification.
template <int DT, int DI, int HI>
__global__ __launch_bounds__(SEL_TPB) void k_select(
    uint32_t* __restrict__ hist, const uint2* __restrict__ list, const uint32_t* __restrict__ ctab,
    uint2* __restrict__ band_g, unsigned long long* __restrict__ bkey_g, uint8_t* __restrict__ flag_g,
    const void* __restrict__ q_idx, const float* __restrict__ w_idx, const void* __restrict__ k_idx,
    int Tq, int Nc, int NcP, long long L, int m, long long pos0, int topk,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out, float* __restrict__ score_out,
    const long long* __restrict__ seq_lens, PageMap pm, const uint8_t* __restrict__ q_scale,
    const uint8_t* __restrict__ k_scale)
{
    constexpr int RB = DT == 0 ? DI * 2 : (DT == 1 ? DI : DI / 2);     // bytes per key / query-head row
    constexpr int SB = DT == 2 ? DI / 32 : 0;                          // MXFP4 scale bytes per row
    // the query's HI rows (MXFP4: widened to exact bf16), its head weights, and the prefetched key rows
    // (raw bytes, MXFP4 scales after them); MXFP4 band keys are widened per wave into mxk
    __shared__ __attribute__((aligned(16))) uint8_t qs[DT == 2 ? HI * DI * 2 : HI * RB];
    __shared__ float ws[HI];
    __shared__ __attribute__((aligned(16))) uint8_t pk[PF_MAX][RB + SB];
    __shared__ __attribute__((aligned(16))) uint16_t mxk[DT == 2 ? SEL_TPB / 64 * DI : 2];
    __shared__ uint32_t pfe[PF_MAX], npf, ovf;
    __shared__ uint8_t pslot[CAND_LDS];               // prefetch slot of each candidate (0xff: none)
    __shared__ uint32_t lh[BINS2];
    __shared__ uint32_t scratch[SEL_TPB / 64], res[4], nband;
    __shared__ uint32_t cpre[2 * SEL_TPB + 1];
    __shared__ unsigned long long bkey[BAND_LDS];
    __shared__ uint32_t bpos[BAND_LDS];
    __shared__ uint2 bl[BAND_LDS];                    // band entries (index, position); more go to HBM
    __shared__ uint2 cl[CAND_LDS];                    // candidates in index order (when they fit)
    __shared__ uint8_t fl[CAND_LDS];                  // their flags
    const int r = blockIdx.x, b = r / Tq, t = r % Tq, tid = threadIdx.x;
    const int lane = lane_id(), wave = tid >> 6;
    const int nv = row_visible(seq_lens, b, t, Tq, L, pos0, m, Nc);
    int32_t* out = idx_out + (size_t)r * topk;
    if (nv <= topk) {                                 // every visible entry is selected (no score is formed)
        for (int i = tid; i < topk; i += SEL_TPB) {
            out[i] = i < nv ? i : -1;
            if (score_out) score_out[(size_t)r * topk + i] = __builtin_nanf("");
        }
        if (cnt_out && tid == 0) cnt_out[r] = nv;
        return;
    }
    const uint32_t* H = hist + (size_t)r * HIST_WORDS;
    const uint2* Lr = list + (size_t)r * NcP;
    uint8_t* F = flag_g + (size_t)r * NcP;
    const char* qrow = (const char*)q_idx + (size_t)r * HI * RB;
    const int NCH = NcP / CCHUNK;                     // <= 1024
    // chunk counts first (the loads below stay in flight behind them)
    const uint32_t c0 = 2 * tid < NCH ? ctab[(size_t)r * NCH + 2 * tid] : 0u;
    const uint32_t c1 = 2 * tid + 1 < NCH ? ctab[(size_t)r * NCH + 2 * tid + 1] : 0u;
    const uint32_t b1 = H[HW_B1], a1 = H[HW_A1];
    const float dmax = __uint_as_float(H[HW_DMAX]);
    // the query row and weights: loaded into registers now, written to LDS after the first barrier (a store
    // right behind its load would hold its wave, and with it the barrier, for a memory round trip)
    constexpr int QW = DT == 2 ? HI * RB / 4 : HI * RB / 16;   // code dwords (MXFP4) or 16-byte chunks
    static_assert(QW <= SEL_TPB, "one staging word per thread");
    u32x4_t qv = u32x4_t{0u, 0u, 0u, 0u};
    uint32_t qd = 0u, qsb = 0u;
    float wv = 0.f;
    if (tid < QW) {
        if constexpr (DT == 2) {
            qd = ((const uint32_t*)qrow)[tid];
            qsb = q_scale[((size_t)r * HI + (8 * tid) / DI) * (DI / 32) + ((8 * tid) % DI) / 32];
        } else {
            qv = ((const u32x4_t*)qrow)[tid];
        }
    }
    if (tid < HI) wv = w_idx[(size_t)r * HI + tid];
    // The first entries of every chunk's region are read before the counts are known (the regions start at
    // fixed offsets), so the candidates cost no second dependent round trip: chunk c's first `spec` entries
    // go to thread registers, spec = 2^ls <= 256 with NCH spec <= CAND_LDS / 2 (the reads cost time in
    // proportion to their bytes: a chunk holding more than spec candidates costs one more round trip).
    int ls = 8;
    while (ls > 0 && (NCH << ls) > CAND_LDS / 2) --ls;
    const uint32_t nspec = (uint32_t)NCH << ls;
    constexpr int SPR = CAND_LDS / 2 / SEL_TPB;      // speculative entries per thread
    uint2 sv[SPR];
#pragma unroll
    for (int u = 0; u < SPR; ++u) {
        const uint32_t i = tid + u * SEL_TPB;
        sv[u] = i < nspec ? Lr[(size_t)(i >> ls) * CCHUNK + (i & ((1u << ls) - 1))] : make_uint2(0u, 0u);
    }
    uint32_t total;
    {   // thread tid owns chunks 2 tid and 2 tid + 1
        if (tid == 0) { npf = 0; ovf = 0; }
        const uint32_t pre = block_scan(c0 + c1, scratch, &total);
        if (2 * tid < NCH) cpre[2 * tid] = pre;
        if (2 * tid + 1 < NCH) cpre[2 * tid + 1] = pre + c0;
        if (tid == 0) cpre[NCH] = total;
        if (max(c0, c1) > (1u << ls)) ovf = 1;       // a chunk holds more than its speculative part
        __syncthreads();
    }
    if (tid < QW) {                                   // (read only after later barriers)
        if constexpr (DT == 2)                        // eight elements of one 32-element block, widened exactly
            *(u32x4_t*)&qs[(8 * tid) * 2] = fp4x8_to_bf16x8(qd, e8m0_scale(qsb));
        else
            ((u32x4_t*)qs)[tid] = qv;
    }
    if (tid < HI) ws[tid] = wv;
    const uint32_t n = total;
    auto chunk_of = [&](uint32_t e) -> int {          // largest c with cpre[c] <= e: a non-empty chunk holding e
        int lo_c = 0, hi_c = NCH - 1;
        while (lo_c < hi_c) {
            const int mid = (lo_c + hi_c + 1) >> 1;
            if (cpre[mid] <= e) lo_c = mid; else hi_c = mid - 1;
        }
        return lo_c;
    };
    auto cand_g = [&](uint32_t e) -> uint2 {          // e-th candidate in index order, from HBM
        const int c = chunk_of(e);
        return Lr[(uint32_t)c * CCHUNK + (e - cpre[c])];
    };
    const bool inl = n <= (uint32_t)CAND_LDS;        // candidates and flags live in LDS (uniform)
    auto cand = [&](uint32_t e) -> uint2 { return inl ? cl[e] : cand_g(e); };
    auto fget = [&](uint32_t e) -> uint8_t { return inl ? fl[e] : F[e]; };
    auto fset = [&](uint32_t e, uint8_t f) { if (inl) fl[e] = f; else F[e] = f; };

    // 1. tau to 24 bits: the bin b1 (level 1, found by k_collect), then key bits 19..8 (level 2) over the
    //    candidates (every entry at or above b1 is one), built in the pass that puts them in LDS.
    for (int i = tid; i < BINS2; i += SEL_TPB) lh[i] = 0;
    __syncthreads();
    auto level2 = [&](uint32_t y) {
        const uint32_t key = f32_key(__uint_as_float(y));
        if ((key >> 20) == b1) atomicAdd(&lh[(key >> 8) & (BINS2 - 1)], 1u);
    };
    if (inl) {
        for (uint32_t e = tid; e < n; e += SEL_TPB) pslot[e] = 0xff;
#pragma unroll
        for (int u = 0; u < SPR; ++u) {
            const uint32_t i = tid + u * SEL_TPB, c = i >> ls, j = i & ((1u << ls) - 1);
            if (i < nspec && j < cpre[c + 1] - cpre[c]) { cl[cpre[c] + j] = sv[u]; level2(sv[u].y); }
        }
        if (ovf)                                      // the rest of the chunks that hold more
            for (uint32_t e = tid; e < n; e += SEL_TPB) {
                const int c = chunk_of(e);
                const uint32_t j = e - cpre[c];
                if (j >= (1u << ls)) {
                    const uint2 v = Lr[(uint32_t)c * CCHUNK + j];
                    cl[e] = v;
                    level2(v.y);
                }
            }
    } else {
        for (uint32_t e = tid; e < n; e += SEL_TPB) level2(cand_g(e).y);
    }
    __syncthreads();
    find_bin_wide(lh, (uint32_t)topk - a1, res, scratch);
    const uint32_t pfx = (b1 << 12) | res[0];
    // The k-th largest S~ lies in the level-2 bin [tlo, thi] and fewer than k entries lie above it, so the
    // classification of the header holds with tau replaced by tlo on the "out" side and by thi on the "in"
    // side: S~ < tlo - 2 Dmax is certainly out, S~ > thi + 2 Dmax certainly in.
    const double lo = (double)key_f32(pfx << 8) - 2.0 * (double)dmax;
    const double hi = (double)key_f32((pfx << 8) | 255u) + 2.0 * (double)dmax;
    // fetch the band's key rows into LDS now: their loads overlap the classification
    if (inl) {
        for (uint32_t e = tid; e < n; e += SEL_TPB) {
            const double x = (double)__uint_as_float(cl[e].y);
            if (x >= lo && x <= hi) {
                const uint32_t slot = atomicAdd(&npf, 1u);
                if (slot < (uint32_t)PF_MAX) { pfe[slot] = cl[e].x; pslot[e] = (uint8_t)slot; }
            }
        }
    }
    __syncthreads();
    // (held in registers: a barrier does not wait for loads, so they stay in flight until they are
    //  written to LDS after the classification)
    constexpr int CH = (RB + 15) / 16;                // 16-byte chunks per key row
    constexpr int HU = (PF_MAX * CH + SEL_TPB - 1) / SEL_TPB;
    const uint32_t np = min(npf, (uint32_t)PF_MAX);
    u32x4_t hv[HU];
    uint32_t hsc = 0;
#pragma unroll
    for (int u = 0; u < HU; ++u) {
        const uint32_t i = tid + u * SEL_TPB;
        if (i < np * CH) {
            const size_t krow = entry_row(pm, b, Nc, (int)pfe[i / CH]);
            hv[u] = *(const u32x4_t*)((const char*)k_idx + krow * RB + 16 * (i % CH));
        }
    }
    if (DT == 2 && tid < np) hsc = *(const uint32_t*)(k_scale + entry_row(pm, b, Nc, (int)pfe[tid]) * SB);

    // 2. classify: flag 1 = certainly in, 2 = band (listed with its position), 0 = out
    if (tid == 0) nband = 0;
    __syncthreads();
    uint2* Bg = band_g + (size_t)r * NcP;
    uint32_t my_in = 0;
    for (uint32_t e = tid; e < n; e += SEL_TPB) {
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
#pragma unroll
    for (int u = 0; u < HU; ++u) {
        const uint32_t i = tid + u * SEL_TPB;
        if (i < np * CH) *(u32x4_t*)&pk[i / CH][16 * (i % CH)] = hv[u];
    }
    if (DT == 2 && tid < np) *(uint32_t*)&pk[tid][RB] = hsc;
    __syncthreads();

    // 3. exact rescoring of the band (one wave per entry; the key row from LDS when it was prefetched);
    //    composite keys (exact score key, inverted index): larger composite = earlier in the order
    unsigned long long* Kg = bkey_g + (size_t)r * NcP;
    if (need > 0 && need < nb) {
        for (uint32_t i = wave; i < nb; i += SEL_TPB / 64) {
            const uint2 be = band(i);
            const uint32_t ps = inl ? pslot[be.y] : 0xffu;
            const size_t krow = ps == 0xffu ? entry_row(pm, b, Nc, (int)be.x) : 0;
            float sx;
            if constexpr (DT == 2) {
                uint16_t* kw = mxk + wave * DI;
                for (int e = lane; e < DI / 2; e += 64) {
                    const uint32_t sb = ps == 0xffu ? k_scale[krow * SB + (2 * e) / 32] : pk[ps][RB + (2 * e) / 32];
                    const float sc = e8m0_scale(sb);
                    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
                    const uint32_t w = ps == 0xffu ? (uint32_t)((const uint8_t*)k_idx)[krow * RB + e] : pk[ps][e];
                    *(uint32_t*)&kw[2 * e] =
                        __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                sx = wave_exact_score<0, DI, HI>(qs, ws, kw);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();   // the next band entry overwrites kw
            } else {
                const void* kp = ps == 0xffu ? (const void*)((const char*)k_idx + krow * RB) : (const void*)pk[ps];
                sx = wave_exact_score<DT, DI, HI>(qs, ws, kp);
            }
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
        for (uint32_t i = tid; i < nb; i += SEL_TPB) fset(band(i).y, 1);
    } else if (need > 0 && nb <= BAND_LDS) {
        for (uint32_t i = tid; i < nb; i += SEL_TPB) {          // rank by counting (keys are distinct)
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
            for (int i = tid; i < 256; i += SEL_TPB) lh[i] = 0;
            __syncthreads();
            for (uint32_t i = tid; i < nb; i += SEL_TPB) {
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
        for (uint32_t i = tid; i < nb; i += SEL_TPB)
            if (Kg[i] >= kp) fset(band(i).y, 1);
    }
    __threadfence_block();
    __syncthreads();

    // 5. compaction in index order: thread tid owns positions [tid*per, (tid+1)*per)
    const uint32_t per = (n + SEL_TPB - 1) / SEL_TPB;
    const uint32_t e0 = min(n, tid * per), e1 = min(n, e0 + per);
    uint32_t mine = 0;
    for (uint32_t e = e0; e < e1; ++e) mine += fget(e) == 1;
    uint32_t tot2;
    uint32_t o = block_scan(mine, scratch, &tot2);
    float* sout = score_out ? score_out + (size_t)r * topk : nullptr;
    for (uint32_t e = e0; e < e1; ++e)
        if (fget(e) == 1 && o < (uint32_t)topk) {
            const uint2 c = cand(e);
            if (sout) sout[o] = __uint_as_float(c.y);          // the approximate score it was ranked by
            out[o++] = (int32_t)c.x;
        }
    if (cnt_out && tid == 0) cnt_out[r] = topk;
    // The row's histogram words back to zero (read above, before the barriers in between; k_collect read
    // the bins in the previous launch), so that a workspace kept across calls needs no clearing launch.
    uint32_t* Hz = hist + (size_t)r * HIST_WORDS;
    for (int i = tid; i < HIST_WORDS; i += SEL_TPB) Hz[i] = 0u;
}

}  // namespace

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// hist [R][HIST_WORDS] (first, so that its place does not depend on Nc) | S~ [R][NcP] f32 | list [R][NcP]
// (index, S~) | chunk counts [R][NcP/CCHUNK] u32 | band [R][NcP] (index, position) | band keys [R][NcP] u64 |
// flags [R][NcP] u8.  k_select leaves every row's histogram words at zero.
static size_t decode_index_ws_bytes(int B, int Tq, int Nc) {
    const size_t R = (size_t)B * Tq;
    const size_t NcP = ((size_t)Nc + CCHUNK - 1) / CCHUNK * CCHUNK;
    return align256(R * HIST_WORDS * 4) + align256(R * NcP * 4) + align256(R * NcP * 8) +
           align256(R * (NcP / CCHUNK) * 4) + align256(R * NcP * 8) + align256(R * NcP * 8) + align256(R * NcP);
}

template <int DT, int DI, int HI>
static int launch_index(const void* q_idx, const float* w_idx, const void* k_idx, int B, int Tq, int Nc,
                        long long L, int m, long long pos0, int topk, int32_t* idx_out, int32_t* cnt_out,
                        float* score_out, const long long* seq_lens, const PageMap& pm, const uint8_t* q_scale,
                        const uint8_t* k_scale, void* ws, bool hist_zero, hipStream_t st) {
    const size_t R = (size_t)B * Tq;
    const int NcP = (Nc + CCHUNK - 1) / CCHUNK * CCHUNK;
    char* p = (char*)ws;
    uint32_t* hist = (uint32_t*)p;              p += align256(R * HIST_WORDS * 4);
    float* S = (float*)p;                       p += align256(R * (size_t)NcP * 4);
    uint2* list = (uint2*)p;                    p += align256(R * (size_t)NcP * 8);
    uint32_t* ctab = (uint32_t*)p;              p += align256(R * (size_t)(NcP / CCHUNK) * 4);
    uint2* band = (uint2*)p;                    p += align256(R * (size_t)NcP * 8);
    unsigned long long* bkey = (unsigned long long*)p; p += align256(R * (size_t)NcP * 8);
    uint8_t* flags = (uint8_t*)p;
    if (!hist_zero) {                           // (a workspace kept across calls is already clear)
        const size_t n = R * HIST_WORDS;
        const int blocks = (int)std::min<size_t>((n + 255) / 256, 2048);
        CSA_LAUNCH("k_fill", k_fill, dim3(blocks), dim3(256), 0, st, hist, n);
    }
    // keys per scoring workgroup (4 waves x tiles of 16): the largest of 4096/2048/1024 that still
    // gives >= 512 workgroups (two per CU), so the grid runs in one round without a tail
    int kpw = KPW_MAX;
    while (kpw > 1024 && (size_t)((Nc + kpw - 1) / kpw) * B < 512) kpw >>= 1;
    // the ring sweep: bf16 / e4m3 keys, one row per group with an LDS histogram (a single query row, or 16
    // heads per row), and paged keys only with the page table staged in LDS (pages of >= 2 entries)
    constexpr int HP = HI < 4 ? 4 : HI;
    const bool ring = DT != 2 && HP >= 8 && (Tq == 1 || HP == 16) && (!pm.table || pm.eshift > 0);
#define CSA_SCORE(PG, RG)                                                                                        \
    CSA_LAUNCH("k_score", (k_score<DT, DI, HI, PG, RG>), dim3((Nc + kpw - 1) / kpw, B), dim3(TPB), 0, st,       \
               q_idx, w_idx, k_idx, Tq, Nc, NcP, L, m, pos0, kpw, topk, S, hist, seq_lens, pm, q_scale, k_scale)
    bool launched = false;
    if constexpr (DT != 2 && HP >= 8) {
        if (ring) {
            if (pm.table) CSA_SCORE(true, true);
            else CSA_SCORE(false, true);
            launched = true;
        }
    }
    if (!launched) {
        if (pm.table) CSA_SCORE(true, false);
        else CSA_SCORE(false, false);
    }
#undef CSA_SCORE
    CSA_LAUNCH("k_collect", k_collect, dim3(NcP / CCHUNK, (unsigned)R), dim3(STPB), 0, st, S, hist, list, ctab, Tq,
               Nc, NcP, L, m, pos0, topk, seq_lens);
    CSA_LAUNCH("k_select", (k_select<DT, DI, HI>), dim3((unsigned)R), dim3(SEL_TPB), 0, st, hist, list, ctab, band,
               bkey, flags, q_idx, w_idx, k_idx, Tq, Nc, NcP, L, m, pos0, topk, idx_out, cnt_out, score_out, seq_lens, pm,
               q_scale, k_scale);
    return 0;
}

size_t index_topk_ws_bytes(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk, bool plain) {
    if (plain && prefill_index_applicable(dtype, HI, dI, B, Tq, Nc, topk))
        return prefill_index_ws_bytes(dtype, HI, dI, B, Tq, Nc);
    return decode_index_ws_bytes(B, Tq, Nc);
}

int index_topk_launch(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B, int Tq,
                      int HI, int dI, int Nc, long long L, int m, long long pos0, int topk,
                      int32_t* idx_out, int32_t* cnt_out, float* score_out, const CacheLayout& lay,
                      const uint8_t* q_scale, const uint8_t* k_scale, void* ws, hipStream_t st, bool hist_zero) {
    const PageMap pm = page_map(lay, m);
    if (!lay.seq_lens && !lay.table && prefill_index_applicable(dtype, HI, dI, B, Tq, Nc, topk))
        return prefill_index_launch(q_idx, w_idx, k_idx, dtype, HI, dI, B, Tq, Nc, L, m, pos0, topk, idx_out,
                                    cnt_out, score_out, q_scale, k_scale, ws, st);
#define CSA_IDX_CASE(DT, DI, HI_)                                                              \
    if (dtype == DT && dI == DI && HI == HI_)                                                  \
        return launch_index<DT, DI, HI_>(q_idx, w_idx, k_idx, B, Tq, Nc, L, m, pos0, topk,     \
                                         idx_out, cnt_out, score_out, lay.seq_lens, pm, q_scale, k_scale, ws, \
                                         hist_zero, st);
#define CSA_IDX_HI(DT, DI) CSA_IDX_CASE(DT, DI, 1) CSA_IDX_CASE(DT, DI, 2) CSA_IDX_CASE(DT, DI, 4) \
                           CSA_IDX_CASE(DT, DI, 8) CSA_IDX_CASE(DT, DI, 16)
    CSA_IDX_HI(0, 64) CSA_IDX_HI(0, 128) CSA_IDX_HI(1, 64) CSA_IDX_HI(1, 128) CSA_IDX_HI(2, 128)
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

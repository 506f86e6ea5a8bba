// attn.hip -- split-KV MQA attention on gfx950 MFMA (CSA core attention and HCA).
//
// Method: "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1:
// CSA's core attention is Multi-Query Attention over the top-k compressed
// entries plus an extra sliding-window branch of raw local tokens; HCA attends
// densely to every compressed entry ("DeepSeek V4 详解", section "第一刀").  One
// vector per entry is both key and value (one shared KV head); the window rows
// and the selected entries share one softmax.
//
// Kernel layout (one workgroup = 4 waves; a wave owns 16 query heads):
//   * the workgroup streams its slice of rows (a split) in tiles of 32 rows
//     through one LDS tile [32][D + 8] bf16 (row-major, padded);
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = key rows from LDS, B = the
//     wave's Q slice held in registers for the whole split;
//   * online softmax in the log2 domain, per head (a lane owns one head);
//   * O^T += V^T P^T: B = P taken straight from the S^T accumulators (a lane's
//     8 probabilities are exactly the MFMA k-slots it must supply), A = V^T read
//     from the same row-major LDS tile with ds_read_b64_tr_b16 (the gfx950
//     transpose read), so K and V share one tile and nothing is re-laid out;
//   * with one split the kernel normalises and writes bf16 output + LSE;
//     otherwise it writes unnormalised fp32 partials that k_combine merges in a
//     fixed split order (deterministic).
#include "common.h"
#include "kernels.h"

namespace {

using namespace csa;

constexpr int TPB = 256;
constexpr int TILE = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Rows {
    int mode;
    const uint16_t* kv;
    int N;
    long long L;
    int ratio;
    const int32_t* idx;
    int topk;
    const uint16_t* kv_raw;
    int Lr;
    long long raw0;
    int W;
};

__device__ __forceinline__ int dense_visible(long long p, long long L, int m, int N) {
    if (p >= L - 1) return N;
    long long v = (p + 1) / m;
    return v < N ? (int)v : N;
}

// Number of rows of query (b, t) and pointer to row r (nullptr = masked row).
struct RowSet {
    int n;
    int b, bt;
    long long w0;
    __device__ const uint16_t* row(const Rows& R, int r, int D) const {
        if (R.mode == 0) return R.kv + ((size_t)b * R.N + r) * D;
        if (r < R.topk) {
            const int j = R.idx[(size_t)bt * R.topk + r];
            return j >= 0 ? R.kv + ((size_t)b * R.N + j) * D : nullptr;
        }
        const long long u = w0 + (r - R.topk);
        return R.kv_raw + ((size_t)b * R.Lr + (size_t)(u - R.raw0)) * D;
    }
};

__device__ __forceinline__ RowSet make_rowset(const Rows& R, int bt, int Tq, long long pos0) {
    RowSet s;
    s.bt = bt;
    s.b = bt / Tq;
    const long long p = pos0 + bt % Tq;
    if (R.mode == 0) {
        s.n = dense_visible(p, R.L, R.ratio, R.N);
        s.w0 = 0;
    } else {
        s.w0 = p - R.W + 1 < 0 ? 0 : p - R.W + 1;
        s.n = R.topk + (R.W > 0 ? (int)(p - s.w0 + 1) : 0);
    }
    return s;
}

template <int D>
__global__ __launch_bounds__(TPB, 2) void k_attn(const uint16_t* __restrict__ q, Rows R, int Tq, int H,
                                                  long long pos0, float scale_log2, int nsplit, int rps,
                                                  float* __restrict__ part_o, float2* __restrict__ part_ml,
                                                  uint16_t* __restrict__ out, float* __restrict__ lse)
{
    constexpr int RS = D + 8;                 // padded LDS row (elements)
    constexpr int KSTEPS = D / 32;
    constexpr int DT = D / 16;
    constexpr int CHUNKS = TILE * D / 8;      // 16-byte chunks per tile
    __shared__ __attribute__((aligned(16))) uint16_t tile[TILE * RS];
    __shared__ float bias[TILE];

    const int split = blockIdx.x, hg = blockIdx.y, bt = blockIdx.z;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int h = hg * 64 + wave * 16 + col;
    const bool wave_active = hg * 64 + wave * 16 < H;

    const RowSet rs = make_rowset(R, bt, Tq, pos0);
    const int r_begin = split * rps;
    const int r_end = min(rs.n, r_begin + rps);

    // Q slice of this lane as B operands (K-slot permutation shared with the A loads)
    bf16x8_t qreg[KSTEPS];
    if (wave_active) {
        const uint16_t* qp = q + ((size_t)bt * H + h) * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qreg[s] = as_bf16x8(*(const u32x4_t*)(qp + 32 * s));
    }
    f32x4_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = f32x4_t{0, 0, 0, 0};
    float m_run = -INFINITY, l_run = 0.f;

    for (int rb = r_begin; rb < r_end; rb += TILE) {
        // ---- load 32 rows into LDS (masked / out-of-range rows are zero) ----
        for (int c = threadIdx.x; c < CHUNKS; c += TPB) {
            const int rr = c / (D / 8), cc = c % (D / 8);
            const int r = rb + rr;
            const uint16_t* src = r < r_end ? rs.row(R, r, D) : nullptr;
            u32x4_t v = u32x4_t{0, 0, 0, 0};
            if (src) v = *(const u32x4_t*)(src + cc * 8);
            *(u32x4_t*)(tile + rr * RS + cc * 8) = v;
            if (cc == 0) bias[rr] = src ? 0.0f : -INFINITY;
        }
        __syncthreads();
        if (wave_active) {
            // ---- S^T = K Q^T for two 16-row subtiles ----
            f32x4_t s0 = {0, 0, 0, 0}, s1 = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const bf16x8_t a0 = as_bf16x8(*(const u32x4_t*)(tile + col * RS + 32 * s + 8 * grp));
                const bf16x8_t a1 = as_bf16x8(*(const u32x4_t*)(tile + (16 + col) * RS + 32 * s + 8 * grp));
                s0 = mfma16_bf16(a0, qreg[s], s0);
                s1 = mfma16_bf16(a1, qreg[s], s1);
            }
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = s0[j] * scale_log2 + bias[4 * grp + j];
                x[4 + j] = s1[j] * scale_log2 + bias[16 + 4 * grp + j];
            }
            float mx = x[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            float alpha = 1.0f;
            float p[8];
            if (m_new == -INFINITY) {
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = 0.f;
            } else {
                alpha = exp2f(m_run - m_new);
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = exp2f(x[j] - m_new);
            }
            float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            ps += shfl_xor_f(ps, 16);
            ps += shfl_xor_f(ps, 32);
            l_run = l_run * alpha + ps;
            m_run = m_new;
            u32x4_t pw;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pw[j] = (uint32_t)f32_to_bf16(p[2 * j]) | ((uint32_t)f32_to_bf16(p[2 * j + 1]) << 16);
            const bf16x8_t pb = as_bf16x8(pw);
            // ---- O^T += V^T P^T via transposed LDS reads ----
            const int rsel = 4 * grp + (col >> 2);          // row this lane addresses
            const int csel = 4 * (col & 3);                 // 4-element column chunk it addresses
#pragma unroll
            for (int d = 0; d < DT; ++d) {
                acc[d] *= alpha;
                const CSA_LDS i16x4_t* p0 = (const CSA_LDS i16x4_t*)(
                    (CSA_LDS uint16_t*)tile + rsel * RS + d * 16 + csel);
                const CSA_LDS i16x4_t* p1 = (const CSA_LDS i16x4_t*)(
                    (CSA_LDS uint16_t*)tile + (16 + rsel) * RS + d * 16 + csel);
                const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<CSA_LDS i16x4_t*>(p0));
                const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<CSA_LDS i16x4_t*>(p1));
                u32x4_t aw;
                aw[0] = (uint32_t)(uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16);
                aw[1] = (uint32_t)(uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16);
                aw[2] = (uint32_t)(uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16);
                aw[3] = (uint32_t)(uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16);
                acc[d] = mfma16_bf16(as_bf16x8(aw), pb, acc[d]);
            }
        }
        __syncthreads();
    }
    if (!wave_active) return;
    // lane holds O^T[d*16 + 4*grp + j][h]
    if (nsplit == 1) {
        const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
        uint16_t* op = out + ((size_t)bt * H + h) * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
            uint2 v;
            v.x = (uint32_t)f32_to_bf16(acc[d][0] * inv) | ((uint32_t)f32_to_bf16(acc[d][1] * inv) << 16);
            v.y = (uint32_t)f32_to_bf16(acc[d][2] * inv) | ((uint32_t)f32_to_bf16(acc[d][3] * inv) << 16);
            *(uint2*)(op + d * 16) = v;
        }
        if (lse && grp == 0) lse[(size_t)bt * H + h] = l_run > 0.f ? (m_run + log2f(l_run)) * LN2 : -INFINITY;
    } else {
        const size_t slot = ((size_t)bt * nsplit + split) * H + h;
        float* op = part_o + slot * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < DT; ++d) *(f32x4_t*)(op + d * 16) = acc[d];
        if (grp == 0) part_ml[slot] = make_float2(m_run, l_run);
    }
}

// ---------------------------------------------------------------------------
// k_attn32 (D = 512, H % 32 == 0): a wave owns 32 heads (v_mfma_f32_32x32x16_bf16),
// so every K / V byte read from LDS feeds 32 heads, the balance point of the
// LDS-read and MFMA rates of a CU.  Waves work in pairs over the two halves of
// D: each computes the partial scores of its 256 dims, the pair exchanges them
// through LDS (summed in a fixed order, so both hold identical S), and each
// accumulates O only for its own half -- 128 accumulators and 64 Q registers
// per lane, two workgroups per CU.  The two pairs of a workgroup take the two
// halves of the split's rows and merge (m, l, O) in LDS at the end.  Tiles are
// unpadded and XOR-swizzled per 16-byte chunk (conflict-free row reads and
// transposed reads).  1D grid, XCD-aware: the H/32 head-group workgroups that
// read the same rows land on the same XCD (workgroup i runs on XCD i mod 8).
// ---------------------------------------------------------------------------
constexpr int HD = 256;   // d-half handled by one wave

// 16-byte chunk c of row r is stored at chunk c ^ f(r & 15), f(x) = 4 (x & 3) + (x >> 2): any 16
// consecutive rows at one chunk, and any 4 aligned rows x 4 aligned chunks (the footprint of a
// transposed read), fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz_chunk(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz(int r, int c) {   // element offset of (row, col) in a [32][256] tile
    return r * HD + (((c >> 3) ^ swz_chunk(r)) << 3) + (c & 7);
}

#ifndef CSA_ATTN32_WAVES_PER_EU
#define CSA_ATTN32_WAVES_PER_EU 1
#endif
// MODE 0: dense prefix (row r = entry r); MODE 1: selected entries then window rows.
template <int MODE>
__global__ __launch_bounds__(TPB, CSA_ATTN32_WAVES_PER_EU) void k_attn32(
    const uint16_t* __restrict__ q, Rows R, int Tq, int H, long long pos0, float scale_log2, int nunits, int nsplit,
    int rps, float* __restrict__ part_o, float2* __restrict__ part_ml, uint16_t* __restrict__ out,
    float* __restrict__ lse)
{
    constexpr int D = 512;
    constexpr int KS = HD / 16;               // 32x32x16 k-steps over a d-half
    constexpr int DT = HD / 32;               // 32-wide d tiles of a d-half
    __shared__ __attribute__((aligned(16))) uint16_t bufA[4 * TILE * HD];     // 64 KiB: tile buffer 0 of each wave
    __shared__ __attribute__((aligned(16))) uint16_t bufB[4 * TILE * HD];     // 64 KiB: tile buffer 1 of each wave
    __shared__ __attribute__((aligned(16))) float sx[4][16][64];              // 16 KiB

    const int HG = H / 32;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int hg = slot % HG, unit = (slot / HG) * 8 + xcd;
    if (unit >= nunits) return;                // padding workgroups (uniform exit)
    const int bt = unit / nsplit, split = unit % nsplit;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const int pr = w & 1, dh = w >> 1;         // row half, d half
    const int hl = lane & 31, g = lane >> 5;
    const int h = hg * 32 + hl;
    uint16_t* const ta = bufA + w * (TILE * HD);
    uint16_t* const tb = bufB + w * (TILE * HD);

    const int b = bt / Tq;
    const long long p = pos0 + bt % Tq;
    int nrows;
    long long w0 = 0;
    if (MODE == 0) {
        nrows = dense_visible(p, R.L, R.ratio, R.N);
    } else {
        w0 = p - R.W + 1 < 0 ? 0 : p - R.W + 1;
        nrows = R.topk + (R.W > 0 ? (int)(p - w0 + 1) : 0);
    }
    const int s_begin = split * rps;
    const int s_end = min(nrows, s_begin + rps);
    const int per_pair = rps / 2;              // multiple of TILE
    const int r_begin = s_begin + pr * per_pair;
    const int r_end = min(s_end, r_begin + per_pair);
    const int ntiles = per_pair / TILE;        // same count for every wave (barriers inside)

    const uint16_t* kvb = R.kv ? R.kv + (size_t)b * R.N * D : nullptr;
    const uint16_t* rawb = MODE == 1 && R.kv_raw ? R.kv_raw + (size_t)b * R.Lr * D : nullptr;
    const uint16_t* fallback = kvb ? kvb : rawb;          // a valid row for masked slots

    // Row code of row r: >= 0 entry index in kv, <= -2 raw row (-code-2), -1 masked.
    auto row_code = [&](int r) -> int {
        if (r >= r_end) return -1;
        if constexpr (MODE == 0) {
            return r;
        } else {
            if (r < R.topk) return R.idx[(size_t)bt * R.topk + r];    // (< 0 -> masked)
            return -2 - (int)(w0 + (r - R.topk) - R.raw0);
        }
    };
    auto row_ptr = [&](int c) -> const uint16_t* {
        if (c >= 0) return kvb + (size_t)c * D;
        if constexpr (MODE == 0) {
            return nullptr;
        } else {
            if (c == -1) return nullptr;
            return rawb + (size_t)(-c - 2) * D;
        }
    };

    bf16x8_t qreg[KS];
    {
        const uint16_t* qp = q + ((size_t)bt * H + h) * D + dh * HD + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) qreg[s] = as_bf16x8(*(const u32x4_t*)(qp + 16 * s));
    }
    f32x16_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int b16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 4 * (b16 >> 1) + (j16 >> 2);
    const int tr_col = 16 * (b16 & 1) + 4 * (j16 & 3);
    const int rsub = lane >> 5, pch = lane & 31;

    // codes of the lane's 16 rows (2 i + rsub) of tile it
    int code[TILE / 2];
    auto fetch_codes = [&](int it) {
        if constexpr (MODE == 0) {
            code[0] = r_begin + it * TILE;                            // dense: the tile's first row
        } else {
#pragma unroll
            for (int i = 0; i < TILE / 2; ++i) code[i] = row_code(r_begin + it * TILE + 2 * i + rsub);
        }
    };
    // Direct global->LDS loads (16 B per lane; lane l lands at base + 16 l): one
    // instruction moves rows (2i, 2i+1) of this d-half; the XOR swizzle goes on
    // the source address.  Masked rows read a valid row and are excluded by the
    // returned validity mask.  Issues no other memory operation.
    auto issue_tile = [&](uint16_t* buf) -> uint32_t {
        if constexpr (MODE == 0) {
            // dense rows are consecutive entries starting at code[0] (wave-uniform)
            const int first = code[0];
            const int nval = max(0, min(TILE, r_end - first));
            const uint16_t* base = kvb + (size_t)(nval > 0 ? first : 0) * D + dh * HD;
#pragma unroll
            for (int i = 0; i < TILE / 2; ++i) {
                const int row = 2 * i + rsub;
                const int rr = row < nval ? row : 0;                  // past the end: reread row 0 (masked)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(base + (size_t)rr * D + ((pch ^ swz_chunk(row)) << 3)),
                    (CSA_LDS void*)(buf + i * 2 * HD), 16, 0, 0);
            }
            return nval >= 32 ? 0xffffffffu : ((1u << nval) - 1u);
        }
        uint32_t vm = 0;
#pragma unroll
        for (int i = 0; i < TILE / 2; ++i) {
            const int row = 2 * i + rsub;
            const uint16_t* src = row_ptr(code[i]);
            const unsigned long long bal = __ballot(src != nullptr);
            vm |= (uint32_t)(bal & 1ull) << (2 * i);
            vm |= (uint32_t)((bal >> 32) & 1ull) << (2 * i + 1);
            const uint16_t* s8 = (src ? src : fallback) + dh * HD + ((pch ^ swz_chunk(row)) << 3);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)s8,
                                             (CSA_LDS void*)(buf + i * 2 * HD), 16, 0, 0);
        }
        return vm;
    };

    // Compute on one tile; the loads of the next tile (into the other LDS object) stay in flight.
    auto compute_tile = [&](const uint16_t* tile, uint32_t vmask) {
        const CSA_LDS uint16_t* tl = (const CSA_LDS uint16_t*)tile;
        // ---- partial S^T[32 rows][32 heads] over this d-half ----
        f32x16_t sacc, sacc1;                    // two chains: even / odd k-steps
#pragma unroll
        for (int j = 0; j < 16; ++j) { sacc[j] = 0.f; sacc1[j] = 0.f; }
#pragma unroll
        for (int s = 0; s < KS; s += 2) {
            const bf16x8_t a0 = as_bf16x8(*(const u32x4_t*)(tile + swz(hl, 16 * s + 8 * g)));
            const bf16x8_t a1 = as_bf16x8(*(const u32x4_t*)(tile + swz(hl, 16 * (s + 1) + 8 * g)));
            sacc = mfma32_bf16(a0, qreg[s], sacc);
            sacc1 = mfma32_bf16(a1, qreg[s + 1], sacc1);
        }
        sacc += sacc1;
        // ---- exchange with the other d-half of the pair; S = S_dh0 + S_dh1 in both ----
#pragma unroll
        for (int j = 0; j < 16; ++j) sx[w][j][lane] = sacc[j];
        __syncthreads();
        float x[16];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float o = sx[w ^ 2][j][lane];
            const float sv = dh == 0 ? sacc[j] + o : o + sacc[j];
            const int row = 8 * (j >> 2) + 4 * g + (j & 3);
            x[j] = ((vmask >> row) & 1u) ? sv * scale_log2 : -INFINITY;
            mx = fmaxf(mx, x[j]);
        }
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        // rescale only when the running max grows by more than 2^8 (exact: the
        // reference point of the exponentials is free; p stays <= 256)
        if (mx > m_run + 8.0f) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - mx);   // 0 on the first tile
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < DT; ++d) acc[d] *= alpha;
            m_run = mx;
        }
        float pv[16], ps = 0.f;
        if (m_run == -INFINITY) {                // nothing valid yet: all probabilities are 0
#pragma unroll
            for (int j = 0; j < 16; ++j) pv[j] = 0.f;
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                pv[j] = __builtin_amdgcn_exp2f(x[j] - m_run);   // argument <= 8; -inf -> 0
                ps += pv[j];
            }
        }
        ps += shfl_xor_f(ps, 32);
        l_run += ps;
        u32x4_t pw0, pw1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pw0[j] = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
            pw1[j] = pack_bf16x2(pv[8 + 2 * j], pv[8 + 2 * j + 1]);
        }
        const bf16x8_t pb0 = as_bf16x8(pw0), pb1 = as_bf16x8(pw1);
        // ---- O^T[d-half][h] += V^T P^T (rows in two k-steps of 16) ----
        typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
            const int c0 = d * 32 + tr_col;
            const u32x2_t w0r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4_t*)(tl + swz(tr_row, c0))));
            const u32x2_t w1r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4_t*)(tl + swz(8 + tr_row, c0))));
            const u32x2_t w2r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4_t*)(tl + swz(16 + tr_row, c0))));
            const u32x2_t w3r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4_t*)(tl + swz(24 + tr_row, c0))));
            acc[d] = mfma32_bf16(as_bf16x8(u32x4_t{w0r[0], w0r[1], w1r[0], w1r[1]}), pb0, acc[d]);
            acc[d] = mfma32_bf16(as_bf16x8(u32x4_t{w2r[0], w2r[1], w3r[0], w3r[1]}), pb1, acc[d]);
        }
    };

    uint32_t vm_a = 0, vm_b = 0;
    if (ntiles > 0) {
        fetch_codes(0);
        vm_a = issue_tile(ta);
        if (ntiles > 1) fetch_codes(1);
    }
    for (int it = 0; it < ntiles; it += 2) {
        __builtin_amdgcn_s_waitcnt(0);           // tile it (buffer A) and the codes of tile it+1 have landed
        __builtin_amdgcn_wave_barrier();
        if (it + 1 < ntiles) {
            vm_b = issue_tile(tb);
            if (it + 2 < ntiles) fetch_codes(it + 2);
        }
        compute_tile(ta, vm_a);
        __syncthreads();                         // sx reuse; buffer A is reloaded next
        if (it + 1 < ntiles) {                   // workgroup-uniform
            __builtin_amdgcn_s_waitcnt(0);       // tile it+1 (buffer B) and the codes of tile it+2
            __builtin_amdgcn_wave_barrier();
            if (it + 2 < ntiles) {
                vm_a = issue_tile(ta);
                if (it + 3 < ntiles) fetch_codes(it + 3);
            }
            compute_tile(tb, vm_b);
            __syncthreads();
        }
    }

    // ---- merge the two row halves: wave (pr=0, dh) += wave (pr=1, dh) ----
    float* ob = (float*)bufA;                  // [2][DT*16][64] floats = 64 KiB
    if (pr == 1) {
        float* dst = ob + (size_t)dh * DT * 16 * 64;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int j = 0; j < 16; ++j) dst[(d * 16 + j) * 64 + lane] = acc[d][j];
        if (g == 0) { sx[dh][0][hl] = m_run; sx[dh][1][hl] = l_run; }
    }
    __syncthreads();
    if (pr == 1) return;
    {
        const float* src = ob + (size_t)dh * DT * 16 * 64;
        const float mo = sx[dh][0][hl], lo = sx[dh][1][hl];
        const float M = fmaxf(m_run, mo);
        const float fa = M == -INFINITY ? 0.f : exp2f(m_run - M);
        const float fb = M == -INFINITY ? 0.f : exp2f(mo - M);
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[d][j] = acc[d][j] * fa + src[(d * 16 + j) * 64 + lane] * fb;
        l_run = l_run * fa + lo * fb;
        m_run = M;
    }
    // lane holds O^T[dh*256 + d*32 + 8 (j/4) + 4 g + j%4][h]
    if (nsplit == 1) {
        const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
        uint16_t* op = out + ((size_t)bt * H + h) * D + dh * HD + 4 * g;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint2 v;
                v.x = pack_bf16x2(acc[d][4 * q4] * inv, acc[d][4 * q4 + 1] * inv);
                v.y = pack_bf16x2(acc[d][4 * q4 + 2] * inv, acc[d][4 * q4 + 3] * inv);
                *(uint2*)(op + d * 32 + 8 * q4) = v;
            }
        if (lse && g == 0 && dh == 0) lse[(size_t)bt * H + h] = l_run > 0.f ? (m_run + log2f(l_run)) * LN2 : -INFINITY;
    } else {
        const size_t sl = ((size_t)bt * nsplit + split) * H + h;
        float* op = part_o + sl * D + dh * HD + 4 * g;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(f32x4_t*)(op + d * 32 + 8 * q4) = f32x4_t{acc[d][4 * q4], acc[d][4 * q4 + 1], acc[d][4 * q4 + 2],
                                                            acc[d][4 * q4 + 3]};
        if (g == 0 && dh == 0) part_ml[sl] = make_float2(m_run, l_run);
    }
}

// Merge split partials in split order: out = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
template <int D>
__global__ __launch_bounds__(D / 4) void k_combine(const float* __restrict__ part_o, const float2* __restrict__ part_ml,
                                                   int H, int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse)
{
    const int h = blockIdx.x, bt = blockIdx.y, d = threadIdx.x * 4;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((size_t)bt * nsplit + s) * H + h].x);
    float l = 0.f;
    f32x4_t o = {0, 0, 0, 0};
    if (M != -INFINITY) {
        for (int s = 0; s < nsplit; ++s) {
            const size_t slot = ((size_t)bt * nsplit + s) * H + h;
            const float2 ml = part_ml[slot];
            const float f = exp2f(ml.x - M);      // 0 for empty splits (m = -inf)
            l += f * ml.y;
            o += f * *(const f32x4_t*)(part_o + slot * D + d);
        }
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    uint2 v;
    v.x = (uint32_t)f32_to_bf16(o[0] * inv) | ((uint32_t)f32_to_bf16(o[1] * inv) << 16);
    v.y = (uint32_t)f32_to_bf16(o[2] * inv) | ((uint32_t)f32_to_bf16(o[3] * inv) << 16);
    *(uint2*)(out + ((size_t)bt * H + h) * D + d) = v;
    if (lse && threadIdx.x == 0) lse[(size_t)bt * H + h] = l > 0.f ? (M + log2f(l)) * LN2 : -INFINITY;
}

}  // namespace

namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split counts.  k_attn (16 heads per wave): enough workgroups to cover the
// chip twice, splits of >= 64 rows.  k_attn32 (32 heads per wave, one
// workgroups per CU): about one workgroup per CU, whole 32-row tiles per wave pair.
static bool use32(int D, int H) { return D == 512 && H % 32 == 0; }

static void choose_split(int BT, int H, int D, int max_rows, int* nsplit, int* rps) {
    if (max_rows <= 0) { *nsplit = 1; *rps = 128; return; }
    if (use32(D, H)) {
        const int HG = H / 32;
        int ns = std::max(1, 256 / (BT * HG));
        int r = (max_rows + ns - 1) / ns;
        r = (r + 2 * TILE - 1) / (2 * TILE) * (2 * TILE);
        *rps = r;
        *nsplit = (max_rows + r - 1) / r;
        return;
    }
    const int HG = (H + 63) / 64;
    const int target = 512;
    int ns = (target + BT * HG - 1) / (BT * HG);
    const int cap = std::max(1, (max_rows + 63) / 64);
    ns = std::min(std::max(ns, 1), cap);
    int r = (max_rows + ns - 1) / ns;
    r = (r + TILE - 1) / TILE * TILE;
    *rps = r;
    *nsplit = (max_rows + r - 1) / r;
}

size_t attn_ws_bytes(int B, int Tq, int H, int D, int max_rows) {
    const int BT = B * Tq;
    int ns, rps;
    choose_split(BT, H, D, max_rows, &ns, &rps);
    if (ns == 1) return 0;
    return align256((size_t)BT * ns * H * D * 4) + align256((size_t)BT * ns * H * 8);
}

int attn_launch(const void* q, const AttnRows& a, int B, int Tq, int H, int D, long long pos0, float scale,
                void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st, const char* tag) {
    Rows R;
    R.mode = a.mode;
    R.kv = (const uint16_t*)a.kv;
    R.N = a.N;
    R.L = a.L;
    R.ratio = a.ratio;
    R.idx = a.idx;
    R.topk = a.topk;
    R.kv_raw = (const uint16_t*)a.kv_raw;
    R.Lr = a.Lr;
    R.raw0 = a.raw0;
    R.W = a.W;
    const int BT = B * Tq;
    const int max_rows = a.mode == 0 ? a.N : a.topk + a.W;
    int ns, rps;
    choose_split(BT, H, D, max_rows, &ns, &rps);
    float* part_o = nullptr;
    float2* part_ml = nullptr;
    if (ns > 1) {
        part_o = (float*)ws;
        part_ml = (float2*)((char*)ws + align256((size_t)BT * ns * H * D * 4));
    }
    const float sl2 = scale * LOG2E;
    if (use32(D, H)) {
        const int nunits = BT * ns, HG = H / 32;
        const int nblk = (nunits + 7) / 8 * 8 * HG;
        if (a.mode == 0)
            CSA_LAUNCH(tag, k_attn32<0>, dim3(nblk), dim3(TPB), 0, st, (const uint16_t*)q, R, Tq, H, pos0, sl2,
                       nunits, ns, rps, part_o, part_ml, (uint16_t*)out, lse);
        else
            CSA_LAUNCH(tag, k_attn32<1>, dim3(nblk), dim3(TPB), 0, st, (const uint16_t*)q, R, Tq, H, pos0, sl2,
                       nunits, ns, rps, part_o, part_ml, (uint16_t*)out, lse);
        if (ns > 1)
            CSA_LAUNCH("k_combine", k_combine<512>, dim3(H, BT), dim3(128), 0, st, part_o, part_ml, H, ns,
                       (uint16_t*)out, lse);
        return 0;
    }
    dim3 grid(ns, (H + 63) / 64, BT);
    if (D == 512) {
        CSA_LAUNCH(tag, k_attn<512>, grid, dim3(TPB), 0, st, (const uint16_t*)q, R, Tq, H, pos0, sl2, ns, rps,
                   part_o, part_ml, (uint16_t*)out, lse);
        if (ns > 1)
            CSA_LAUNCH("k_combine", k_combine<512>, dim3(H, BT), dim3(128), 0, st, part_o, part_ml, H, ns,
                       (uint16_t*)out, lse);
    } else if (D == 128) {
        CSA_LAUNCH(tag, k_attn<128>, grid, dim3(TPB), 0, st, (const uint16_t*)q, R, Tq, H, pos0, sl2, ns, rps,
                   part_o, part_ml, (uint16_t*)out, lse);
        if (ns > 1)
            CSA_LAUNCH("k_combine", k_combine<128>, dim3(H, BT), dim3(32), 0, st, part_o, part_ml, H, ns,
                       (uint16_t*)out, lse);
    } else {
        return fail(6, "attention: D = %d unsupported", D);
    }
    return 0;
}

}  // namespace csa_host

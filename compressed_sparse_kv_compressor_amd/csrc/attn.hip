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
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "attn_common.h"

namespace {

using namespace csa;
using namespace csa_attn;

constexpr int TPB = 256;
// Number of rows of query (b, t) and the byte address of row r's key (value = false) or value (value = true)
// data (nullptr = masked row); `ent` is set for compressed entries (which may be FP8 rows), cleared for raw
// window rows (always bf16).  Entries go through the page map; keys and values are one row unless separate
// value arrays are given.
struct RowSet {
    int n;
    int b, bt;
    long long w0, raw0, p;
    __device__ const char* row(const Rows& R, int r, int D, bool value, bool& ent) const {
        const size_t eb = R.kv_fp8 ? (size_t)D + 80 : (size_t)D * 2;
        const char* base = (const char*)(value && R.v ? R.v : R.kv);
        ent = true;
        if (R.mode == 0) return base + entry_row(R.pm, b, R.N, r) * eb;
        if (r < R.topk) {
            const int j = R.idx[(size_t)bt * R.topk + r];
            return j >= 0 ? base + entry_row(R.pm, b, R.N, j) * eb : nullptr;
        }
        ent = false;
        const long long u = w0 + (r - R.topk);
        const uint16_t* raw = value && R.v_raw ? R.v_raw : R.kv_raw;
        return (const char*)(raw + ((size_t)b * R.Lr + (size_t)(u - raw0)) * D);
    }
};

// 16-byte chunk cc (dimensions 8 cc .. 8 cc + 7) of a row as bf16: from a bf16 row, or from an FP8 row (codes of
// the non-RoPE dimensions times their group's power-of-two scale, exact in bf16; the RoPE dimensions stored
// as bf16 after the codes).
template <int D>
__device__ __forceinline__ u32x4_t row_chunk(const char* p, int cc, bool fp8) {
    if (!fp8) return *(const u32x4_t*)(p + cc * 16);
    constexpr int NOPE = D - 64;
    if (cc >= NOPE / 8) return *(const u32x4_t*)(p + NOPE + (cc - NOPE / 8) * 16);
    const uint2 w = *(const uint2*)(p + cc * 8);
    const uint32_t s = (uint32_t)(uint8_t)p[D + 64 + (cc * 8) / 64];
    const float scale = __uint_as_float((s < 1u ? 1u : s) << 23);       // 2^(s - 127)
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
#define CSA_FP8_PAIR(X, HI) __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(X, scale, HI))
    return u32x4_t{CSA_FP8_PAIR(w.x, false), CSA_FP8_PAIR(w.x, true), CSA_FP8_PAIR(w.y, false),
                   CSA_FP8_PAIR(w.y, true)};
#undef CSA_FP8_PAIR
}

__device__ __forceinline__ RowSet make_rowset(const Rows& R, int bt, int Tq, long long pos0) {
    RowSet s;
    s.bt = bt;
    s.b = bt / Tq;
    int nd;
    const long long p = row_geo(R, s.b, bt % Tq, Tq, pos0, s.raw0, nd);
    s.p = p;
    if (R.mode == 0) {
        s.n = nd;
        s.w0 = 0;
    } else {
        s.w0 = p - R.W + 1 < 0 ? 0 : p - R.W + 1;
        s.n = R.topk + (R.W > 0 ? (int)(p - s.w0 + 1) : 0);
    }
    return s;
}

template <int D, bool SEPV, bool FP8, bool ROPE>
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
    __shared__ __attribute__((aligned(16))) uint16_t vtile_[SEPV ? TILE * RS : 8];   // separate values
    __shared__ float bias[TILE];
    uint16_t* vtile = SEPV ? vtile_ : tile;

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
        if constexpr (ROPE) {                   // fused rotary embedding of the last 64 dims, at +p
#pragma unroll
            for (int s = KSTEPS - ROPE_FUSED_RD / 32; s < KSTEPS; ++s)
                qreg[s] = as_bf16x8(rope8(__builtin_bit_cast(u32x4_t, qreg[s]), 32 * s + 8 * grp, D, R, (double)rs.p));
        }
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
            bool ent = false;
            const char* src = r < r_end ? rs.row(R, r, D, false, ent) : nullptr;
            u32x4_t v = u32x4_t{0, 0, 0, 0};
            if (src) v = row_chunk<D>(src, cc, FP8 && ent);
            *(u32x4_t*)(tile + rr * RS + cc * 8) = v;
            if constexpr (SEPV) {
                const char* vsrc = src ? rs.row(R, r, D, true, ent) : nullptr;
                u32x4_t vv = u32x4_t{0, 0, 0, 0};
                if (vsrc) vv = row_chunk<D>(vsrc, cc, FP8 && ent);
                *(u32x4_t*)(vtile + rr * RS + cc * 8) = vv;
            }
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
                    (CSA_LDS uint16_t*)vtile + rsel * RS + d * 16 + csel);
                const CSA_LDS i16x4_t* p1 = (const CSA_LDS i16x4_t*)(
                    (CSA_LDS uint16_t*)vtile + (16 + rsel) * RS + d * 16 + csel);
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
        float lse_v;
        const float inv = sink_norm(m_run, l_run, sink_log2(R.sink, h), lse_v);
        if constexpr (ROPE) {                   // the output's last 64 dims turn back by -p
#pragma unroll
            for (int d = DT - ROPE_FUSED_RD / 16; d < DT; ++d) {
                CSA_ROPE_PAIR(acc[d], 0, 1, d * 16 + 4 * grp, D, R, -(double)rs.p)
                CSA_ROPE_PAIR(acc[d], 2, 3, d * 16 + 4 * grp + 2, D, R, -(double)rs.p)
            }
        }
        uint16_t* op = out + ((size_t)bt * H + h) * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
            uint2 v;
            v.x = (uint32_t)f32_to_bf16(acc[d][0] * inv) | ((uint32_t)f32_to_bf16(acc[d][1] * inv) << 16);
            v.y = (uint32_t)f32_to_bf16(acc[d][2] * inv) | ((uint32_t)f32_to_bf16(acc[d][3] * inv) << 16);
            *(uint2*)(op + d * 16) = v;
        }
        if (lse && grp == 0) lse[(size_t)bt * H + h] = lse_v;
    } else {
        const size_t slot = ((size_t)bt * nsplit + split) * H + h;
        float* op = part_o + slot * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < DT; ++d) *(f32x4_t*)(op + d * 16) = acc[d];
        if (grp == 0) part_ml[slot] = make_float2(m_run, l_run);
    }
}

// ---------------------------------------------------------------------------
// k_attn64 (D = 512, H % 32 == 0): one workgroup = 4 waves = 64 heads (two head
// groups of 32) x the two halves of D.  A wave owns 32 heads of one d-half
// (v_mfma_f32_32x32x16_bf16: every K / V byte read from LDS feeds 32 heads);
// the two head groups share each K tile in LDS, so a tile is fetched once per
// 64 heads.  The two d-half waves of a head group compute partial scores over
// their 256 dims and exchange them through LDS (summed in a fixed order, so
// both hold identical S); each accumulates O only for its own d-half (128
// accumulators and 64 Q registers per lane).  The split's rows stream through
// three tile buffers filled by direct global->LDS loads, so a tile's loads have
// a whole tile of compute to land.  Per tile the waves run one software-
// pipelined step: the softmax of tile t overlaps the QK MFMAs of tile t+1,
// then the PV MFMAs of tile t, then the score exchange (the one barrier).
// Tiles are unpadded and XOR-swizzled per 16-byte chunk (conflict-free row
// reads and transposed reads).  1D grid, XCD-aware: the head-pair workgroups
// that read the same rows land on the same XCD (workgroup i runs on XCD i mod 8).
// FP8 entry rows (592 bytes: e4m3 codes of dims 0..447, bf16 RoPE dims 448..511,
// one power-of-two scale per 64-dim group): each d-half slot (512 bytes) takes the
// bytes its half needs at its top (half 0: codes 0..255 + scales; half 1: codes
// 256..447, the RoPE dims, the scales) and the wave that loaded it widens it in
// place to the bf16 layout above before the tile's barrier; raw window rows stay
// bf16.
// ---------------------------------------------------------------------------
constexpr int HD = 256;   // d-half handled by one wave

constexpr int ATT64_QK_AHEAD = 4;  // K-operand LDS reads in flight ahead of the QK MFMAs
constexpr int ATT64_PV_AHEAD = 2;  // d-tiles of V reads in flight ahead of the PV MFMAs
constexpr int ATT_TILES = 3;      // tile buffers; a split's tile count is a multiple of this

// MODE 0: dense prefix (row r = entry r); MODE 1: selected entries then window rows.  Every array must
// be within reach of 32-bit byte offsets: tiles are moved by buffer loads only, which keeps the LDS wait
// counting exact in the main loop (larger arrays run the generic kernel).  PAGED: the selected entries go
// through the page map (a compile-time switch: the page-map code in the tile loop cost the batch-major
// kernel half its rate).
typedef float SxArr[4][4][64][4];         // score exchange [wave][j/4][lane][j%4] (one parity)

template <int MODE, bool PAGED, bool ROPE, bool FP8>
__device__ __forceinline__ void attn64_body(
    int bid, uint16_t* bufA, uint16_t* bufB, uint16_t* bufC, SxArr* sx, float (*amx)[32],
    const uint16_t* __restrict__ q, const Rows& R, int Tq, int H, long long pos0, float scale_log2, int nunits,
    int nsplit, int rps, float* __restrict__ part_o, float2* __restrict__ part_ml, uint16_t* __restrict__ out,
    float* __restrict__ lse)
{
    constexpr int D = 512;
    constexpr int KS = HD / 16;               // 32x32x16 k-steps over a d-half
    constexpr int DT = HD / 32;               // 32-wide d tiles of a d-half
    constexpr int HALF_B = TILE * HD * 2;     // bytes of one d-half of a tile (16 KiB)

    const int HP = (H + 63) / 64;
    // XCD-aware order: workgroup i runs on XCD i mod 8, and XCD x takes the contiguous range [x per, (x + 1) per)
    // of the (unit, head pair) blocks, so the head pairs of a unit (the same rows) and the splits of a query
    // (whose partials the merge reads) share an XCD and its L2
    const int per = (nunits * HP + 7) / 8;
    const int vb = (bid & 7) * per + (bid >> 3);
    if (vb >= nunits * HP) return;             // padding workgroups (uniform exit)
    const int hp = vb % HP, unit = vb / HP;
    const int bt = unit / nsplit, split = unit % nsplit;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // w: wave-uniform
    const int hgl = w & 1, dh = w >> 1;        // head group within the pair, d half
    const int hl = lane & 31, g = lane >> 5;
    const int hbase = hp * 64 + hgl * 32;      // first head of this wave
    const bool hv = hbase < H;                 // the wave's heads exist (H % 64 == 32: the last pair is half)
    const int h = hbase + hl;

    const int b = bt / Tq;
    long long raw0;
    int ndense;
    const long long p = row_geo(R, b, bt % Tq, Tq, pos0, raw0, ndense);
    // MODE 1 row space: [0, topk) selected entries, [topk, topk32) masked padding (so that no tile
    // mixes the two sources), [topk32, topk32 + window) raw window rows.
    const int topk32 = MODE == 1 ? (R.topk + TILE - 1) / TILE * TILE : 0;
    int nrows;
    long long w0 = 0;
    if (MODE == 0) {
        nrows = ndense;
    } else {
        w0 = p - R.W + 1 < 0 ? 0 : p - R.W + 1;
        nrows = topk32 + (R.W > 0 ? (int)(p - w0 + 1) : 0);
    }
    const int s_begin = split * rps;
    const int s_end = min(nrows, s_begin + rps);
    // a multiple of ATT_TILES tiles, the same for every wave (barriers inside); an empty split runs none
    const int ntiles = s_begin < nrows ? rps / TILE : 0;

    // paged entries address the whole pool (the page map gives pool rows); batch-major ones this sequence's
    constexpr int FROWB = D + 80;             // bytes of an FP8 row
    const uint16_t* kvb = R.kv ? (PAGED ? R.kv : (const uint16_t*)((const char*)R.kv + (size_t)b * R.N * (FP8 ? FROWB : D * 2))) : nullptr;
    const size_t kv_rows = PAGED ? (size_t)R.pm.nblocks << R.pm.eshift : (size_t)R.N;
    const uint16_t* rawb = MODE == 1 && R.kv_raw ? R.kv_raw + (size_t)b * R.Lr * D : nullptr;

    bf16x8_t qreg[KS];
    {
        const uint16_t* qp = q + ((size_t)bt * H + (hv ? h : 0)) * D + dh * HD + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) qreg[s] = hv ? as_bf16x8(*(const u32x4_t*)(qp + 16 * s)) : as_bf16x8(u32x4_t{0, 0, 0, 0});
        if (ROPE && dh == 1) {                  // fused rotary embedding of the last 64 dims, at +p
#pragma unroll
            for (int s = KS - ROPE_FUSED_RD / 16; s < KS; ++s)
                qreg[s] = as_bf16x8(rope8(__builtin_bit_cast(u32x4_t, qreg[s]), HD + 16 * s + 8 * g, D, R, (double)p));
        }
    }
    const bf16x8_t qmask = as_bf16x8(u32x4_t{g == 0 && dh == 0 ? BF16_NEG_2P100 : 0u, 0u, 0u, 0u});
    f32x16_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int b16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 4 * (b16 >> 1) + (j16 >> 2);
    const int rsub = lane >> 5, pch = lane & 31;

    // ---- tile loads ----
    // Instruction i (0..15) moves row slots 2i (lanes 0-31) and 2i+1 (lanes 32-63) of one d-half, 16 B
    // per lane, landing at (half + 1024 i + 16 lane); the XOR swizzle goes on the source: the lane
    // fetches logical chunk pch ^ swz_chunk(2i + rsub) = (pch ^ 4 rsub) ^ kappa(i), kappa(i) =
    // 8 (i & 1) | ((i >> 1) & 3).  The two waves of a d-half split the 16 instructions; masked slots
    // load a valid row (their data is never weighted).
    auto kappa = [](int i) -> uint32_t { return (uint32_t)(8 * (i & 1) | ((i >> 1) & 3)); };
    const uint32_t lane_chunk = 16u * (uint32_t)(pch ^ (4 * rsub));
    const uint32_t lane_row = (uint32_t)rsub * (D * 2);
    const int i0 = 8 * hgl;                    // this wave's instructions: i0 .. i0 + 7

    // MODE 1: entry indices of the lane's 16 row slots of a tile, loaded one tile ahead and only used
    // after the next full wait (a use right after the load would also wait for the tile loads).
    int code[TILE / 2];
    auto fetch_codes = [&](int t) {
        if constexpr (MODE == 1) {
            const int r0 = s_begin + t * TILE;
#pragma unroll
            for (int i = 0; i < TILE / 2; ++i) {
                const int r = r0 + 2 * i + rsub;
                const int j = (r < s_end && r < R.topk) ? R.idx[(size_t)bt * R.topk + r] : -1;
                code[i] = PAGED && j >= 0 ? (int)entry_row(R.pm, b, R.N, j) : j;
            }
        }
    };
    // Buffer resources over this d-half of the batch's rows (raw buffer, byte offsets).  An absent
    // array gets an empty resource: nothing is ever loaded through it.
    const bool has_kv = kvb != nullptr, has_raw = MODE == 1 && rawb != nullptr;
    const __amdgpu_buffer_rsrc_t rs_kv = FP8 ?
        make_rsrc(kvb, has_kv ? (uint32_t)(kv_rows * FROWB) : 0u) :
        make_rsrc(has_kv ? kvb + dh * HD : nullptr, has_kv ? (uint32_t)(kv_rows * D * 2 - dh * HD * 2) : 0u);
    // FP8 rows: slot chunk pch of the lane's half takes row chunk f8src (half 0: chunks 15..30 <- codes 0..15,
    // 31 <- the scales; half 1: chunks 11..31 <- row chunks 16..36; the chunks below repeat row chunks that the
    // widening overwrites)
    const uint32_t f8src = dh == 0 ? (pch == 31 ? 36u : (pch >= 15 ? (uint32_t)pch - 15u : (uint32_t)pch))
                                   : (pch >= 11 ? (uint32_t)pch + 5u : (uint32_t)pch + 16u);
    const __amdgpu_buffer_rsrc_t rs_raw =
        make_rsrc(has_raw ? rawb + dh * HD : nullptr, has_raw ? (uint32_t)((size_t)R.Lr * D * 2 - dh * HD * 2) : 0u);
    const int raw_first = MODE == 1 ? (int)(w0 - raw0) : 0;           // raw row of the first window row
    // Issue this wave's part of tile t into `buf`; returns the tile's validity mask (bit = row slot).
    auto issue_tile = [&](uint16_t* buf, int t) -> uint32_t {
        CSA_LDS char* lb = (CSA_LDS char*)buf + dh * HALF_B;
        const int r0 = s_begin + t * TILE;
        auto bdma = [&](__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, int i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (CSA_LDS void*)(lb + 1024 * i), 16, (int)voff, (int)soff, 0, 0);
        };
        const int nval = max(0, min(TILE, s_end - r0));
        if constexpr (MODE == 0) {
            if (FP8) {                                  // (slots past the array reread row 0)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = i0 + k, r = r0 + 2 * i + rsub;
                    bdma(rs_kv, (uint32_t)(r < R.N ? r : 0) * FROWB + 16u * f8src, 0u, i);
                }
            } else if (r0 + TILE <= R.N) {              // all 32 row slots lie inside the array
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = i0 + k;
                    bdma(rs_kv, (lane_row + lane_chunk) ^ (16u * kappa(i)), (uint32_t)r0 * (D * 2) + 2048u * i, i);
                }
            } else {                                    // tail: slots past the array reread row 0
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = i0 + k, r = r0 + 2 * i + rsub;
                    bdma(rs_kv, (uint32_t)(r < R.N ? r : 0) * (D * 2) + (lane_chunk ^ (16u * kappa(i))), 0u, i);
                }
            }
            return nval >= 32 ? 0xffffffffu : ((1u << nval) - 1u);
        } else {
            uint32_t vm = 0;
            if (r0 < topk32) {                          // selected entries (masked slots read row 0)
                uint32_t roff[TILE / 2];
#pragma unroll
                for (int i = 0; i < TILE / 2; ++i) {
                    const bool ok = code[i] >= 0;
                    const unsigned long long bal = __ballot(ok);
                    vm |= (uint32_t)(bal & 1ull) << (2 * i);
                    vm |= (uint32_t)((bal >> 32) & 1ull) << (2 * i + 1);
                    roff[i] = ok ? (uint32_t)code[i] : 0u;
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = i0 + k;
                    if constexpr (FP8) bdma(rs_kv, roff[i] * FROWB + 16u * f8src, 0u, i);
                    else bdma(rs_kv, roff[i] * (D * 2) + (lane_chunk ^ (16u * kappa(i))), 0u, i);
                }
            } else {                                    // raw window rows (masked slots read the first one)
                const int u0 = raw_first + (r0 - topk32);                   // raw row of slot 0
                vm = nval >= 32 ? 0xffffffffu : ((1u << nval) - 1u);
                if (nval == TILE) {
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int i = i0 + k;
                        bdma(rs_raw, (lane_row + lane_chunk) ^ (16u * kappa(i)), (uint32_t)u0 * (D * 2) + 2048u * i, i);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int i = i0 + k, slot_ = 2 * i + rsub;
                        const int u = slot_ < nval ? u0 + slot_ : raw_first;
                        bdma(rs_raw, (uint32_t)u * (D * 2) + (lane_chunk ^ (16u * kappa(i))), 0u, i);
                    }
                }
            }
            return vm;
        }
    };

    typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
    // FP8 tiles: the wave widens the 16 half rows it loaded (rows 16 hgl .. + 15 of its d-half), once its
    // own loads of the tile have landed.  Lane (rsub, pch) writes logical chunk pch of its half row at the
    // swizzled place, from 8 codes times the group's scale or (half 1, pch >= 24) the stored RoPE dims.  A
    // row's write takes its data from every read of that row, so it is issued after them, and LDS executes
    // one wave's instructions in order: the in-place widening never overwrites bytes still to be read.
    auto widen = [&](uint16_t* buf, int t) {
        if constexpr (FP8) {
            if (t >= ntiles || (MODE == 1 && s_begin + t * TILE >= topk32)) return;   // raw rows are bf16
            CSA_LDS char* lb = (CSA_LDS char*)buf + dh * HALF_B;
            const bool nope = dh == 0 || pch < 24;
            const uint32_t a0 = dh == 0 ? 240u + 8u * pch : (nope ? 176u + 8u * pch : 16u * (pch - 1));
            const uint32_t sa = dh == 0 ? 496u + (pch >> 3) : 500u + (nope ? (uint32_t)(pch >> 3) : 0u);
            const uint32_t keep = nope ? 0u : ~0u;
            typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {          // two groups of 4 row pairs: all reads, then the writes
                u32x2_t x0[4], x1[4];
                uint32_t sb[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int row = 2 * (i0 + 4 * h2 + k) + rsub;
                    const CSA_LDS char* rb = lb + 512 * row;
                    x0[k] = *(const CSA_LDS u32x2_t*)(rb + a0);
                    x1[k] = *(const CSA_LDS u32x2_t*)(rb + a0 + 8);
                    sb[k] = *(const CSA_LDS uint8_t*)(rb + sa);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int row = 2 * (i0 + 4 * h2 + k) + rsub;
                    const float scale = __uint_as_float((sb[k] < 1u ? 1u : sb[k]) << 23);      // 2^(s - 127)
#define CSA_W8(X, HI) __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(X, scale, HI))
                    const u32x4_t o = {(CSA_W8(x0[k][0], false) & ~keep) | (x0[k][0] & keep),
                                       (CSA_W8(x0[k][0], true) & ~keep) | (x0[k][1] & keep),
                                       (CSA_W8(x0[k][1], false) & ~keep) | (x1[k][0] & keep),
                                       (CSA_W8(x0[k][1], true) & ~keep) | (x1[k][1] & keep)};
#undef CSA_W8
                    *(CSA_LDS u32x4_t*)(lb + 512 * row + 16 * (pch ^ swz_chunk(row))) = o;
                }
            }
        }
    };

    // ---- LDS reads ----
    // Byte offsets of this lane's reads inside a tile buffer.  With the half 512-byte aligned the
    // swizzled address of k-step s is (qk_off ^ 32 s), and that of the transposed read of rows 8k.. and
    // d-tile d is ((tr_off ^ (64 d + 32 (k & 1))) + 4096 k) (the XOR touches bits 5..8 only).
    const uint32_t qk_off = dh * HALF_B + hl * 512 + 16 * (g ^ swz_chunk(hl));
    const uint32_t tr_off = dh * HALF_B + tr_row * 512 +
                            16 * ((2 * (b16 & 1) + ((j16 >> 1) & 1)) ^ swz_chunk(tr_row)) + 8 * (j16 & 1);
    // max / sum over the two lane halves (the two 16-row groups of a head's column)
    auto xhalf_max = [](float v) -> float {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    auto xhalf_sum = [](float v) -> float {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    };

    // QK of one tile: partial S^T[32 rows][32 heads] over this d-half plus the row mask.
    float x[16];                               // scaled scores of the tile being finished
    auto write_scores = [&](const f32x16_t& sacc, int par) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *(f32x4_t*)&sx[par][w][q4][lane][0] = f32x4_t{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
    };
    auto read_scores = [&](const f32x16_t& sacc, int par) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t o = *(const f32x4_t*)&sx[par][w ^ 2][q4][lane][0];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sv = dh == 0 ? sacc[4 * q4 + i] + o[i] : o[i] + sacc[4 * q4 + i];
                x[4 * q4 + i] = sv * scale_log2;
            }
        }
    };
    // LDS writes complete, then a plain barrier (the tile loads in flight are not waited for here)
    auto exchange_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    // One pipelined step: softmax of tile t (x) interleaved with QK of tile t+1 (from Qb, mask vmn),
    // then PV of tile t (from Pb); returns the partial scores of tile t+1.  Reads are formed from the
    // buffer objects themselves so that the compiler tells them from the loads in flight.
    auto step = [&](const uint16_t* Pbuf, const uint16_t* Qbuf, uint32_t vmn) -> f32x16_t {
        const CSA_LDS char* Pb = (const CSA_LDS char*)Pbuf;
        const CSA_LDS char* Qb = (const CSA_LDS char*)Qbuf;
        uint32_t qb = qk_off, trb = tr_off;
        asm volatile("" : "+v"(qb), "+v"(trb));   // keep the per-read XORs in the loop (no hoisted address table)
        constexpr int QK_AHEAD = ATT64_QK_AHEAD;
        bf16x8_t ka[KS];
        f32x16_t sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
        for (int s = 0; s < QK_AHEAD; ++s) ka[s] = as_bf16x8(*(const CSA_LDS u32x4_t*)(Qb + (qb ^ (32u * s))));
        {
            const uint32_t masked = g == 0 && !((vmn >> hl) & 1u) ? BF16_ONE : 0u;
            sacc = mfma32_bf16(as_bf16x8(u32x4_t{masked, 0u, 0u, 0u}), qmask, sacc);
        }
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(x[8], x[9]), fmaxf(x[10], x[11])), fmaxf(fmaxf(x[12], x[13]), fmaxf(x[14], x[15]))));
        __builtin_amdgcn_sched_barrier(0);
        // the softmax of tile t is spread over the 16 k-steps of tile t+1
        float alpha = 1.f, m_use = 0.f, ps = 0.f;
        u32x4_t pw0, pw1;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sacc = mfma32_bf16(ka[s], qreg[s], sacc);
            if (s + QK_AHEAD < KS)
                ka[s + QK_AHEAD] = as_bf16x8(*(const CSA_LDS u32x4_t*)(Qb + (qb ^ (32u * (s + QK_AHEAD)))));
            if (s == 0) {
                // rescale only when the running max grows by more than 2^8 (exact: the reference
                // point of the exponentials is free; p stays <= 256)
                mx = xhalf_max(mx);
                const bool grow = mx > m_run + 8.0f;
                alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;     // 0 on the first valid tile
                m_run = grow ? mx : m_run;
                m_use = m_run == -INFINITY ? 0.f : m_run;                      // all -inf so far: every p is 0
            } else if (s <= 8) {
                const int j = 2 * (s - 1);
                x[j] = __builtin_amdgcn_exp2f(x[j] - m_use);                   // masked rows -> 0
                x[j + 1] = __builtin_amdgcn_exp2f(x[j + 1] - m_use);
                ps += x[j] + x[j + 1];
            } else if (s <= 12) {
                const int j = s - 9;
                pw0[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
                pw1[j] = pack_bf16x2(x[8 + 2 * j], x[8 + 2 * j + 1]);
            } else if (s == 13) {
                l_run = l_run * alpha + xhalf_sum(ps);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // (rare) the running max grew: rescale the accumulators before this tile's PV
        if (__builtin_expect(__builtin_amdgcn_readfirstlane((uint32_t)__ballot(alpha != 1.0f) |
                                                            (uint32_t)(__ballot(alpha != 1.0f) >> 32)) != 0u, 0)) {
#pragma unroll
            for (int d = 0; d < DT; ++d) acc[d] *= alpha;
        }
        const bf16x8_t pb0 = as_bf16x8(pw0), pb1 = as_bf16x8(pw1);
        // ---- O^T[d-half][h] += V^T P^T (rows in two k-steps of 16); V reads run PV_AHEAD d-tiles ahead ----
        auto trd = [&](uint32_t off) -> u32x2_t {
            return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (CSA_LDS i16x4_t*)const_cast<CSA_LDS char*>(Pb + off)));
        };
        constexpr int PV_AHEAD = ATT64_PV_AHEAD;
        u32x2_t vr[DT][4];
        auto load_d = [&](int d) {
            const uint32_t e = trb ^ (64u * d), o = trb ^ (64u * d + 32u);
            vr[d][0] = trd(e); vr[d][1] = trd(o + 4096u); vr[d][2] = trd(e + 8192u); vr[d][3] = trd(o + 12288u);
        };
#pragma unroll
        for (int d = 0; d < PV_AHEAD; ++d) load_d(d);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < DT; ++d) {
            const u32x2_t* v = vr[d];
            acc[d] = mfma32_bf16(as_bf16x8(u32x4_t{v[0][0], v[0][1], v[1][0], v[1][1]}), pb0, acc[d]);
            acc[d] = mfma32_bf16(as_bf16x8(u32x4_t{v[2][0], v[2][1], v[3][0], v[3][1]}), pb1, acc[d]);
            if (d + PV_AHEAD < DT) load_d(d + PV_AHEAD);
            __builtin_amdgcn_sched_barrier(0);
        }
        return sacc;
    };
    // QK alone (the first tile): partial scores of the tile in Qbuf.
    auto qk_only = [&](const uint16_t* Qbuf, uint32_t vm) -> f32x16_t {
        const CSA_LDS char* Qb = (const CSA_LDS char*)Qbuf;
        f32x16_t sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
        const uint32_t masked = g == 0 && !((vm >> hl) & 1u) ? BF16_ONE : 0u;
        sacc = mfma32_bf16(as_bf16x8(u32x4_t{masked, 0u, 0u, 0u}), qmask, sacc);
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sacc = mfma32_bf16(as_bf16x8(*(const CSA_LDS u32x4_t*)(Qb + (qk_off ^ (32u * s)))), qreg[s], sacc);
        return sacc;
    };

    // ---- the tile pipeline ----
    // Tile t lives in buffer t % 3.  Step t: softmax(t) + QK(t+1), PV(t), exchange of S(t+1) with one
    // barrier; before the barrier each wave waits for its own loads of tile t+2, so after it tile t+2
    // is complete for all waves and buffer t % 3 (PV of tile t done everywhere) takes the loads of
    // tile t+3.  Steps past the last tile compute on stale buffers and their results are dropped.
    uint32_t vm0 = 0, vm1 = 0, vm2 = 0;
    if (ntiles > 0) {
        fetch_codes(0);
        __builtin_amdgcn_s_waitcnt(0);
        vm0 = issue_tile(bufA, 0);
        fetch_codes(1);
        __builtin_amdgcn_s_waitcnt(0);         // own loads of tile 0, codes of tile 1
        widen(bufA, 0);
        vm1 = issue_tile(bufB, 1);
        fetch_codes(2);
        exchange_barrier();                    // tile 0 complete for all waves
        const f32x16_t s0 = qk_only(bufA, vm0);
        write_scores(s0, 0);
        __builtin_amdgcn_s_waitcnt(0);         // own loads of tile 1, codes of tile 2
        widen(bufB, 1);
        exchange_barrier();
        vm2 = issue_tile(bufC, 2);
        fetch_codes(3);
        read_scores(s0, 0);
    }
    for (int t = 0; t < ntiles; t += ATT_TILES) {
        // step t (P = A, QK = B), step t+1 (P = B, QK = C), step t+2 (P = C, QK = A)
#define CSA_ATT_STEP(PB, QB, WB, VMN, DMA_BUF, VM_OUT, K)                                         \
        {                                                                                         \
            const int par = (t + K + 1) & 1;   /* exchange parity of tile t+K+1 */                  \
            const f32x16_t sn = step(PB, QB, VMN);                                                \
            write_scores(sn, par);                                                                \
            __builtin_amdgcn_s_waitcnt(0);     /* own loads of tile t+K+2, codes of tile t+K+3 */  \
            widen(WB, t + K + 2);                                                                 \
            exchange_barrier();                                                                   \
            if (t + K + 3 < ntiles) {                                                             \
                VM_OUT = issue_tile(DMA_BUF, t + K + 3);                                          \
                fetch_codes(t + K + 4);                                                           \
            } else {                                                                              \
                VM_OUT = 0u;                                                                      \
            }                                                                                     \
            read_scores(sn, par);                                                                 \
        }
        CSA_ATT_STEP(bufA, bufB, bufC, vm1, bufA, vm0, 0)
        CSA_ATT_STEP(bufB, bufC, bufA, vm2, bufB, vm1, 1)
        CSA_ATT_STEP(bufC, bufA, bufB, vm0, bufC, vm2, 2)
#undef CSA_ATT_STEP
    }

    // ---- output: both d-half waves of a head group hold the same (m, l) ----
    // Split partials go out as fp16 scaled by one power of two per (split, head), so the two d-half waves of
    // a head group agree on max |O| through LDS first (before the exit of the waves past H, so that every
    // wave of the workgroup reaches the barrier; such a wave's partner is past H too).
    float amax = 0.f;
    if (nsplit > 1) {                          // uniform
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(acc[d][j]));
        amax = xhalf_max(amax);
        if (g == 0) amx[w][hl] = amax;
        __syncthreads();
        amax = fmaxf(amax, amx[w ^ 2][hl]);
    }
    if (!hv) return;
    const bool empty = !(m_run > EMPTY_M);     // no valid row: garbage-weighted sums under a tiny max
    if (empty) {
        m_run = -INFINITY;
        l_run = 0.f;
    }
    // lane holds O^T[dh*256 + d*32 + 8 (j/4) + 4 g + j%4][h]
    if (nsplit == 1) {
        float lse_v;
        const float inv = sink_norm(m_run, l_run, sink_log2(R.sink, h), lse_v);
        if (ROPE && dh == 1) {                  // the output's last 64 dims turn back by -p
#pragma unroll
            for (int d = DT - ROPE_FUSED_RD / 32; d < DT; ++d)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    CSA_ROPE_PAIR(acc[d], 4 * q4, 4 * q4 + 1, HD + d * 32 + 8 * q4 + 4 * g, D, R, -(double)p)
                    CSA_ROPE_PAIR(acc[d], 4 * q4 + 2, 4 * q4 + 3, HD + d * 32 + 8 * q4 + 4 * g + 2, D, R, -(double)p)
                }
        }
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
        if (lse && g == 0 && dh == 0) lse[(size_t)bt * H + h] = lse_v;
    } else {
        // O 2^-e (fp16, round to nearest even) with 2^e >= max |O| over the head's 512 values, stored with m + e
        // and l 2^-e: every term of the merge is unchanged, and each value keeps a relative error <= 2^-11 of
        // the head's largest
        const int e = empty || !(amax > 0.f) ? 0 : __builtin_amdgcn_frexp_expf(amax);
        const float sc = empty ? 0.f : __builtin_amdgcn_ldexpf(1.0f, -e);
        typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
        auto ph = [&](float a, float b2) -> uint32_t {
            const f16x2_t v = {(_Float16)(a * sc), (_Float16)(b2 * sc)};
            return __builtin_bit_cast(uint32_t, v);
        };
        const size_t sl = ((size_t)bt * nsplit + split) * H + h;
        uint16_t* op = (uint16_t*)part_o + sl * D + dh * HD + 4 * g;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(uint2*)(op + d * 32 + 8 * q4) = make_uint2(ph(acc[d][4 * q4], acc[d][4 * q4 + 1]),
                                                             ph(acc[d][4 * q4 + 2], acc[d][4 * q4 + 3]));
        if (g == 0 && dh == 0) part_ml[sl] = make_float2(m_run + (float)e, l_run * sc);
    }
}

// Tile buffers [d-half][32 rows][256] bf16 (distinct objects: the compiler tells a read of one from the
// loads in flight into another) and the score exchange [parity][wave][j/4][lane][j%4].
#define CSA_ATT64_LDS                                                         \
    __shared__ __attribute__((aligned(1024))) uint16_t bufA[2 * TILE * HD];   \
    __shared__ __attribute__((aligned(1024))) uint16_t bufB[2 * TILE * HD];   \
    __shared__ __attribute__((aligned(1024))) uint16_t bufC[2 * TILE * HD];   \
    __shared__ __attribute__((aligned(16))) float sx[2][4][4][64][4];       \
    __shared__ float amx[4][32];

template <int MODE, bool PAGED, bool ROPE, bool FP8>
__global__ __launch_bounds__(TPB, 1) void k_attn64(
    const uint16_t* __restrict__ q, Rows R, int Tq, int H, long long pos0, float scale_log2, int nunits, int nsplit,
    int rps, float* __restrict__ part_o, float2* __restrict__ part_ml, uint16_t* __restrict__ out,
    float* __restrict__ lse)
{
    CSA_ATT64_LDS
    attn64_body<MODE, PAGED, ROPE, FP8>(blockIdx.x, bufA, bufB, bufC, sx, amx, q, R, Tq, H, pos0, scale_log2, nunits, nsplit, rps,
                           part_o, part_ml, out, lse);
}

#undef CSA_ATT64_LDS

// four partial values at element offset i: fp16 (converted exactly to fp32) or fp32
template <bool F16>
__device__ __forceinline__ f32x4_t part4(const float* p, size_t i) {
    if constexpr (F16) {
        typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
        const f16x4_t h = *(const f16x4_t*)((const uint16_t*)p + i);
        return f32x4_t{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    } else {
        return *(const f32x4_t*)(p + i);
    }
}

// Merge split partials in split order: out = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.  Thread tid
// owns d = 4 tid .. 4 tid + 3 of head h; the split loop is unrolled so that several partial loads are
// in flight (the order of the sums is fixed, so the result is deterministic).
// F16: the partials are fp16 (k_attn64's, scaled as above), else fp32 (k_attn's).
template <int D, bool F16>
__device__ __forceinline__ void combine_body(const float* __restrict__ part_o, const float2* __restrict__ part_ml,
                                             int H, int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse,
                                             const float* __restrict__ sink, int h, int bt, const Rows& R, int Tq,
                                             long long pos0)
{
    const int d = threadIdx.x * 4;
    const size_t s0 = (size_t)bt * nsplit * H + h;     // slot of split 0; split s at s0 + s H
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[s0 + (size_t)s * H].x);
    float l = 0.f;
    f32x4_t o = {0, 0, 0, 0};
    if (M != -INFINITY) {
        int s = 0;
        for (; s + 4 <= nsplit; s += 4) {
            float2 ml[4];
            f32x4_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const size_t slot = s0 + (size_t)(s + u) * H;
                ml[u] = part_ml[slot];
                v[u] = part4<F16>(part_o, slot * D + d);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = exp2f(ml[u].x - M);      // 0 for empty splits (m = -inf)
                l += f * ml[u].y;
                o += f * v[u];
            }
        }
        for (; s < nsplit; ++s) {
            const size_t slot = s0 + (size_t)s * H;
            const float2 ml = part_ml[slot];
            const float f = exp2f(ml.x - M);
            l += f * ml.y;
            o += f * part4<F16>(part_o, slot * D + d);
        }
    }
    float lse_v;
    const float inv = sink_norm(M, l, sink_log2(sink, h), lse_v);
    if (R.rope_rd && d + 4 > D - ROPE_FUSED_RD) {      // the output's last 64 dims turn back by -p
        long long raw0;
        int nd;
        const double sp = -(double)row_geo(R, bt / Tq, bt % Tq, Tq, pos0, raw0, nd);
        CSA_ROPE_PAIR(o, 0, 1, d, D, R, sp)
        CSA_ROPE_PAIR(o, 2, 3, d + 2, D, R, sp)
    }
    uint2 v;
    v.x = (uint32_t)f32_to_bf16(o[0] * inv) | ((uint32_t)f32_to_bf16(o[1] * inv) << 16);
    v.y = (uint32_t)f32_to_bf16(o[2] * inv) | ((uint32_t)f32_to_bf16(o[3] * inv) << 16);
    *(uint2*)(out + ((size_t)bt * H + h) * D + d) = v;
    if (lse && threadIdx.x == 0) lse[(size_t)bt * H + h] = lse_v;
}

// grid (H, BT), or with XMAP a 1-D grid of jobs (query, head) laid out by XCD (see XcdJobs)
template <int D, bool XMAP, bool F16>
__global__ __launch_bounds__(D / 4) void k_combine(const float* __restrict__ part_o, const float2* __restrict__ part_ml,
                                                   int H, int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse,
                                                   const float* __restrict__ sink, Rows R, int Tq, long long pos0,
                                                   XcdJobs xj)
{
    int h = blockIdx.x, bt = blockIdx.y;
    if constexpr (XMAP) {
        const int x = (int)(blockIdx.x & 7u), J = xj.lo[x] + (int)(blockIdx.x >> 3);
        if (J >= xj.lo[x + 1]) return;
        h = J % H;
        bt = J / H;
    }
    combine_body<D, F16>(part_o, part_ml, H, nsplit, out, lse, sink, h, bt, R, Tq, pos0);
}

}  // namespace

namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split counts.  k_attn (16 heads per wave): enough workgroups to cover the
// chip twice, splits of >= 64 rows.  k_attn64 (64 heads per workgroup, one
// workgroup per CU): about one workgroup per CU, but at least ATT_MIN_TILES
// tiles per split (each split writes 64 heads x 512 fp32 partials), tile counts
// a multiple of 3.  (Measured at 32 x 128K, 64 heads, k = 512: splits of 3 tiles
// on 224 workgroups take 26.7 us with the merge against 28.6 us for 6 tiles on 128.)
constexpr int ATT_MIN_TILES = 3, ATT_TARGET_WG = 256;
static bool use64(int D, int H) { return D == 512 && H % 32 == 0; }

static void choose_split(int BT, int H, int D, int max_rows, int* nsplit, int* rps) {
    if (max_rows <= 0) { *nsplit = 1; *rps = 128; return; }
    if (use64(D, H)) {
        const int HP = (H + 63) / 64;
        const int ns = std::max(1, ATT_TARGET_WG / (BT * HP));
        const int unit = ATT_TILES * TILE;
        int r = (max_rows + ns - 1) / ns;
        r = std::max(r, ATT_MIN_TILES * TILE);
        r = (r + unit - 1) / unit * unit;
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

// Row-space size of one query: dense N; sparse topk (padded to whole tiles for k_attn64) + window.
static int attn_rows(int mode, int H, int D, int n, int W) {
    if (mode == 0) return n;
    return (use64(D, H) ? (n + TILE - 1) / TILE * TILE : n) + W;
}

// k_attn128 (128 heads per workgroup, one workgroup per CU): the rows per split are the same for every
// workgroup of a launch (whole tiles), chosen so that the launch's tiles spread over about
// A128_TARGET_WG workgroups, and at least A128_MIN_TILES tiles per split.
constexpr int A128_TARGET_WG = 256, A128_MIN_TILES = 4;
static bool use128(int D, int H) { return D == 512 && H % 128 == 0; }
static int a128_tiles(int rows) { return (rows + TILE - 1) / TILE; }
static int a128_rps(long long total_tiles) {
    long long tpw = (total_tiles + A128_TARGET_WG - 1) / A128_TARGET_WG;
    tpw = std::max<long long>(tpw, A128_MIN_TILES);
    long long r = (tpw * TILE + ATT128_UNIT - 1) / ATT128_UNIT * ATT128_UNIT;
    return (int)std::min<long long>(r, ATT128_MAX_RPS);
}
static int a128_nsplit(int max_rows, int rps) { return max_rows <= 0 ? 1 : (max_rows + rps - 1) / rps; }
// row space of k_attn128 (topk padded to whole tiles, then the window)
static int a128_rows(int mode, int n, int W) { return mode == 0 ? n : a128_tiles(n) * TILE + W; }
static size_t part_bytes(int BT, int ns, int H, int D) {
    if (ns <= 1) return 0;
    return align256((size_t)BT * ns * H * D * 4) + align256((size_t)BT * ns * H * 8);
}

size_t attn_ws_bytes(int B, int Tq, int H, int D, int mode, int n, int W) {
    const int BT = B * Tq;
    const int max_rows = attn_rows(mode, H, D, n, W);
    int ns, rps;
    choose_split(BT, H, D, max_rows, &ns, &rps);
    size_t s = part_bytes(BT, ns, H, D);
    if (use128(D, H)) {      // either kernel may run (k_attn64 when an array is beyond 32-bit offsets)
        const int r128 = a128_rows(mode, n, W);
        const int rp = a128_rps((long long)BT * (H / 128) * a128_tiles(r128));
        s = std::max(s, part_bytes(BT, a128_nsplit(r128, rp), H, D));
    }
    return s;
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
    R.sink = a.sink;
    R.seq_lens = a.seq_lens;
    R.pm = a.pm;
    R.v = (const uint16_t*)a.v;
    R.v_raw = (const uint16_t*)a.v_raw;
    R.kv_fp8 = a.kv_fp8;
    R.rope_rd = a.rope_rd;
    R.rope_l2t = a.rope_rd ? log2(a.rope_theta) : 0.0;
    const int BT = B * Tq;
    const int max_rows = a.mode == 0 ? a.N : attn_rows(1, H, D, a.topk, a.W);
    int ns, rps;
    choose_split(BT, H, D, max_rows, &ns, &rps);
    float* part_o = nullptr;
    float2* part_ml = nullptr;
    if (ns > 1) {
        part_o = (float*)ws;
        part_ml = (float2*)((char*)ws + align256((size_t)BT * ns * H * D * 4));
    }
    const float sl2 = scale * LOG2E;
    // The buffer-load kernels (k_attn128, k_attn64) need every array within reach of 32-bit byte offsets (a
    // cache of more than 4 GiB per sequence, or a page pool of more than 4 GiB, runs the generic kernel, which
    // addresses rows with 64-bit pointers), keys that are their own values, and, for k_attn64, a dense row
    // set that is contiguous (paged dense rows run the generic kernel too).
    const size_t kv_rows = a.pm.table ? (size_t)a.pm.nblocks << a.pm.eshift : (size_t)a.N;
    const bool fp8 = a.kv_fp8 != 0;                  // FP8 entry rows: every kernel widens them to bf16 in LDS
    const bool big32 = kv_rows * (fp8 ? D + 80 : D * 2) > 0xffffffffull ||
                       (a.mode == 1 && (size_t)a.Lr * D * 2 > 0xffffffffull);
    const bool sepv = a.v || a.v_raw;
    if (use128(D, H) && !big32 && !sepv) {
        const int r128 = a.mode == 0 ? a.N : a128_rows(1, a.topk, a.W);
        AttnJob j{};
        j.q = (const uint16_t*)q; j.R = R; j.Tq = Tq; j.H = H; j.pos0 = pos0; j.scale_log2 = sl2;
        j.rps = a128_rps((long long)BT * (H / 128) * a128_tiles(r128));
        j.nsplit = a128_nsplit(r128, j.rps);
        j.nunits = BT * j.nsplit;
        j.out = (uint16_t*)out; j.lse = lse;
        // k_attn128 applies an attention sink and the output's rotation in its merge only: a sink or a rotation
        // with a single split runs k_attn64
        if (!((R.sink || R.rope_rd) && j.nsplit == 1)) {
            if (j.nsplit > 1) {
                j.part_o = (float*)ws;
                j.part_ml = (float2*)((char*)ws + align256((size_t)BT * j.nsplit * H * D * 4));
            }
            return attn128_launch(j, st, tag);
        }
    }
    if (use64(D, H) && !big32 && !sepv && !(a.pm.table && a.mode == 0)) {
        const int nunits = BT * ns, HP = (H + 63) / 64;
        const int per = (nunits * HP + 7) / 8, nblk = 8 * per;
#define CSA_ATT64(MODE_, PAGED_, ROPE_, FP8_)                                                                \
    CSA_LAUNCH(tag, (k_attn64<MODE_, PAGED_, ROPE_, FP8_>), dim3(nblk), dim3(TPB), 0, st, (const uint16_t*)q, R, Tq, H, \
               pos0, sl2, nunits, ns, rps, part_o, part_ml, (uint16_t*)out, lse)
#define CSA_ATT64_F(MODE_, PAGED_, ROPE_) \
    do { if (fp8) CSA_ATT64(MODE_, PAGED_, ROPE_, true); else CSA_ATT64(MODE_, PAGED_, ROPE_, false); } while (0)
        const bool rope = R.rope_rd != 0;
        if (a.mode == 0) { if (rope) CSA_ATT64_F(0, false, true); else CSA_ATT64_F(0, false, false); }
        else if (a.pm.table) { if (rope) CSA_ATT64_F(1, true, true); else CSA_ATT64_F(1, true, false); }
        else { if (rope) CSA_ATT64_F(1, false, true); else CSA_ATT64_F(1, false, false); }
#undef CSA_ATT64_F
#undef CSA_ATT64
        if (ns > 1) {
            // a query's head h: the XCD of its middle split's block of head pair h / 64
            int most;
            const XcdJobs xj = xcd_jobs(BT * H, 1, [&](int g) {
                return ((g / H * ns + ns / 2) * HP + g % H / 64) / per; }, &most);
            CSA_LAUNCH("k_combine", (k_combine<512, true, true>), dim3(8 * most), dim3(128), 0, st, part_o, part_ml, H, ns,
                       (uint16_t*)out, lse, R.sink, R, Tq, pos0, xj);
        }
        return 0;
    }
    dim3 grid(ns, (H + 63) / 64, BT);
#define CSA_GENERIC(D_, S_, F_)                                                                            \
    do {                                                                                                     \
        if (R.rope_rd)                                                                                       \
            CSA_LAUNCH(tag, (k_attn<D_, S_, F_, true>), grid, dim3(TPB), 0, st, (const uint16_t*)q, R, Tq, H, pos0, \
                       sl2, ns, rps, part_o, part_ml, (uint16_t*)out, lse);                                  \
        else                                                                                                 \
            CSA_LAUNCH(tag, (k_attn<D_, S_, F_, false>), grid, dim3(TPB), 0, st, (const uint16_t*)q, R, Tq, H, pos0, \
                       sl2, ns, rps, part_o, part_ml, (uint16_t*)out, lse);                                  \
    } while (0)
    if (D == 512) {
        if (sepv && fp8) CSA_GENERIC(512, true, true);
        else if (sepv) CSA_GENERIC(512, true, false);
        else if (fp8) CSA_GENERIC(512, false, true);
        else CSA_GENERIC(512, false, false);
        if (ns > 1)
            CSA_LAUNCH("k_combine", (k_combine<512, false, false>), dim3(H, BT), dim3(128), 0, st, part_o, part_ml, H, ns,
                       (uint16_t*)out, lse, R.sink, R, Tq, pos0, XcdJobs{});
    } else if (D == 128) {
        if (sepv && fp8) CSA_GENERIC(128, true, true);
        else if (sepv) CSA_GENERIC(128, true, false);
        else if (fp8) CSA_GENERIC(128, false, true);
        else CSA_GENERIC(128, false, false);
        if (ns > 1)
            CSA_LAUNCH("k_combine", (k_combine<128, false, false>), dim3(H, BT), dim3(32), 0, st, part_o, part_ml, H, ns,
                       (uint16_t*)out, lse, R.sink, R, Tq, pos0, XcdJobs{});
    } else {
        return fail(6, "attention: D = %d unsupported", D);
    }
#undef CSA_GENERIC
    return 0;
}

}  // namespace csa_host

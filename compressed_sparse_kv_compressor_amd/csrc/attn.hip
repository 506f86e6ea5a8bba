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

// Split count: enough workgroups to cover the chip twice, splits of >= 64 rows.
static void choose_split(int BT, int HG, int max_rows, int* nsplit, int* rps) {
    if (max_rows <= 0) { *nsplit = 1; *rps = 32; return; }
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
    const int BT = B * Tq, HG = (H + 63) / 64;
    int ns, rps;
    choose_split(BT, HG, max_rows, &ns, &rps);
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
    const int BT = B * Tq, HG = (H + 63) / 64;
    const int max_rows = a.mode == 0 ? a.N : a.topk + a.W;
    int ns, rps;
    choose_split(BT, HG, max_rows, &ns, &rps);
    float* part_o = nullptr;
    float2* part_ml = nullptr;
    if (ns > 1) {
        part_o = (float*)ws;
        part_ml = (float2*)((char*)ws + align256((size_t)BT * ns * H * D * 4));
    }
    const float sl2 = scale * LOG2E;
    dim3 grid(ns, HG, BT);
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

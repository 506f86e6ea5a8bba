// compress.hip -- token-level KV compressor on gfx950.
//
// Method: "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1:
// a token-level compressor merges the KV of every m tokens into one entry (HCA:
// a much larger m'); "DeepSeek-V4 技术报告解读" item 1: the sequence shrinks to
// 1/m.  The pooling weights are not printed on the pages; this library uses a
// softmax gate inside each block (the block mean when the gate is zero).
//
// Pipeline: k_pool reads each block's hidden rows once, computes the gate
// logits (block reduction) and the softmax-pooled hidden row with an online
// softmax over the block's tokens (any m), and stores it as bf16; k_gemm then
// projects pooled rows by the output-major weights with v_mfma_f32_16x16x32_bf16
// (pool-then-project: equal to project-then-pool by linearity, m times fewer
// FLOPs).  The window rows (raw projected KV of the last W tokens) use the same
// GEMM with raw hidden rows as its A operand.
#include "common.h"
#include "kernels.h"

namespace {

using namespace csa;

constexpr int PTPB = 256;
constexpr int TG = 4;   // tokens per reduction round

template <int CPT>   // 16-byte chunks per thread (Dh = CPT * 8 * 256 at most)
__global__ __launch_bounds__(PTPB) void k_pool(const uint16_t* __restrict__ X, const float* __restrict__ w_gate,
                                              const float* __restrict__ b_slot, long long L, int Dh, int m, int Nc,
                                              uint16_t* __restrict__ pooled)
{
    __shared__ float red[TG][PTPB / 64];
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = lane_id(), wave = tid >> 6;
    const long long t0 = (long long)j * m;
    const int nt = (int)(min((long long)(j + 1) * m, L) - t0);
    const int nchunk = Dh / 8;
    float gw[CPT][8];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int ch = tid + c * PTPB;
#pragma unroll
        for (int e = 0; e < 8; ++e) gw[c][e] = ch < nchunk ? w_gate[ch * 8 + e] : 0.f;
    }
    float acc[CPT][8];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
    float mrun = -INFINITY, lrun = 0.f;
    const uint16_t* Xb = X + ((size_t)b * L + t0) * Dh;
    for (int tb = 0; tb < nt; tb += TG) {
        float xv[TG][CPT][8];
        float part[TG];
#pragma unroll
        for (int u = 0; u < TG; ++u) {
            part[u] = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int ch = tid + c * PTPB;
                u32x4_t v = u32x4_t{0, 0, 0, 0};
                if (tb + u < nt && ch < nchunk) v = *(const u32x4_t*)(Xb + (size_t)(tb + u) * Dh + ch * 8);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xv[u][c][2 * e] = __uint_as_float(v[e] << 16);
                    xv[u][c][2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) part[u] = fmaf(xv[u][c][e], gw[c][e], part[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < TG; ++u) {
            float v = part[u];
            for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_f(v, o);
            if (lane == 0) red[u][wave] = v;
        }
        __syncthreads();
        float z[TG];
        float zmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < TG; ++u) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < PTPB / 64; ++w) s += red[u][w];
            s += b_slot ? b_slot[min(tb + u, m - 1)] : 0.f;
            z[u] = tb + u < nt ? s : -INFINITY;
            zmax = fmaxf(zmax, z[u]);
        }
        __syncthreads();
        const float mnew = fmaxf(mrun, zmax);
        const float alpha = exp2f((mrun - mnew) * 1.4426950408889634f);
        float pw[TG];
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < TG; ++u) { pw[u] = exp2f((z[u] - mnew) * 1.4426950408889634f); ps += pw[u]; }
        lrun = lrun * alpha + ps;
        mrun = mnew;
#pragma unroll
        for (int c = 0; c < CPT; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = acc[c][e] * alpha;
#pragma unroll
                for (int u = 0; u < TG; ++u) a = fmaf(pw[u], xv[u][c][e], a);
                acc[c][e] = a;
            }
    }
    const float inv = 1.0f / lrun;
    uint16_t* dst = pooled + ((size_t)b * Nc + j) * Dh;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int ch = tid + c * PTPB;
        if (ch < nchunk) {
            u32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = (uint32_t)f32_to_bf16(acc[c][2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[c][2 * e + 1] * inv) << 16);
            *(u32x4_t*)(dst + ch * 8) = v;
        }
    }
}

// C[M][N] = A[M][K] . Wt[N][K]^T, bf16 in, fp32 accumulate, bf16 / e4m3 out.
// A rows are addressed through a row map: mode 0 -> A + i*K; mode 1 (window)
// -> row i = b*W + u of hidden token L-W+u (zero when negative).
struct ARows {
    int mode;
    const uint16_t* A;
    long long L;
    int W;
};

constexpr int GT = 128, GK = 64, GTPB = 256, GRS = GK + 8;

__device__ __forceinline__ const uint16_t* arow(const ARows& a, int i, int K) {
    if (a.mode == 0) return a.A + (size_t)i * K;
    const int b = i / a.W, u = i % a.W;
    const long long t = a.L - a.W + u;
    return t < 0 ? nullptr : a.A + ((size_t)b * a.L + t) * K;
}

template <int OUT_E4M3>
__global__ __launch_bounds__(GTPB) void k_gemm(ARows a, const uint16_t* __restrict__ Wt, int M, int N, int K,
                                               void* __restrict__ C)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[GT * GRS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[GT * GRS];
    const int m0 = blockIdx.x * GT, n0 = blockIdx.y * GT;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f32x4_t{0, 0, 0, 0};
    for (int k0 = 0; k0 < K; k0 += GK) {
        // 128 rows x 64 k = 1024 chunks of 16 B for each of A and B
        for (int c = tid; c < GT * GK / 8; c += GTPB) {
            const int r = c / (GK / 8), cc = c % (GK / 8);
            const int gi = m0 + r, gj = n0 + r;
            u32x4_t va = u32x4_t{0, 0, 0, 0}, vb = u32x4_t{0, 0, 0, 0};
            if (gi < M) {
                const uint16_t* src = arow(a, gi, K);
                if (src) va = *(const u32x4_t*)(src + k0 + cc * 8);
            }
            if (gj < N) vb = *(const u32x4_t*)(Wt + (size_t)gj * K + k0 + cc * 8);
            *(u32x4_t*)(As + r * GRS + cc * 8) = va;
            *(u32x4_t*)(Bs + r * GRS + cc * 8) = vb;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < GK / 32; ++ks) {
            bf16x8_t av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = as_bf16x8(*(const u32x4_t*)(As + (wm + i * 16 + col) * GRS + ks * 32 + 8 * grp));
                bv[i] = as_bf16x8(*(const u32x4_t*)(Bs + (wn + i * 16 + col) * GRS + ks * 32 + 8 * grp));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[i][jj] = mfma16_bf16(av[i], bv[jj], acc[i][jj]);
        }
        __syncthreads();
    }
    // lane holds C[wm + i*16 + 4*grp + r][wn + jj*16 + col]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int gi = m0 + wm + i * 16 + 4 * grp + r;
            if (gi >= M) continue;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int gj = n0 + wn + jj * 16 + col;
                if (gj >= N) continue;
                const float v = acc[i][jj][r];
                if (OUT_E4M3) ((uint8_t*)C)[(size_t)gi * N + gj] = f32_to_e4m3(v);
                else ((uint16_t*)C)[(size_t)gi * N + gj] = f32_to_bf16(v);
            }
        }
}

}  // namespace

namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t compress_ws_bytes(int B, long long L, int Dh, int m) {
    const long long Nc = (L + m - 1) / m;
    return align256((size_t)B * Nc * Dh * 2);
}

int compress_launch(const void* hidden, const void* w_kv, const void* w_ik, const float* w_gate,
                    const float* b_slot, int B, long long L, int Dh, int D, int dI, int m, int W,
                    int ik_dtype, void* kv_out, void* ik_out, void* win_out, void* ws, hipStream_t st) {
    const int Nc = (int)((L + m - 1) / m);
    uint16_t* pooled = (uint16_t*)ws;
    const int cpt = (Dh / 8 + PTPB - 1) / PTPB;
    dim3 gp(Nc, B);
#define CSA_POOL(C)                                                                                    \
    if (cpt <= C) {                                                                                    \
        CSA_LAUNCH("k_pool", k_pool<C>, gp, dim3(PTPB), 0, st, (const uint16_t*)hidden, w_gate, b_slot, \
                   L, Dh, m, Nc, pooled);                                                             \
    } else
    CSA_POOL(1) CSA_POOL(2) CSA_POOL(4) CSA_POOL(8) { return fail(6, "compress: Dh = %d too large", Dh); }
#undef CSA_POOL
    const int M = B * Nc;
    ARows pa{0, pooled, L, 0};
    CSA_LAUNCH("k_gemm", k_gemm<0>, dim3((M + GT - 1) / GT, (D + GT - 1) / GT), dim3(GTPB), 0, st, pa,
               (const uint16_t*)w_kv, M, D, Dh, kv_out);
    if (w_ik && ik_out) {
        if (ik_dtype == 1)
            CSA_LAUNCH("k_gemm", k_gemm<1>, dim3((M + GT - 1) / GT, (dI + GT - 1) / GT), dim3(GTPB), 0, st, pa,
                       (const uint16_t*)w_ik, M, dI, Dh, ik_out);
        else
            CSA_LAUNCH("k_gemm", k_gemm<0>, dim3((M + GT - 1) / GT, (dI + GT - 1) / GT), dim3(GTPB), 0, st, pa,
                       (const uint16_t*)w_ik, M, dI, Dh, ik_out);
    }
    if (win_out && W > 0) {
        ARows wa{1, (const uint16_t*)hidden, L, W};
        const int Mw = B * W;
        CSA_LAUNCH("k_gemm", k_gemm<0>, dim3((Mw + GT - 1) / GT, (D + GT - 1) / GT), dim3(GTPB), 0, st, wa,
                   (const uint16_t*)w_kv, Mw, D, Dh, win_out);
    }
    return 0;
}

}  // namespace csa_host

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

// ---------------------------------------------------------------------------
// k_pool2: one streaming pass over the hidden rows that pools fine blocks (m tokens, CSA) and
// coarse blocks (mc tokens, HCA) at once, so that both caches cost one read of the hidden rows.
// A workgroup covers a span of S tokens (the coarse block, or 128 tokens without one); each of its
// four waves takes S/4 consecutive tokens, G at a time (G = m with fine blocks, else 4).  A lane
// holds CPL 16-byte chunks of each token row (chunk c at element 8 (64 c + lane)), so the gate dot
// products are lane partials plus one wave reduction, and no workgroup barrier is needed until the
// coarse merge at the end.  Fine: softmax over the group's valid tokens, pooled row written at
// once.  Coarse: an online softmax per wave, then the four waves' (max, sum, accumulator) merged
// through LDS.  Each fp32 gate weight is staged in LDS as two bf16 terms (hi + lo, within 2^-17
// of it), as [chunk][hi, lo][lane] 16-byte vectors, so that the gate products run as bf16 pair dot
// instructions straight on the packed rows (fp32 accumulation) and each read is one contiguous
// 16-byte access per lane.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
// (by value: a bit_cast applied directly to a vector-element expression was compiled as element 0)
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }
constexpr float LOG2E = 1.4426950408889634f;

// Sum over the wave, the same value in every lane: DPP within rows of 16 (swap neighbours, swap
// pairs, mirror the halves of 8, mirror the row), then the row swaps of permlane16 / permlane32.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

template <int CPL, int G, int MODE>   // MODE bit 0: fine blocks, bit 1: coarse blocks
__global__ __launch_bounds__(256, 2) void k_pool2(const uint16_t* __restrict__ X, long long L, int Dh, int S,
                                               int m, const float* __restrict__ gate_f, const float* __restrict__ bslot_f,
                                               int Nf, uint16_t* __restrict__ out_f,
                                               int mc, const float* __restrict__ gate_c, const float* __restrict__ bslot_c,
                                               int Ncc, uint16_t* __restrict__ out_c, int b0)
{
    __shared__ u32x4_t gl[2][CPL * 2 * 64];                    // gates: [fine, coarse][chunk][hi, lo][lane]
    __shared__ f32x4_t mrg[4][CPL / 2 * 2 * 64];               // coarse merge: half of the chunks at a time
    __shared__ float ml[4][2];
    const int b = b0 + (int)blockIdx.y, tid = threadIdx.x, lane = lane_id(), w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long long t0 = (long long)blockIdx.x * S;
    constexpr bool fine = MODE & 1, coarse = MODE & 2;
    // each fp32 gate weight as the sum of two bf16 values (hi = RNE(g), lo = RNE(g - hi): within
    // 2^-17 of g), so that the dot products run as bf16 pair dots on the packed rows
    auto split_gate = [&](const float* g, int c, int l, u32x4_t& hi, u32x4_t& lo) {
        const f32x4_t a = *(const f32x4_t*)(g + 8 * (64 * c + l)), b2 = *(const f32x4_t*)(g + 8 * (64 * c + l) + 4);
        const float v[8] = {a[0], a[1], a[2], a[3], b2[0], b2[1], b2[2], b2[3]};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            hi[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
            lo[p] = pack_bf16x2(v[2 * p] - __uint_as_float(hi[p] << 16), v[2 * p + 1] - __uint_as_float(hi[p] & 0xffff0000u));
        }
    };
    for (int i = tid; i < CPL * 64; i += 256) {
        const int c = i / 64, l = i & 63;
        if (fine) split_gate(gate_f, c, l, gl[0][(2 * c) * 64 + l], gl[0][(2 * c + 1) * 64 + l]);
        if (coarse) split_gate(gate_c, c, l, gl[1][(2 * c) * 64 + l], gl[1][(2 * c + 1) * 64 + l]);
    }
    __syncthreads();
    const int span = S / 4;
    const long long tw = t0 + (long long)w * span;             // this wave's first token
    float acc[CPL][8];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
    float mrun = -INFINITY, lrun = 0.f;
    const uint16_t* Xb = X + (size_t)b * L * Dh;
#pragma unroll 1
    for (int g0 = 0; g0 < span; g0 += G) {
        const long long tg = tw + g0;
        if (tg >= L) break;                                     // uniform
        u32x4_t x[G][CPL];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const long long tk = min(tg + u, L - 1);            // missing tokens reread the last one
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[u][c] = *(const u32x4_t*)(Xb + (size_t)tk * Dh + 8 * (64 * c + lane));
        }
        float zf[G], zc[G];
#pragma unroll
        for (int u = 0; u < G; ++u) zf[u] = zc[u] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {                   // hi parts, then lo parts of the gates
                const u32x4_t gf = fine ? gl[0][(2 * c + hf) * 64 + lane] : u32x4_t{0, 0, 0, 0};
                const u32x4_t gc = coarse ? gl[1][(2 * c + hf) * 64 + lane] : u32x4_t{0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < G; ++u)
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const bf16x2_t xv = as_bf16x2(x[u][c][p]);
                        if (fine) zf[u] = __builtin_amdgcn_fdot2_f32_bf16(xv, as_bf16x2(gf[p]), zf[u], false);
                        if (coarse) zc[u] = __builtin_amdgcn_fdot2_f32_bf16(xv, as_bf16x2(gc[p]), zc[u], false);
                    }
                // (keeps the gate reads of later chunks from being hoisted here: they would hold
                // 8 CPL more registers)
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (fine) zf[u] = wave_sum(zf[u]);
            if (coarse) zc[u] = wave_sum(zc[u]);
        }
        // the packed rows are expanded again below (the expanded values of the gate phase are not
        // kept: that would take 8 G CPL more registers)
#pragma unroll
        for (int u = 0; u < G; ++u)
#pragma unroll
            for (int c = 0; c < CPL; ++c) asm volatile("" : "+v"(x[u][c]));
        // weights of the group's tokens: fine softmax over the block; coarse online softmax, whose
        // running maximum (and the rescale of the accumulators) moves only when the group's
        // maximum exceeds it (a uniform branch)
        float pf[G], pcw[G], inv = 0.f;
        if (fine) {
            float mx = -INFINITY, l = 0.f;
#pragma unroll
            for (int u = 0; u < G; ++u) {
                zf[u] += bslot_f ? bslot_f[u] : 0.f;
                if (tg + u < L) mx = fmaxf(mx, zf[u]);
            }
#pragma unroll
            for (int u = 0; u < G; ++u) { pf[u] = tg + u < L ? exp2f((zf[u] - mx) * LOG2E) : 0.f; l += pf[u]; }
            inv = 1.0f / l;
        }
        if (coarse) {
            const long long jb = (long long)blockIdx.x * S;    // the coarse block's first token (S = mc)
            float gm = -INFINITY;
#pragma unroll
            for (int u = 0; u < G; ++u) {
                zc[u] += bslot_c ? bslot_c[(int)(tg + u - jb)] : 0.f;
                if (tg + u < L) gm = fmaxf(gm, zc[u]);
            }
            if (gm > mrun) {
                const float alpha = exp2f((mrun - gm) * LOG2E);
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[c][e] *= alpha;
                lrun *= alpha;
                mrun = gm;
            }
#pragma unroll
            for (int u = 0; u < G; ++u) { pcw[u] = tg + u < L ? exp2f((zc[u] - mrun) * LOG2E) : 0.f; lrun += pcw[u]; }
        }
        // one expansion of each packed element feeds both poolings
        uint16_t* dst = fine ? out_f + ((size_t)b * Nf + (size_t)(tg / (fine ? m : 1))) * Dh : nullptr;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float flo = 0.f, fhi = 0.f;
                float clo = coarse ? acc[c][2 * q] : 0.f, chi = coarse ? acc[c][2 * q + 1] : 0.f;
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    const float lo = __uint_as_float(x[u][c][q] << 16), hi = __uint_as_float(x[u][c][q] & 0xffff0000u);
                    if (fine) { flo = fmaf(pf[u], lo, flo); fhi = fmaf(pf[u], hi, fhi); }
                    if (coarse) { clo = fmaf(pcw[u], lo, clo); chi = fmaf(pcw[u], hi, chi); }
                }
                if (fine) o[q] = pack_bf16x2(flo * inv, fhi * inv);
                if (coarse) { acc[c][2 * q] = clo; acc[c][2 * q + 1] = chi; }
            }
            if (fine) *(u32x4_t*)(dst + 8 * (64 * c + lane)) = o;
        }
    }
    if (!coarse) return;
    // merge the four waves' partial softmax sums (waves without tokens carry max -inf and sum 0)
    if (lane == 0) { ml[w][0] = mrun; ml[w][1] = lrun; }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, ml[v][0]);
    float sc[4], Lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) { sc[v] = ml[v][1] > 0.f ? exp2f((ml[v][0] - M) * LOG2E) : 0.f; Lsum += ml[v][1] * sc[v]; }
    const float inv = 1.0f / Lsum;
    uint16_t* dst = out_c + ((size_t)b * Ncc + blockIdx.x) * Dh;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {                            // chunks [hp CPL/2, (hp + 1) CPL/2)
#pragma unroll
        for (int c = 0; c < CPL / 2; ++c)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int cc = hp * (CPL / 2) + c;
                mrg[w][(2 * c + hf) * 64 + lane] = f32x4_t{acc[cc][4 * hf], acc[cc][4 * hf + 1], acc[cc][4 * hf + 2],
                                                           acc[cc][4 * hf + 3]};
            }
        __syncthreads();
        // wave w combines chunk slots [w CPL/8 ..) of this half: CPL/2 chunks x 2 halves x 64 lanes
        for (int i = tid; i < CPL / 2 * 2 * 64; i += 256) {
            f32x4_t a = mrg[0][i] * sc[0];
#pragma unroll
            for (int v = 1; v < 4; ++v) a += mrg[v][i] * sc[v];
            const int c = i / 128, hf = (i / 64) & 1, l = i & 63;
            const int e0 = 8 * (64 * (hp * (CPL / 2) + c) + l) + 4 * hf;
            uint2 o;
            o.x = pack_bf16x2(a[0] * inv, a[1] * inv);
            o.y = pack_bf16x2(a[2] * inv, a[3] * inv);
            *(uint2*)(dst + e0) = o;
        }
        __syncthreads();
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

// ---------------------------------------------------------------------------
// k_gemm2: C = A . [B0; B1]^T for contiguous A rows (pooled entries, or one sequence's window
// rows), bf16 in, fp32 accumulate.  Output columns [0, N0) go to C0 ([M][N0], bf16) and
// [N0, N0 + N1) to C1 ([M][N1], bf16 or e4m3), so the KV and indexer-key projections of the same
// pooled rows are one launch.  gridDim.y batches of rows: batch y reads A + y a_bstride and writes
// rows y M ..  With S > 1 the K range is split S ways and each split writes fp32 partial sums to
// P [y][S][M][N0 + N1], which k_g2reduce adds in split order (deterministic) and rounds.
// A workgroup owns a 256 x 256 tile: eight waves (two per SIMD, so that one computes while the other
// waits on a barrier or LDS), each 128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (128 fp32
// accumulators per lane; four waves of 128 x 128 with the accumulators in AGPRs ran ~6% slower).  K advances 32 at a time through
// four LDS buffers (64-byte rows, 16-byte chunk c of row r stored at c ^ ((r >> 2) & 3): the 16
// lanes a 16-byte read serves per cycle then cover all 64 banks), filled by buffer-load DMA issued
// two steps ahead; every step issues the same number of loads (steps past the end reread the last
// one), so the wait for a step is an exact vmcnt.  Workgroups are laid out so that each
// XCD takes a contiguous run of tiles, N fastest: the tiles sharing an A block share an L2.
// ---------------------------------------------------------------------------
constexpr int G2_T = 256, G2_KS = 32, G2_NB = 4, G2_ROWB = G2_KS * 2;     // tile, K step, buffers, row bytes
constexpr int G2_BUF = 2 * G2_T * G2_ROWB;                                 // A rows then B rows: 32 KiB
constexpr int G2_NW = 8;                                                   // waves per workgroup (4 or 8)
constexpr int G2_WNB = 16 / G2_NW;                                         // 32-column blocks per wave (4 or 2)
constexpr int G2_WNW = G2_T / (32 * G2_WNB);                               // waves across N (2 or 4)
constexpr int G2_DMA = G2_T * G2_ROWB / 1024 / G2_NW;                      // 1 KiB loads per wave per operand

// s_waitcnt immediate: vmcnt(n) with expcnt and lgkmcnt left free
__device__ __forceinline__ constexpr int vmcnt_imm2(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t g2_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int C1_E4M3>
__global__ __launch_bounds__(64 * G2_NW) void k_gemm2(const uint16_t* __restrict__ A, long long a_bstride, int M, int K,
                                               const uint16_t* __restrict__ B0, int N0, const uint16_t* __restrict__ B1,
                                               int N1, uint16_t* __restrict__ C0, void* __restrict__ C1, int S,
                                               float* __restrict__ P)
{
    __shared__ __attribute__((aligned(1024))) char g2_lds[G2_NB * G2_BUF];
    const int N = N0 + N1;
    const int ntn = (N + G2_T - 1) / G2_T, ntm = (M + G2_T - 1) / G2_T, nunits = ntm * ntn * S;
    const int per_xcd = (nunits + 7) / 8;
    const int unit = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (unit >= nunits) return;
    const int tile = unit / S, ks = unit % S;
    const int m0 = (tile / ntn) * G2_T, n0 = (tile % ntn) * G2_T;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (w / G2_WNW) * 128, wn = (w % G2_WNW) * (32 * G2_WNB);
    const int nk = K / S / G2_KS, kbeg = ks * (K / S);
    const int y = blockIdx.y;
    A += (size_t)y * a_bstride;
    C0 += (size_t)y * M * N0;

    // sources: the tile's A rows through one resource; B rows through B0's or B1's (each 16-row load
    // lies within one of them: N0 is a multiple of 16); rows past the end reread the last valid row
    const int mrows = min(G2_T, M - m0);
    const __amdgpu_buffer_rsrc_t ra = g2_rsrc(A + (size_t)m0 * K, (uint32_t)((size_t)mrows * K * 2));
    const __amdgpu_buffer_rsrc_t rb0 = g2_rsrc(B0, (uint32_t)((size_t)N0 * K * 2));
    const __amdgpu_buffer_rsrc_t rb1 = g2_rsrc(N1 > 0 ? B1 : B0, (uint32_t)((size_t)(N1 > 0 ? N1 : N0) * K * 2));
    const int drow = lane >> 2, dpos = lane & 3;
    auto issue = [&](int buf, int step) {
        const int k0 = kbeg + min(step, nk - 1) * G2_KS;
        CSA_LDS char* lb = (CSA_LDS char*)g2_lds + buf * G2_BUF;
#pragma unroll
        for (int i = 0; i < G2_DMA; ++i) {                 // A rows 16 I .. 16 I + 15
            const int I = w + G2_NW * i, row = 16 * I + drow;
            const int r = min(row, mrows - 1);
            const uint32_t voff = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)(k0 + 8 * (dpos ^ ((row >> 2) & 3))) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (CSA_LDS void*)(lb + 1024 * I), 16, (int)voff, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < G2_DMA; ++i) {                 // B rows 16 I .. 16 I + 15 of the tile
            const int I = w + G2_NW * i, row = 16 * I + drow;
            const int nbase = n0 + 16 * I;
            const bool second = nbase >= N0 && nbase < N;           // uniform per load
            const int br = second ? min(n0 + row - N0, N1 - 1) : min(n0 + row, N0 - 1);
            const uint32_t voff = (uint32_t)br * (uint32_t)K * 2u + (uint32_t)(k0 + 8 * (dpos ^ ((row >> 2) & 3))) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rb1 : rb0, (CSA_LDS void*)(lb + G2_T * G2_ROWB + 1024 * I),
                                                     16, (int)voff, 0, 0, 0);
        }
    };
    f32x16_t acc[4][G2_WNB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < G2_WNB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // this lane's fragment offset within a buffer for row `row`, k sub-step s (logical chunk 2 s + lane/32)
    auto frag = [&](int row, int s) {
        return (uint32_t)row * G2_ROWB + 16u * (uint32_t)((2 * s + (lane >> 5)) ^ ((row >> 2) & 3));
    };
    const int r32 = lane & 31;
    auto read_frags = [&](int step, u32x4_t (&fa)[4][2], u32x4_t (&fb)[G2_WNB][2]) {
        const CSA_LDS char* lb = (const CSA_LDS char*)g2_lds + (step % G2_NB) * G2_BUF;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i][s2] = *(const CSA_LDS u32x4_t*)(lb + frag(wm + 32 * i + r32, s2));
#pragma unroll
            for (int j = 0; j < G2_WNB; ++j)
                fb[j][s2] = *(const CSA_LDS u32x4_t*)(lb + G2_T * G2_ROWB + frag(wn + 32 * j + r32, s2));
        }
    };
    auto mfmas = [&](const u32x4_t (&fa)[4][2], const u32x4_t (&fb)[G2_WNB][2], int s2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < G2_WNB; ++j)
                acc[i][j] = mfma32_bf16(as_bf16x8(fa[i][s2]), as_bf16x8(fb[j][s2]), acc[i][j]);
    };
    // Step t's fragments are read from LDS during step t - 1, between its two halves of MFMAs, so
    // that the LDS latency hides behind MFMAs.  The barrier in step t certifies step t + 1's tile
    // (each wave first waits for its own loads of it) and that every wave is done with step t - 1's
    // buffer, which then receives the loads of step t + NB - 1.
#pragma unroll
    for (int b = 0; b < G2_NB - 1; ++b) issue(b, b);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm2((G2_NB - 2) * 2 * G2_DMA));
    __syncthreads();
    u32x4_t ca[4][2], cb[G2_WNB][2];
    read_frags(0, ca, cb);
    for (int t = 0; t < nk; ++t) {
        mfmas(ca, cb, 0);
        u32x4_t na[4][2], nb[G2_WNB][2];
        if (t + 1 < nk) {                                  // uniform
            __builtin_amdgcn_s_waitcnt(vmcnt_imm2((G2_NB - 3) * 2 * G2_DMA));
            __syncthreads();
            issue((t + G2_NB - 1) % G2_NB, t + G2_NB - 1);
            read_frags(t + 1, na, nb);
        }
        mfmas(ca, cb, 1);
        if (t + 1 < nk) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) ca[i][s2] = na[i][s2];
#pragma unroll
                for (int j = 0; j < G2_WNB; ++j) cb[j][s2] = nb[j][s2];
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm2(0));             // the reread loads past the end land before exit
    // lane holds C[wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4][wn + 32 j + lane % 32]
    if (S > 1) {
        float* Pk = P + ((size_t)y * S + ks) * M * N;
#pragma unroll
        for (int j = 0; j < G2_WNB; ++j) {
            const int gj = n0 + wn + 32 * j + r32;
            if (n0 + wn + 32 * j >= N) continue;             // uniform: N0 and N1 are multiples of 32
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gi = m0 + wm + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
                    if (gi < M) Pk[(size_t)gi * N + gj] = acc[i][j][r];
                }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < G2_WNB; ++j) {
        const int gj = n0 + wn + 32 * j + r32;
        if (n0 + wn + 32 * j >= N) continue;                 // uniform: N0 and N1 are multiples of 32
        const bool second = n0 + wn + 32 * j >= N0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = m0 + wm + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
                if (gi >= M) continue;
                const float v = acc[i][j][r];
                if (!second) C0[(size_t)gi * N0 + gj] = f32_to_bf16(v);
                else if (C1_E4M3) ((uint8_t*)C1)[((size_t)y * M + gi) * N1 + gj - N0] = f32_to_e4m3(v);
                else ((uint16_t*)C1)[((size_t)y * M + gi) * N1 + gj - N0] = f32_to_bf16(v);
            }
    }
}

// Sum of the S split-K partials of k_gemm2 in split order, rounded to the outputs; one thread per
// four consecutive columns of a row.
template <int C1_E4M3>
__global__ __launch_bounds__(256) void k_g2reduce(const float* __restrict__ P, int S, int M, int N0, int N1,
                                                  uint16_t* __restrict__ C0, void* __restrict__ C1)
{
    const int N = N0 + N1, y = blockIdx.y;
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;   // quad index within the batch
    if (q >= (long long)M * N / 4) return;
    const int row = (int)(q / (N / 4)), col = (int)(q % (N / 4)) * 4;
    const float* p = P + (size_t)y * S * M * N + (size_t)row * N + col;
    f32x4_t a = *(const f32x4_t*)p;
    for (int k = 1; k < S; ++k) a += *(const f32x4_t*)(p + (size_t)k * M * N);
    const size_t orow = (size_t)y * M + row;
    if (col < N0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) C0[orow * N0 + col + e] = f32_to_bf16(a[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (C1_E4M3) ((uint8_t*)C1)[orow * N1 + col - N0 + e] = f32_to_e4m3(a[e]);
            else ((uint16_t*)C1)[orow * N1 + col - N0 + e] = f32_to_bf16(a[e]);
        }
    }
}

// K splits of a k_gemm2 launch: until the launch has two workgroups per CU, halve the K range
// while it keeps at least 256 (eight steps)
int g2_splits(int batch, int M, int N, int K) {
    const long long tiles = (long long)batch * ((M + G2_T - 1) / G2_T) * ((N + G2_T - 1) / G2_T);
    int S = 1;
    while (tiles * S < 512 && K % (2 * S * G2_KS) == 0 && K / (2 * S) >= 256) S *= 2;
    return S;
}

}  // namespace

namespace csa_host {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// pooled rows [B][Nc][Dh] bf16 | split-K partials of the pooled or the window projection (fp32)
// split-K partials (fp32) of the projections of one compression: pooled rows (D + dI outputs),
// window rows (D), and optionally a second pooled set (Nh rows, D outputs)
static size_t partial_floats(int B, long long L, int Dh, int D, int dI, int m, int W, long long Nh) {
    const long long Nc = (L + m - 1) / m;
    const int Np = D + dI;
    const int Sp = g2_splits(1, (int)(B * Nc), Np, Dh);
    const int Sw = (W > 0 && L >= W) ? g2_splits(B, W, D, Dh) : 1;
    const int Sh = Nh > 0 ? g2_splits(1, (int)(B * Nh), D, Dh) : 1;
    const size_t pp = Sp > 1 ? (size_t)Sp * B * Nc * Np : 0;
    const size_t pw = Sw > 1 ? (size_t)Sw * B * W * D : 0;
    const size_t ph = Sh > 1 ? (size_t)Sh * B * Nh * D : 0;
    return std::max(pp, std::max(pw, ph));
}

size_t compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W) {
    const long long Nc = (L + m - 1) / m;
    return align256((size_t)B * Nc * Dh * 2) + align256(partial_floats(B, L, Dh, D, dI, m, W, 0) * 4);
}

size_t hca_compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W, int mh) {
    const long long Nc = (L + m - 1) / m, Nh = (L + mh - 1) / mh;
    return align256((size_t)B * Nc * Dh * 2) + align256((size_t)B * Nh * Dh * 2) +
           align256(partial_floats(B, L, Dh, D, dI, m, W, Nh) * 4);
}

// one k_gemm2 launch (+ its reduction when the K range is split)
// (P holds pcap floats: the split count is lowered until its partial sums fit)
static int gemm2_launch(const uint16_t* A, long long a_bstride, int batch, int M, int K, const uint16_t* B0, int N0,
                        const uint16_t* B1, int N1, int c1_e4m3, uint16_t* C0, void* C1, float* P, size_t pcap,
                        hipStream_t st) {
    const int N = N0 + N1;
    int S = g2_splits(batch, M, N, K);
    while (S > 1 && (size_t)S * batch * M * N > pcap) S >>= 1;
    const int units = ((M + G2_T - 1) / G2_T) * ((N + G2_T - 1) / G2_T) * S;
    const dim3 grid((unsigned)((units + 7) / 8 * 8), (unsigned)batch);
    if (c1_e4m3)
        CSA_LAUNCH("k_gemm2", k_gemm2<1>, grid, dim3(64 * G2_NW), 0, st, A, a_bstride, M, K, B0, N0, B1, N1, C0, C1, S, P);
    else
        CSA_LAUNCH("k_gemm2", k_gemm2<0>, grid, dim3(64 * G2_NW), 0, st, A, a_bstride, M, K, B0, N0, B1, N1, C0, C1, S, P);
    if (S > 1) {
        const dim3 rg((unsigned)(((long long)M * N / 4 + 255) / 256), (unsigned)batch);
        if (c1_e4m3)
            CSA_LAUNCH("k_g2reduce", k_g2reduce<1>, rg, dim3(256), 0, st, P, S, M, N0, N1, C0, C1);
        else
            CSA_LAUNCH("k_g2reduce", k_g2reduce<0>, rg, dim3(256), 0, st, P, S, M, N0, N1, C0, C1);
    }
    return 0;
}

// The streaming pool kernel covers hidden sizes of 1024 .. 4096 in steps of 1024 (except 3072),
// fine blocks of m in {1, 2, 4} and coarse blocks that are a multiple of 16 (and of 4 m with both).
static bool pool2_fine_ok(int Dh, int m) {
    const int cpl = Dh / 512;
    return (m == 1 || m == 2 || m == 4) && m * cpl <= 32;
}
static bool pool2_dh_ok(int Dh) { return Dh == 1024 || Dh == 2048 || Dh == 4096; }

// pooled rows of fine blocks (m > 0) and / or coarse blocks (mc > 0) from one pass; returns -1 when
// the streaming kernel does not cover the shape
static int pool2_launch(const uint16_t* X, int B, long long L, int Dh, int m, const float* gate_f, const float* bslot_f,
                        uint16_t* out_f, int mc, const float* gate_c, const float* bslot_c, uint16_t* out_c,
                        hipStream_t st, int b0 = 0, int nb = -1) {
    if (nb < 0) nb = B - b0;
    if (!pool2_dh_ok(Dh)) return -1;
    if (m > 0 && !pool2_fine_ok(Dh, m)) return -1;
    if (mc > 0 && (mc % 16 != 0 || (m > 0 && (m != 4 || mc % (4 * m) != 0)))) return -1;
    if (m <= 0 && mc <= 0) return -1;
    const int S = mc > 0 ? mc : 128;
    const int G = m > 0 ? m : 4;
    const int Nf = m > 0 ? (int)((L + m - 1) / m) : 0;
    const int Ncc = mc > 0 ? (int)((L + mc - 1) / mc) : 0;
    const dim3 grid((unsigned)((L + S - 1) / S), (unsigned)nb);
    const int cpl = Dh / 512;
    const int mode = (m > 0 ? 1 : 0) | (mc > 0 ? 2 : 0);
#define CSA_POOL2(C, GG, MD)                                                                                    \
    if (cpl == C && G == GG && mode == MD) {                                                                    \
        CSA_LAUNCH("k_pool2", (k_pool2<C, GG, MD>), grid, dim3(256), 0, st, X, L, Dh, S, m, gate_f, bslot_f, Nf,  \
                   out_f, mc, gate_c, bslot_c, Ncc, out_c, b0);                                                 \
        return 0;                                                                                               \
    }
    CSA_POOL2(2, 1, 1) CSA_POOL2(2, 2, 1) CSA_POOL2(2, 4, 1) CSA_POOL2(4, 1, 1) CSA_POOL2(4, 2, 1) CSA_POOL2(4, 4, 1)
    CSA_POOL2(8, 1, 1) CSA_POOL2(8, 2, 1) CSA_POOL2(8, 4, 1)
    CSA_POOL2(2, 4, 2) CSA_POOL2(4, 4, 2) CSA_POOL2(8, 4, 2)
    CSA_POOL2(2, 4, 3) CSA_POOL2(4, 4, 3) CSA_POOL2(8, 4, 3)
#undef CSA_POOL2
    return -1;
}

// the block-per-entry pool kernel (any Dh, any m)
static int pool1_launch(const void* hidden, const float* w_gate, const float* b_slot, int B, long long L, int Dh, int m,
                        uint16_t* pooled, hipStream_t st) {
    const int Nc = (int)((L + m - 1) / m);
    const int cpt = (Dh / 8 + PTPB - 1) / PTPB;
    dim3 gp(Nc, B);
#define CSA_POOL(C)                                                                                    \
    if (cpt <= C) {                                                                                    \
        CSA_LAUNCH("k_pool", k_pool<C>, gp, dim3(PTPB), 0, st, (const uint16_t*)hidden, w_gate, b_slot, \
                   L, Dh, m, Nc, pooled);                                                             \
    } else
    CSA_POOL(1) CSA_POOL(2) CSA_POOL(4) CSA_POOL(8) { return fail(6, "compress: Dh = %d too large", Dh); }
#undef CSA_POOL
    return 0;
}

static int pool_launch(const void* hidden, const float* w_gate, const float* b_slot, int B, long long L, int Dh, int m,
                       uint16_t* pooled, hipStream_t st) {
    const bool fine = m <= 4;
    int rc = pool2_launch((const uint16_t*)hidden, B, L, Dh, fine ? m : 0, w_gate, b_slot, pooled, fine ? 0 : m,
                          w_gate, b_slot, pooled, st);
    if (rc < 0) rc = pool1_launch(hidden, w_gate, b_slot, B, L, Dh, m, pooled, st);
    return rc;
}

// projections of the pooled rows (KV and indexer keys in one launch) and of the window rows
static int project_launch(const void* hidden, const uint16_t* pooled, const void* w_kv, const void* w_ik, int B,
                          long long L, int Dh, int D, int dI, int Nc, int W, int ik_dtype, void* kv_out, void* ik_out,
                          void* win_out, float* partial, size_t pcap, hipStream_t st) {
    const int N1 = (w_ik && ik_out) ? dI : 0;
    int rc = gemm2_launch(pooled, 0, 1, B * Nc, Dh, (const uint16_t*)w_kv, D, (const uint16_t*)w_ik, N1,
                          N1 && ik_dtype == 1, (uint16_t*)kv_out, ik_out, partial, pcap, st);
    if (rc) return rc;
    if (win_out && W > 0) {
        if (L >= W) {
            // each sequence's last W hidden rows are contiguous: one batch of the GEMM per sequence
            rc = gemm2_launch((const uint16_t*)hidden + (size_t)(L - W) * Dh, L * Dh, B, W, Dh, (const uint16_t*)w_kv,
                              D, nullptr, 0, 0, (uint16_t*)win_out, nullptr, partial, pcap, st);
            if (rc) return rc;
        } else {
            ARows wa{1, (const uint16_t*)hidden, L, W};
            const int Mw = B * W;
            CSA_LAUNCH("k_gemm", k_gemm<0>, dim3((Mw + GT - 1) / GT, (D + GT - 1) / GT), dim3(GTPB), 0, st, wa,
                       (const uint16_t*)w_kv, Mw, D, Dh, win_out);
        }
    }
    return 0;
}

int compress_launch(const void* hidden, const void* w_kv, const void* w_ik, const float* w_gate,
                    const float* b_slot, int B, long long L, int Dh, int D, int dI, int m, int W,
                    int ik_dtype, void* kv_out, void* ik_out, void* win_out, void* ws, hipStream_t st) {
    const int Nc = (int)((L + m - 1) / m);
    uint16_t* pooled = (uint16_t*)ws;
    float* partial = (float*)((char*)ws + align256((size_t)B * Nc * Dh * 2));
    const size_t pcap = partial_floats(B, L, Dh, D, (w_ik && ik_out) ? dI : 0, m, win_out ? W : 0, 0);
    int rc = pool_launch(hidden, w_gate, b_slot, B, L, Dh, m, pooled, st);
    if (rc) return rc;
    return project_launch(hidden, pooled, w_kv, w_ik, B, L, Dh, D, dI, Nc, W, ik_dtype, kv_out, ik_out, win_out,
                          partial, pcap, st);
}

int hca_compress_launch(const void* hidden, const void* w_kv, const void* w_ik, const float* w_gate,
                        const float* b_slot, int B, long long L, int Dh, int D, int dI, int m, int W, int ik_dtype,
                        void* kv_out, void* ik_out, void* win_out, const void* w_kv_h, const float* w_gate_h,
                        const float* b_slot_h, int mh, void* kv_h_out, void* ws, hipStream_t st) {
    const int Nc = (int)((L + m - 1) / m), Nh = (int)((L + mh - 1) / mh);
    uint16_t* pooled = (uint16_t*)ws;
    uint16_t* pooled_h = (uint16_t*)((char*)ws + align256((size_t)B * Nc * Dh * 2));
    float* partial = (float*)((char*)pooled_h + align256((size_t)B * Nh * Dh * 2));
    const int N1 = (w_ik && ik_out) ? dI : 0;
    const size_t pcap = partial_floats(B, L, Dh, D, N1, m, win_out ? W : 0, Nh);
    // both pooled sets from one read of the hidden rows where the streaming kernel covers the shape
    int rc = pool2_launch((const uint16_t*)hidden, B, L, Dh, m, w_gate, b_slot, pooled, mh, w_gate_h, b_slot_h,
                          pooled_h, st);
    if (rc < 0) {
        rc = pool_launch(hidden, w_gate, b_slot, B, L, Dh, m, pooled, st);
        if (rc) return rc;
        rc = pool_launch(hidden, w_gate_h, b_slot_h, B, L, Dh, mh, pooled_h, st);
    }
    if (rc) return rc;
    rc = project_launch(hidden, pooled, w_kv, w_ik, B, L, Dh, D, dI, Nc, W, ik_dtype, kv_out, ik_out, win_out, partial,
                        pcap, st);
    if (rc) return rc;
    return gemm2_launch(pooled_h, 0, 1, B * Nh, Dh, (const uint16_t*)w_kv_h, D, nullptr, 0, 0, (uint16_t*)kv_h_out,
                        nullptr, partial, pcap, st);
}

}  // namespace csa_host

// lowp.hip -- the low-precision cache formats: FP8 KV rows with BF16 RoPE dimensions, and MXFP4 indexer
// operands.
//
// "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1 (last paragraph): the KV cache keeps
// the RoPE dimensions in BF16 and the others in FP8; "DeepSeek V4 详解", section "mHC、Muon、FP4：这些不是论文
// 装饰": the Lightning Indexer's QK path runs in FP4.  The pages fix no encoding; this library uses
//   * FP8 KV row (D + 80 bytes): OCP e4m3 codes of the first D - 64 dimensions in groups of 64, each group
//     divided by its smallest power-of-two scale 2^e with max|x| <= 448 * 2^e (exact division, no
//     saturation); the 64 RoPE dimensions as bf16; one byte e + 127 per group (16 bytes, unused ones 0);
//   * MXFP4 (the OCP Microscaling FP4 format): E2M1 codes, two per byte (element 2i in the low nibble), and
//     one E8M0 scale byte X + 127 per 32 elements with X = floor(log2 max|x|) - 2, codes rounded to nearest,
//     ties to the even code, saturating at 6.
// Both encoders are exact functions of the bf16 input (no accumulation), so they are bit-exact.
#include "common.h"
#include "kernels.h"

namespace {

using namespace csa;

// smallest e with a <= 448 * 2^e (a > 0, a bf16 value, so every step is exact in fp64)
__device__ __forceinline__ int fp8_group_exp(float a) {
    int k;
    (void)frexp((double)a, &k);                       // a in [2^(k-1), 2^k)
    return (double)a <= ldexp(448.0, k - 9) ? k - 9 : k - 8;   // 448 * 2^(k-9) = 0.875 * 2^k
}

// One lane per 16-byte chunk of a row (8 dims: D / 8 lanes per row, so a wave holds one row at D = 512 and
// four at D = 128, and every load and store is a vector access); the 8 lanes of a 64-dim group find its
// maximum by xor shuffles.  Lanes of one group always belong to one row, so a row past the end leaves whole
// groups idle.
__global__ __launch_bounds__(256) void k_kv_fp8(const uint16_t* __restrict__ x, long long n, int D,
                                                uint8_t* __restrict__ y)
{
    const int lpr = D / 8;
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long r = t / lpr;
    const int c = (int)(t - r * lpr), G = (D - 64) / 64;
    if (r >= n) return;
    const u32x4_t v = *(const u32x4_t*)(x + r * D + 8 * c);
    uint8_t* yr = y + r * (D + 80);
    if (c < 8 * G) {                                 // an e4m3 chunk of group c / 8
        float f[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = bf16_to_f32((uint16_t)(v[k] & 0xffffu));
            f[2 * k + 1] = bf16_to_f32((uint16_t)(v[k] >> 16));
        }
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
        const int e = a > 0.f ? fp8_group_exp(a) : 0;
        // exact scaling (a bf16 value times a power of two; what underflows fp32 lies far below e4m3's
        // smallest half-step and codes to a signed zero either way), |.| <= 448, then the hardware's
        // round-to-nearest-even conversion, two values at a time
        uint32_t w[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[4 * k], -e), ldexpf(f[4 * k + 1], -e), 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[4 * k + 2], -e), ldexpf(f[4 * k + 3], -e), pk, true);
            w[k] = (uint32_t)pk;
        }
        *(uint2*)(yr + 8 * c) = make_uint2(w[0], w[1]);
        if ((c & 7) == 0) yr[D + 64 + c / 8] = (uint8_t)(e + 127);
    } else {                                         // a RoPE chunk, kept as bf16
        *(u32x4_t*)(yr + (D - 64) + 16 * (c - 8 * G)) = v;
        if (c == 8 * G)
            for (int g = G; g < 16; ++g) yr[D + 64 + g] = 0;   // unused scale bytes
    }
}

// E2M1 code of v (|v| < 8 after scaling): the count of midpoints below |v|, a tie going up only to an even code
__device__ __forceinline__ uint32_t e2m1_code(float v) {
    const float a = fabsf(v);
    uint32_t k = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return (v < 0.f && k ? 8u : 0u) | k;
}

// One lane per 16-byte chunk (8 elements) of a row of len elements (len % 32 == 0): the 4 lanes of a 32-element
// block find its maximum by xor shuffles, and each lane writes its 8 codes as one dword.
__global__ __launch_bounds__(256) void k_mxfp4(const uint16_t* __restrict__ x, long long n, int len,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int lpr = len / 8;
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long r = t / lpr;
    const int c = (int)(t - r * lpr);
    if (r >= n) return;
    const u32x4_t v = *(const u32x4_t*)(x + r * len + 8 * c);
    float f[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = bf16_to_f32((uint16_t)(v[k] & 0xffffu));
        f[2 * k + 1] = bf16_to_f32((uint16_t)(v[k] >> 16));
    }
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(f[k]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    int X = -127;
    if (a > 0.f) {
        int k;
        (void)frexp((double)a, &k);
        X = min(127, max(-127, k - 1 - 2));
    }
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) w |= e2m1_code(ldexpf(f[k], -X)) << (4 * k);     // exact scaling
    *(uint32_t*)(codes + r * (len / 2) + 4 * c) = w;
    if ((c & 3) == 0) scales[r * (len / 32) + c / 4] = (uint8_t)(X + 127);
}

}  // namespace

namespace csa_host {

int kv_fp8_launch(const void* x, long long n, int D, void* y, hipStream_t st) {
    const long long threads = n * (D / 8);
    CSA_LAUNCH("k_kv_fp8", k_kv_fp8, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, (const uint16_t*)x, n,
               D, (uint8_t*)y);
    return 0;
}

int mxfp4_launch(const void* x, long long n, int len, void* codes, void* scales, hipStream_t st) {
    const long long threads = n * (len / 8);
    CSA_LAUNCH("k_mxfp4", k_mxfp4, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, (const uint16_t*)x, n,
               len, (uint8_t*)codes, (uint8_t*)scales);
    return 0;
}

}  // namespace csa_host

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

// One wave per row: lane j holds dimension 64 g + j of every group g.
__global__ __launch_bounds__(256) void k_kv_fp8(const uint16_t* __restrict__ x, long long n, int D,
                                                uint8_t* __restrict__ y)
{
    const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n) return;
    const int lane = threadIdx.x & 63, G = (D - 64) / 64, RB = D + 80;
    const uint16_t* xr = x + r * D;
    uint8_t* yr = y + r * RB;
    for (int g = 0; g < G; ++g) {
        const float v = bf16_to_f32(xr[64 * g + lane]);
        float a = fabsf(v);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
        const int e = a > 0.f ? fp8_group_exp(a) : 0;
        yr[64 * g + lane] = f32_to_e4m3((float)ldexp((double)v, -e));   // exact scaling, |.| <= 448
        if (lane == 0) yr[D + 64 + g] = (uint8_t)(e + 127);
    }
    if (lane < 8) *(u32x4_t*)(yr + (D - 64) + 16 * lane) = *(const u32x4_t*)(xr + (D - 64) + 8 * lane);
    if (lane >= G && lane < 16) yr[D + 64 + lane] = 0;
}

// E2M1 code of v (|v| < 8 after scaling): the count of midpoints below |v|, a tie going up only to an even code
__device__ __forceinline__ uint32_t e2m1_code(float v) {
    const float a = fabsf(v);
    uint32_t k = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return (v < 0.f && k ? 8u : 0u) | k;
}

// One wave per row of len elements (len % 32 == 0, len <= 4096): lane l owns the element pairs 2l + 128 i.
__global__ __launch_bounds__(256) void k_mxfp4(const uint16_t* __restrict__ x, long long n, int len,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n) return;
    const int lane = threadIdx.x & 63;
    const uint16_t* xr = x + r * len;
    for (int base = 0; base < len; base += 128) {
        const int i = base + 2 * lane;                 // the block of i is (i / 32): 16 lanes per block
        const bool act = i < len;
        const float v0 = act ? bf16_to_f32(xr[i]) : 0.f, v1 = act ? bf16_to_f32(xr[i + 1]) : 0.f;
        float a = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
        int X = -127;
        if (a > 0.f) {
            int k;
            (void)frexp((double)a, &k);
            X = min(127, max(-127, k - 1 - 2));
        }
        const uint32_t c = e2m1_code((float)ldexp((double)v0, -X)) | (e2m1_code((float)ldexp((double)v1, -X)) << 4);
        if (act) {
            codes[r * (len / 2) + i / 2] = (uint8_t)c;
            if ((lane & 15) == 0) scales[r * (len / 32) + i / 32] = (uint8_t)(X + 127);
        }
    }
}

}  // namespace

namespace csa_host {

int kv_fp8_launch(const void* x, long long n, int D, void* y, hipStream_t st) {
    CSA_LAUNCH("k_kv_fp8", k_kv_fp8, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, (const uint16_t*)x, n, D,
               (uint8_t*)y);
    return 0;
}

int mxfp4_launch(const void* x, long long n, int len, void* codes, void* scales, hipStream_t st) {
    CSA_LAUNCH("k_mxfp4", k_mxfp4, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, (const uint16_t*)x, n, len,
               (uint8_t*)codes, (uint8_t*)scales);
    return 0;
}

}  // namespace csa_host

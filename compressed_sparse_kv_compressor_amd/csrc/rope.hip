// Partial rotary position embedding (V4 technical summary, section 1.1 "hybrid attention"): the rotation
// acts on the last rd dimensions of a query / KV row only, and the attention output takes the inverse
// rotation at its query position.  Pair j = (D-rd+2j, D-rd+2j+1) turns by pos * theta^(-2j/rd) (the
// opposite angle for the inverse); the first D-rd dimensions pass through.
//
// HBM-bound elementwise work: one lane per 16-byte chunk (8 bf16) of a row, grid-stride over all chunks,
// so every wave reads and writes whole contiguous 1 KiB spans.  Angles are formed and reduced in fp64
// (positions reach 2^20 and more: an fp32 product pos * f would already be off by ~0.1 rad there): a lane's
// four frequencies are one fp64 exp2 and three steps of the ratio theta^(-2/rd), each angle is reduced
// modulo 2 pi with a two-term (Cody-Waite) constant, and only the reduced angle, in [-pi, pi], goes to an
// fp32 sincos; the rotation is fp32 and each output is rounded once to bf16.  In place (y == x) is allowed: a lane
// reads its chunk before it writes it and no lane touches another's.
#include "common.h"
#include "kernels.h"

using namespace csa;

namespace {

constexpr int RT = 256;
constexpr double TWO_PI_HI = 6.283185307179586;            // 2 pi rounded to double
constexpr double TWO_PI_LO = 2.4492935982947064e-16;       // 2 pi - TWO_PI_HI
constexpr double INV_TWO_PI = 0.15915494309189535;

__global__ __launch_bounds__(RT) void k_rope(const uint16_t* x, uint16_t* y, const long long* __restrict__ pos,
                                            long long n, int D, int rd, int group, double log2_theta,
                                            double ratio, int inverse)
{
    const int cpr = D / 8;
    const long long total = n * cpr;
    const int first = (D - rd) / 8;          // first rotated chunk of a row
    for (long long i = (long long)blockIdx.x * RT + threadIdx.x; i < total; i += (long long)gridDim.x * RT) {
        const long long r = i / cpr;
        const int c = (int)(i - r * cpr);
        uint4 v = *(const uint4*)(x + r * D + 8 * c);
        if (c >= first) {
            const double p = (double)pos[r / group];
            const double sp = inverse ? -p : p;
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
            double f = exp2(-2.0 * (4 * (c - first)) / rd * log2_theta);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const double a = sp * f;
                const double q = rint(a * INV_TWO_PI);
                const float r = (float)fma(-q, TWO_PI_LO, fma(-q, TWO_PI_HI, a));
                f *= ratio;
                float sf, cf;
                sincosf(r, &sf, &cf);
                const float u = bf16_to_f32((uint16_t)(w[k] & 0xffffu)), t = bf16_to_f32((uint16_t)(w[k] >> 16));
                w[k] = (uint32_t)f32_to_bf16(u * cf - t * sf) | ((uint32_t)f32_to_bf16(u * sf + t * cf) << 16);
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        *(uint4*)(y + r * D + 8 * c) = v;
    }
}

// D = 512, rd <= 128: a row is 64 chunks, so every wave of the grid-stride loop holds exactly one row (256 and
// the grid stride are multiples of 64, and the chunk count is too, so whole waves enter and leave the loop
// together).  Lane j forms pair j's angle once and the rotated lanes fetch their four (cos, sin) by shuffle:
// the angle work is spread over the wave instead of running on its last rd / 8 lanes only.
__global__ __launch_bounds__(RT) void k_rope512(const uint16_t* x, uint16_t* y, const long long* __restrict__ pos,
                                               long long n, int rd, int group, double log2_theta, int inverse)
{
    const int lane = threadIdx.x & 63;
    const int first = (512 - rd) / 8;
    const long long total = n * 64;
    for (long long i = (long long)blockIdx.x * RT + threadIdx.x; i < total; i += (long long)gridDim.x * RT) {
        const long long r = i >> 6;
        uint4 v = *(const uint4*)(x + r * 512 + 8 * lane);
        const double p = (double)pos[r / group];
        float sn, cs;
        rope_cs(inverse ? -p : p, lane < rd / 2 ? lane : 0, rd, log2_theta, cs, sn);
        const int src = lane >= first ? 4 * (lane - first) : 0;
        float sk[4], ck[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sk[k] = __shfl(sn, src + k);
            ck[k] = __shfl(cs, src + k);
        }
        if (lane >= first) {
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float u = bf16_to_f32((uint16_t)(w[k] & 0xffffu)), t = bf16_to_f32((uint16_t)(w[k] >> 16));
                w[k] = (uint32_t)f32_to_bf16(u * ck[k] - t * sk[k]) | ((uint32_t)f32_to_bf16(u * sk[k] + t * ck[k]) << 16);
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        *(uint4*)(y + r * 512 + 8 * lane) = v;
    }
}

}  // namespace

namespace csa_host {

int rope_launch(const void* x, void* y, const long long* pos, long long n, int D, int rd, int group, double theta,
                int inverse, hipStream_t st) {
    if (n == 0) return 0;
    const long long chunks = n * (D / 8);
    const long long blocks = (chunks + RT - 1) / RT;
    const int grid = (int)(blocks < 2048 ? blocks : 2048);
    if (D == 512 && rd <= 128) {
        CSA_LAUNCH("k_rope", k_rope512, dim3(grid), dim3(RT), 0, st, (const uint16_t*)x, (uint16_t*)y, pos, n, rd,
                   group, log2(theta), inverse);
        return 0;
    }
    CSA_LAUNCH("k_rope", k_rope, dim3(grid), dim3(RT), 0, st, (const uint16_t*)x, (uint16_t*)y, pos, n, D, rd,
               group, log2(theta), pow(theta, -2.0 / rd), inverse);
    return 0;
}

}  // namespace csa_host

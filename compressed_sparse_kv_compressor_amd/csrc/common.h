// common.h -- shared device/host helpers of libcsa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA bf16 operand (16 B)
typedef __attribute__((ext_vector_type(4))) float f32x4_t;      // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(16))) float f32x16_t;    // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) short i16x4_t;      // LDS transpose-read result
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;   // 16 raw bytes

#define CSA_LDS __attribute__((address_space(3)))

namespace csa {

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even fp32 -> bf16 (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Round-to-nearest-even fp32 -> OCP e4m3fn, saturating to +-448.
__device__ __forceinline__ uint8_t f32_to_e4m3(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t s = (u >> 24) & 0x80u;
    float a = fminf(fabsf(f), 448.0f);
    uint32_t au = __float_as_uint(a);
    int e = (int)(au >> 23) - 127;                 // unbiased exponent of |f|
    if (a < 0.0009765625f) {                       // < 2^-10: rounds to 0 (2^-10 is a tie -> even 0)
        return (uint8_t)s;
    }
    if (e < -6) {                                  // subnormal: quantum 2^-9
        float n = rintf(a * 512.0f);               // exact scaling; rintf = ties to even
        return (uint8_t)(s | (uint32_t)n);         // n in 0..8 (8 -> smallest normal 0x08)
    }
    // normal: keep 3 mantissa bits with RNE
    uint32_t mant = au & 0x7fffffu;
    uint32_t keep = mant >> 20, rest = mant & 0xfffffu;
    uint32_t code = (uint32_t)(e + 7) << 3 | keep;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1;   // may carry into exponent
    if (code > 0x7eu) code = 0x7eu;
    return (uint8_t)(s | code);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Order-preserving map of an fp32 to uint32 (larger float -> larger key); -0 maps like +0.
__host__ __device__ __forceinline__ uint32_t f32_key(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__host__ __device__ __forceinline__ float key_f32(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// ---------------------------------------------------------------------------
// paged caches
// ---------------------------------------------------------------------------
// With a block table, entry s of sequence b lives in physical row
// (table[b][s >> eshift] << eshift) | (s & (2^eshift - 1)) of a pool of nblocks pages of 2^eshift entries;
// page ids outside [0, nblocks) are clamped into it (wrong data, never an access out of bounds).  Without a
// table, entry s lives in row b * N + s of the batch-major array.
struct PageMap {
    const int32_t* table;     // [B][max_blocks] or null
    int max_blocks;
    int eshift;               // log2(entries per page)
    int nblocks;              // pages in the pool
};
__device__ __forceinline__ size_t entry_row(const PageMap& pm, int b, int N, int s) {
    if (!pm.table) return (size_t)b * N + s;
    uint32_t blk = (uint32_t)pm.table[(size_t)b * pm.max_blocks + (s >> pm.eshift)];
    blk = blk < (uint32_t)pm.nblocks ? blk : (uint32_t)pm.nblocks - 1u;
    return ((size_t)blk << pm.eshift) | (size_t)(s & ((1 << pm.eshift) - 1));
}

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ f32x4_t mfma16_bf16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32_bf16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Rotary embedding angle of pair j (of rd rotated dimensions) at position p: cos and sin of
// p * theta^(-2j/rd), the angle formed in fp64 (positions reach 2^20 and more) and reduced modulo 2 pi with a
// two-term (Cody-Waite) constant, then an fp32 sincos of the reduced angle.  log2_theta = log2(theta).
constexpr double ROPE_TWO_PI_HI = 6.283185307179586;          // 2 pi rounded to double
constexpr double ROPE_TWO_PI_LO = 2.4492935982947064e-16;     // 2 pi - ROPE_TWO_PI_HI
constexpr double ROPE_INV_TWO_PI = 0.15915494309189535;
__device__ __forceinline__ void rope_cs(double p, int j, int rd, double log2_theta, float& c, float& s) {
    const double a = p * exp2(-2.0 * j / rd * log2_theta);
    const double q = rint(a * ROPE_INV_TWO_PI);
    sincosf((float)fma(-q, ROPE_TWO_PI_LO, fma(-q, ROPE_TWO_PI_HI, a)), &s, &c);
}

}  // namespace csa

// ---------------------------------------------------------------------------
// Host side: launch bookkeeping shared by all translation units.
// ---------------------------------------------------------------------------
namespace csa_host {
// Record a kernel launch window for the optional timing registry (no-op when disabled).
void* prof_begin(const char* name, hipStream_t s);
void prof_end(void* token, hipStream_t s);
// Set the thread-local error text; returns `code`.
int fail(int code, const char* fmt, ...);
}  // namespace csa_host

#define CSA_LAUNCH(name, kernel, grid, block, lds, stream, ...)                        \
    do {                                                                               \
        void* _tok = csa_host::prof_begin(name, stream);                               \
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);             \
        hipError_t _e = hipGetLastError();                                             \
        csa_host::prof_end(_tok, stream);                                              \
        if (_e != hipSuccess)                                                          \
            return csa_host::fail(7, "launch of %s failed: %s", name, hipGetErrorString(_e)); \
    } while (0)

// attn_common.h -- row sets, job records and tile constants shared by the MQA attention kernels.
//
// Method: "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1 (CSA attends to the
// selected compressed entries plus a window of raw tokens; HCA attends to every compressed entry).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace csa_attn {

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
    const float* sink;        // [H] attention-sink logits (natural log) or null
};

__device__ __forceinline__ int dense_visible(long long p, long long L, int m, int N) {
    if (p >= L - 1) return N;
    long long v = (p + 1) / m;
    return v < N ? (int)v : N;
}

// Final normalization of one head.  The rows give (m, l) in the log2 domain (m = -inf, l = 0: no row) and
// value sums O relative to 2^m; s2 is the head's attention-sink logit in log2 units (-inf: none), one more
// denominator term with no value row.  Returns f with out = O f and sets the natural-log lse; without a
// sink this is f = 1 / l, lse = (m + log2 l) ln 2 exactly.
__device__ __forceinline__ float sink_norm(float m, float l, float s2, float& lse_out) {
    const float M = fmaxf(m, s2);
    if (!(M > -INFINITY)) {
        lse_out = -INFINITY;
        return 0.f;
    }
    const float a = m > -INFINITY ? exp2f(m - M) : 0.f;
    const float lt = l * a + exp2f(s2 - M);
    lse_out = (M + log2f(lt)) * LN2;
    return lt > 0.f ? a / lt : 0.f;
}
__device__ __forceinline__ float sink_log2(const float* sink, int h) {
    return sink ? sink[h] * LOG2E : -INFINITY;
}

// 16-byte chunk c of row r is stored at chunk c ^ f(r & 15), f(x) = 4 (x & 3) + (x >> 2): any 16
// consecutive rows at one chunk, and any 4 aligned rows x 4 aligned chunks (the footprint of a
// transposed read), fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz_chunk(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Raw buffer resource (stride 0, byte offsets) over [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Masked rows get -2^100 added to their scores by one extra MFMA k-step (A: a 1 in column 0 of each
// masked row; B: -2^100 in row 0 of one k-step of the contraction), which sends their probabilities to exactly 0
// without any per-element select on the common path.  A split with no valid row at all ends with a
// running max below EMPTY_M, which the output step treats as empty.
constexpr uint32_t BF16_ONE = 0x3f80u, BF16_NEG_2P100 = 0xf180u;
constexpr float EMPTY_M = -1.0e25f;

// One attention problem (the parameters of one launch).
struct AttnJob {
    const uint16_t* q;
    Rows R;
    int Tq, H;
    long long pos0;
    float scale_log2;
    int nunits, nsplit, rps;
    float* part_o;
    float2* part_ml;
    uint16_t* out;
    float* lse;
};

}  // namespace csa_attn

namespace csa_host {
// k_attn128 (attn128.hip): D = 512, H % 128 == 0, every array within reach of 32-bit byte offsets.
// Rows per split must be a multiple of ATT128_UNIT and at most ATT128_MAX_RPS.
constexpr int ATT128_UNIT = 128, ATT128_MAX_RPS = 2048;
// Launches the attention and, for a job with more than one split, the merge of the split partials
// (part_o then holds fp16 partials, half the bytes of the fp32 ones of k_attn64; part_ml as there).
int attn128_launch(const csa_attn::AttnJob& j, hipStream_t st, const char* tag);
}  // namespace csa_host

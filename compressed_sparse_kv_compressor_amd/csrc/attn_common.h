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
    const long long* seq_lens;  // [B] raw tokens per sequence (variable-length batch) or null
    csa::PageMap pm;          // entries through a block table (pm.table null: batch-major [B][N][D])
    const uint16_t* v;        // values of the entries when they differ from the keys (kv), or null
    const uint16_t* v_raw;    // values of the raw rows when they differ from kv_raw, or null
    int kv_fp8;               // entry rows (kv, v) in the FP8 format (D + 80 bytes: e4m3 groups + bf16 RoPE dims)
    int rope_rd;              // fused rotary embedding of the last rope_rd dims (0: none; a multiple of 8)
    double rope_l2t;          // log2 of its base theta
};

constexpr int ROPE_FUSED_RD = 64;         // the fused rotation covers the last 64 dims (the pages' RoPE width)
// Fused partial rotary embedding: the query's last rd dimensions turn by +p before the scores (rounded to
// bf16 as the MFMA operand, as the separate rotary kernel rounds them) and the output's by -p after the
// softmax (in fp32, before its single bf16 rounding).  Pairs (2i, 2i+1) of a row's dims.
// Eight consecutive bf16 dims d0 .. d0 + 7 (d0 a multiple of 8) of a row of width D, turned by angle sign * p.
__device__ __forceinline__ u32x4_t rope8(u32x4_t v, int d0, int D, const Rows& R, double sp) {
    if (R.rope_rd == 0 || d0 < D - R.rope_rd) return v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float c, s;
        csa::rope_cs(sp, (d0 - (D - R.rope_rd)) / 2 + k, R.rope_rd, R.rope_l2t, c, s);
        const float u = csa::bf16_to_f32((uint16_t)(v[k] & 0xffffu)), t = csa::bf16_to_f32((uint16_t)(v[k] >> 16));
        v[k] = (uint32_t)csa::f32_to_bf16(u * c - t * s) | ((uint32_t)csa::f32_to_bf16(u * s + t * c) << 16);
    }
    return v;
}
// One fp32 pair (x at even dim d, y at d + 1) turned by angle sign * p; CSA_ROPE_PAIR updates two elements
// of a vector value in place.
__device__ __forceinline__ float2 rope2(float x, float y, int d, int D, const Rows& R, double sp) {
    if (R.rope_rd == 0 || d < D - R.rope_rd) return make_float2(x, y);
    float c, s;
    csa::rope_cs(sp, (d - (D - R.rope_rd)) / 2, R.rope_rd, R.rope_l2t, c, s);
    return make_float2(x * c - y * s, x * s + y * c);
}
#define CSA_ROPE_PAIR(V, I, J, DIM, DD, RR, SP)                  \
    {                                                          \
        const float2 rp_ = rope2((V)[I], (V)[J], DIM, DD, RR, SP); \
        (V)[I] = rp_.x;                                        \
        (V)[J] = rp_.y;                                        \
    }

__device__ __forceinline__ int dense_visible(long long p, long long L, int m, int N) {
    if (p >= L - 1) return N;
    long long v = (p + 1) / m;
    return v < N ? (int)v : N;
}

// Positions of query t of sequence b.  Variable-length batch: sequence b holds Lb = seq_lens[b] raw tokens
// (clamped to [Tq, L] for the dense rows, whose array holds ceil(L / ratio) entries), its queries are its
// last Tq tokens and its Lr raw rows its last Lr tokens; otherwise Lb = L, p = pos0 + t, raw rows start at
// raw0.  Returns p; sets Lb, the raw position of raw row 0, and the dense row count visible to p.
__device__ __forceinline__ long long row_geo(const Rows& R, int b, int t, int Tq, long long pos0, long long& raw0,
                                             int& ndense) {
    long long Lb = R.L, p = pos0 + t;
    raw0 = R.raw0;
    if (R.seq_lens) {
        const long long x = R.seq_lens[b], hi = R.mode == 0 ? R.L : (1LL << 62);
        Lb = x < Tq ? Tq : (x > hi ? hi : x);
        p = Lb - Tq + t;
        raw0 = Lb - R.Lr;
    }
    ndense = R.mode == 0 ? dense_visible(p, Lb, R.ratio, (int)((Lb + R.ratio - 1) / R.ratio)) : 0;
    return p;
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

// Merge jobs laid out by XCD: workgroup i runs on XCD i mod 8 and takes job lo[x] + i / 8 of the jobs
// [lo[x], lo[x + 1]) whose query's split partials were written on XCD x (jobs in query-major order, so the
// ranges are contiguous).  xcd_jobs builds the table from G groups of jpg jobs and the home XCD of each group
// (non-decreasing in the group).
struct XcdJobs { int lo[9]; };
template <class Home>
inline XcdJobs xcd_jobs(int G, int jpg, Home home, int* most) {
    XcdJobs xj;
    int x = 0;
    xj.lo[0] = 0;
    for (int g = 0; g < G; ++g) {
        const int h = home(g);
        while (x < h && x < 8) xj.lo[++x] = g * jpg;
    }
    while (x < 8) xj.lo[++x] = G * jpg;
    *most = 0;
    for (int k = 0; k < 8; ++k) *most = xj.lo[k + 1] - xj.lo[k] > *most ? xj.lo[k + 1] - xj.lo[k] : *most;
    return xj;
}

}  // namespace csa_attn

namespace csa_host {
// k_attn128 (attn128.hip): D = 512, H % 128 == 0, every array within reach of 32-bit byte offsets.
// Rows per split must be a multiple of ATT128_UNIT and at most ATT128_MAX_RPS.
constexpr int ATT128_UNIT = 32, ATT128_MAX_RPS = 2048;
// Launches the attention and, for a job with more than one split, the merge of the split partials
// (part_o then holds fp16 partials, half the bytes of the fp32 ones of k_attn64; part_ml as there).
int attn128_launch(const csa_attn::AttnJob& j, hipStream_t st, const char* tag);
}  // namespace csa_host

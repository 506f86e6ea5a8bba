// append.hip -- incremental compression during decode: the per-request state cache.
//
// "DeepSeek V4 详解", section "第二刀：KV cache 被当成系统在管": the compressed entries live in a classical
// cache while every request also keeps a small state of fixed size -- the raw tokens of its sliding window
// and the tail tokens that have not yet filled a compression block.  Here a decode step appends T new
// tokens per sequence:
//   * k_app_proj projects each new token once: its KV row (CSA ratio m, which is also the window row),
//     its indexer key, its HCA row, and its two gate logits ("DeepSeek-V4 技术解析" section 1.1: the
//     token-level compressor merges every m tokens' KV into one entry; the gate is this library's pooling
//     weight, a softmax over the block);
//   * k_app_state folds the tokens, in order, into the running softmax-gated pools of the open CSA and HCA
//     blocks (running maximum M, sum S of exp(z - M), weighted sums A of the projected rows), rewrites
//     the entries of the blocks it touched as A / S rounded once, shifts the window by T rows, and
//     advances the sequence's length.
// The caches therefore always hold ceil(L/m) and ceil(L/m') entries, the last ones pooled over the tokens
// of the open block so far, which is what compressing the whole prefix gives (up to the order of the
// fp32 sums).
#include "common.h"
#include "kernels.h"

namespace {

using namespace csa;

constexpr int AP_TPB = 256;                  // k_app_proj: 4 waves, one output column each
constexpr int AP_ROWS = 8;                   // token rows per workgroup
constexpr int AP_CHUNK = 4096;               // hidden elements staged in LDS per pass
constexpr int AS_TPB = 1024;                 // k_app_state: one workgroup per sequence
constexpr int AS_COLS = 2;                   // state columns per thread (D + dI + D <= 2 * 1024)

// Y[r][c] for the token rows r of this workgroup, c = wave's column: 0..D-1 CSA KV (w_kv), D..D+dI-1 indexer
// key (w_ik), D+dI..2D+dI-1 HCA KV (w_kvh), then the CSA and the HCA gate logits (fp32 weights).  fp32
// accumulation of the exact bf16 products, one wave reduction per row.
__global__ __launch_bounds__(AP_TPB) void k_app_proj(
    const uint16_t* __restrict__ X, int R, int Dh, const uint16_t* __restrict__ w_kv,
    const uint16_t* __restrict__ w_ik, const uint16_t* __restrict__ w_kvh, const float* __restrict__ g_c,
    const float* __restrict__ g_h, int D, int dI, float* __restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[AP_ROWS * AP_CHUNK];
    const int ncol = 2 * D + dI + 2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = blockIdx.x * (AP_TPB / 64) + wave;
    const int r0 = blockIdx.y * AP_ROWS;
    const int nr = min(AP_ROWS, R - r0);
    const uint16_t* wrow = nullptr;
    const float* grow = nullptr;
    if (col < D) wrow = w_kv + (size_t)col * Dh;
    else if (col < D + dI) wrow = w_ik + (size_t)(col - D) * Dh;
    else if (col < 2 * D + dI) wrow = w_kvh + (size_t)(col - D - dI) * Dh;
    else if (col == ncol - 2) grow = g_c;
    else if (col == ncol - 1) grow = g_h;
    float acc[AP_ROWS];
#pragma unroll
    for (int r = 0; r < AP_ROWS; ++r) acc[r] = 0.f;
    for (int k0 = 0; k0 < Dh; k0 += AP_CHUNK) {
        const int kn = min(AP_CHUNK, Dh - k0);            // a multiple of 64
        __syncthreads();
        for (int c = threadIdx.x; c < nr * (kn / 8); c += AP_TPB) {
            const int r = c / (kn / 8), cc = c % (kn / 8);
            *(u32x4_t*)(xs + r * AP_CHUNK + cc * 8) = *(const u32x4_t*)(X + (size_t)(r0 + r) * Dh + k0 + cc * 8);
        }
        __syncthreads();
        if (col >= ncol) continue;
        for (int i = lane * 8; i < kn; i += 512) {
            float wv[8];
            if (wrow) {
                const u32x4_t w = *(const u32x4_t*)(wrow + k0 + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wv[2 * e] = __uint_as_float(w[e] << 16);
                    wv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                }
            } else {
                const f32x4_t a = *(const f32x4_t*)(grow + k0 + i), c2 = *(const f32x4_t*)(grow + k0 + i + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { wv[e] = a[e]; wv[4 + e] = c2[e]; }
            }
#pragma unroll
            for (int r = 0; r < AP_ROWS; ++r) {
                if (r < nr) {
                    const u32x4_t x = *(const u32x4_t*)(xs + r * AP_CHUNK + i);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[r] = fmaf(wv[2 * e], __uint_as_float(x[e] << 16), acc[r]);
                        acc[r] = fmaf(wv[2 * e + 1], __uint_as_float(x[e] & 0xffff0000u), acc[r]);
                    }
                }
            }
        }
    }
    if (col >= ncol) return;
#pragma unroll
    for (int r = 0; r < AP_ROWS; ++r) {
        float v = acc[r];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0 && r < nr) Y[(size_t)(r0 + r) * ncol + col] = v;
    }
}

// One workgroup per sequence.  State layout (fp32): [M_c, S_c, M_h, S_h, A_c[D + dI], A_h[D]] (running
// maximum and sum of the open CSA / HCA block's gate exponentials, and its weighted row sums).
__global__ __launch_bounds__(AS_TPB) void k_app_state(
    const float* __restrict__ Y, int T, long long* __restrict__ seq_lens, long long L, const float* __restrict__ b_slot,
    const float* __restrict__ b_slot_h, int D, int dI, int m, int mh, int ik_dtype, float* __restrict__ state,
    int state_words, uint16_t* __restrict__ kv, void* __restrict__ ik, uint16_t* __restrict__ kvh, int Nc, int Nh,
    PageMap pm_c, PageMap pm_h, uint16_t* __restrict__ win, int W)
{
    __shared__ long long sp0;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int ncol = 2 * D + dI + 2;
    if (tid == 0) sp0 = seq_lens[b];
    __syncthreads();
    const long long p0 = sp0 < 0 ? 0 : (sp0 > L ? L : sp0);
    const int Tn = (int)min((long long)T, L - p0);        // tokens beyond the capacity are dropped
    float* st = state + (size_t)b * state_words;
    float Mc = st[0], Sc = st[1], Mh = st[2], Sh = st[3];
    float A[AS_COLS];
#pragma unroll
    for (int k = 0; k < AS_COLS; ++k) {
        const int c = tid + k * AS_TPB;
        A[k] = c < 2 * D + dI ? st[4 + c] : 0.f;
    }
    for (int t = 0; t < Tn; ++t) {
        const long long p = p0 + t;
        const float* y = Y + ((size_t)b * T + t) * ncol;
        // CSA block: slot p mod m (a new block restarts the pool)
        const int sc = (int)(p % m), sh = (int)(p % mh);
        const float zc = y[ncol - 2] + (b_slot ? b_slot[sc] : 0.f);
        const float zh = y[ncol - 1] + (b_slot_h ? b_slot_h[sh] : 0.f);
        float fc_old, fc_new, fh_old, fh_new;
        if (sc == 0) { Mc = zc; Sc = 1.f; fc_old = 0.f; fc_new = 1.f; }
        else {
            const float Mn = fmaxf(Mc, zc);
            fc_old = expf(Mc - Mn);
            fc_new = expf(zc - Mn);
            Sc = Sc * fc_old + fc_new;
            Mc = Mn;
        }
        if (sh == 0) { Mh = zh; Sh = 1.f; fh_old = 0.f; fh_new = 1.f; }
        else {
            const float Mn = fmaxf(Mh, zh);
            fh_old = expf(Mh - Mn);
            fh_new = expf(zh - Mn);
            Sh = Sh * fh_old + fh_new;
            Mh = Mn;
        }
        // the entry of a block is written when the block closes or at the chunk's last token
        const bool wc = sc == m - 1 || t == Tn - 1 || p == L - 1;
        const bool wh = sh == mh - 1 || t == Tn - 1 || p == L - 1;
        const int jc = (int)(p / m), jh = (int)(p / mh);
#pragma unroll
        for (int k = 0; k < AS_COLS; ++k) {
            const int c = tid + k * AS_TPB;
            if (c < D + dI) {
                A[k] = A[k] * fc_old + fc_new * y[c];
                if (wc) {
                    const float v = A[k] / Sc;
                    const size_t row = entry_row(pm_c, b, Nc, jc);
                    if (c < D) kv[row * D + c] = f32_to_bf16(v);
                    else if (ik_dtype == 0) ((uint16_t*)ik)[row * dI + (c - D)] = f32_to_bf16(v);
                    else ((uint8_t*)ik)[row * dI + (c - D)] = f32_to_e4m3(v);
                }
            } else if (c < 2 * D + dI) {
                A[k] = A[k] * fh_old + fh_new * y[c];
                if (wh) kvh[entry_row(pm_h, b, Nh, jh) * D + (c - D - dI)] = f32_to_bf16(A[k] / Sh);
            }
        }
    }
    // the window: row i holds raw position p0 + Tn - W + i; rows of old positions move down by Tn (read in
    // groups in increasing row order, each group before it is overwritten: the source rows lie Tn rows
    // further on), new positions take the projected KV rows
    if (W > 0 && Tn > 0) {
        uint16_t* wb = win + (size_t)b * W * D;
        const int cpr = D / 8;                              // 16-byte chunks per row
        const int per = AS_TPB / cpr;                       // rows per group
        for (int i0 = 0; i0 < W; i0 += per) {
            const int i = i0 + tid / cpr, cc = tid % cpr;
            u32x4_t v = u32x4_t{0, 0, 0, 0};
            const bool act = tid < per * cpr && i < W;
            if (act) {
                const long long u = p0 + Tn - W + i;
                if (u >= p0) {
                    const float* y = Y + ((size_t)b * T + (int)(u - p0)) * ncol + cc * 8;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
                } else {
                    v = *(const u32x4_t*)(wb + (size_t)(i + Tn) * D + cc * 8);
                }
            }
            __syncthreads();
            if (act) *(u32x4_t*)(wb + (size_t)i * D + cc * 8) = v;
            __syncthreads();
        }
    }
    if (tid == 0) {
        st[0] = Mc; st[1] = Sc; st[2] = Mh; st[3] = Sh;
        seq_lens[b] = p0 + Tn;
    }
#pragma unroll
    for (int k = 0; k < AS_COLS; ++k) {
        const int c = tid + k * AS_TPB;
        if (c < 2 * D + dI) st[4 + c] = A[k];
    }
}

}  // namespace

namespace csa_host {

size_t append_state_words(int D, int dI) { return ((size_t)(4 + 2 * D + dI) + 3) / 4 * 4; }

size_t append_ws_bytes(int B, int T, int D, int dI) {
    return ((size_t)B * T * (2 * D + dI + 2) * 4 + 255) / 256 * 256;
}

int append_launch(const void* hidden, int B, int T, int Dh, const void* w_kv, const void* w_ik, const float* w_gate,
                  const float* b_slot, int D, int dI, int m, int ik_dtype, const void* w_kv_h, const float* w_gate_h,
                  const float* b_slot_h, int mh, long long L, long long* seq_lens, void* state, void* kv, void* ik,
                  void* kv_h, void* win, int W, const CacheLayout& lay, void* ws, hipStream_t st) {
    const int R = B * T, ncol = 2 * D + dI + 2;
    float* Y = (float*)ws;
    CSA_LAUNCH("k_app_proj", k_app_proj, dim3((ncol + 3) / 4, (R + AP_ROWS - 1) / AP_ROWS), dim3(AP_TPB), 0, st,
               (const uint16_t*)hidden, R, Dh, (const uint16_t*)w_kv, (const uint16_t*)w_ik,
               (const uint16_t*)w_kv_h, w_gate, w_gate_h, D, dI, Y);
    const int Nc = (int)((L + m - 1) / m), Nh = (int)((L + mh - 1) / mh);
    CSA_LAUNCH("k_app_state", k_app_state, dim3(B), dim3(AS_TPB), 0, st, Y, T, seq_lens, L, b_slot, b_slot_h, D, dI, m,
               mh, ik_dtype, (float*)state, (int)append_state_words(D, dI), (uint16_t*)kv, ik, (uint16_t*)kv_h, Nc, Nh,
               page_map(lay, m), page_map(lay, mh), (uint16_t*)win, W);
    return 0;
}

}  // namespace csa_host

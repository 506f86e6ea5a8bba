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

constexpr int AP_WAVES = 8;                  // k_app_proj: the K range of a 16 x 16 tile split over 8 waves
constexpr int AP_KS = 4;                     // k_app_proj: and over 4 workgroups (partial sums, added in order)
constexpr int AS_TPB = 1024;                 // k_app_state: one workgroup per sequence
constexpr int AS_COLS = 2;                   // state columns per thread (D + dI + D <= 2 * 1024)

// Y[k][r][c], the partial sum over the k-th quarter of the hidden dimension, for the new tokens' rows r:
// c = 0..D-1 CSA KV (w_kv), D..D+dI-1 indexer key (w_ik), D+dI..2D+dI-1 HCA KV (w_kvh), then the CSA and
// the HCA gate logits (fp32 weights).  A 1-D grid of (row block of 16) x (column block of 16, plus one
// block for the two gate columns) x (quarter k).  A column block is one 16 x 16 output tile of
// v_mfma_f32_16x16x32_bf16 (A: 16 weight rows, B: 16 token rows, fp32 accumulation of the exact bf16
// products); its 8 waves take every 8th 32-wide step of the quarter and their partial tiles are added in
// wave order through LDS.  The gate block computes its 2 x 16 dot products with fp32 FMAs.  k_app_state
// adds the four quarters in order.
__global__ __launch_bounds__(64 * AP_WAVES) void k_app_proj(
    const uint16_t* __restrict__ X, int R, int Dh, const uint16_t* __restrict__ w_kv,
    const uint16_t* __restrict__ w_ik, const uint16_t* __restrict__ w_kvh, const float* __restrict__ g_c,
    const float* __restrict__ g_h, int D, int dI, float* __restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) f32x4_t red[AP_WAVES][64];
    const int ncol = 2 * D + dI + 2, ncb = (2 * D + dI) / 16;
    const int ks = blockIdx.x % AP_KS, cb = (blockIdx.x / AP_KS) % (ncb + 1);
    const int r0 = (blockIdx.x / AP_KS / (ncb + 1)) * 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lq = lane >> 4;
    const int NS = Dh / 32, s_lo = ks * NS / AP_KS, s_hi = (ks + 1) * NS / AP_KS;   // this quarter's steps
    Y += (size_t)ks * R * ncol;
    if (cb < ncb) {
        const int col = cb * 16 + li;          // this lane's weight row (A operand row li)
        const uint16_t* wrow = col < D ? w_kv + (size_t)col * Dh
                             : col < D + dI ? w_ik + (size_t)(col - D) * Dh : w_kvh + (size_t)(col - D - dI) * Dh;
        const bool rv = r0 + li < R;           // this lane's token row (B operand column li)
        const uint16_t* xrow = X + (size_t)(rv ? r0 + li : 0) * Dh;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        constexpr int U = 8;
        int s = s_lo + wave;
        for (; s + (U - 1) * AP_WAVES < s_hi; s += U * AP_WAVES) {    // U steps' loads in flight
            u32x4_t wa[U], xa[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = 32 * (s + u * AP_WAVES) + 8 * lq;
                wa[u] = *(const u32x4_t*)(wrow + k);
                xa[u] = rv ? *(const u32x4_t*)(xrow + k) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc = mfma16_bf16(as_bf16x8(wa[u]), as_bf16x8(xa[u]), acc);
        }
        for (; s < s_hi; s += AP_WAVES) {
            const int k = 32 * s + 8 * lq;
            const u32x4_t wa = *(const u32x4_t*)(wrow + k);
            const u32x4_t xa = rv ? *(const u32x4_t*)(xrow + k) : u32x4_t{0u, 0u, 0u, 0u};
            acc = mfma16_bf16(as_bf16x8(wa), as_bf16x8(xa), acc);
        }
        red[wave][lane] = acc;
        __syncthreads();
        // element (column 4 q + i, row j) of the tile sits in lane 16 q + j, entry i, of every wave
        const int t = threadIdx.x;
        if (t < 256) {
            const int q = t >> 6, j = (t >> 2) & 15, i = t & 3;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < AP_WAVES; ++w) v += red[w][16 * q + j][i];
            if (r0 + j < R) Y[(size_t)(r0 + j) * ncol + cb * 16 + 4 * q + i] = v;
        }
    } else {
        // the two gate columns: pair p = (column p & 1, row p >> 1) per wave, lanes stride the hidden dim
        for (int p = wave; p < 32; p += AP_WAVES) {
            const int c = p & 1, r = r0 + (p >> 1);
            if (r >= R) continue;
            const float* g = c == 0 ? g_c : g_h;
            const uint16_t* x = X + (size_t)r * Dh;
            float a = 0.f;
            for (int k = 32 * s_lo + 8 * lane; k < 32 * s_hi; k += 512) {
                const u32x4_t xv = *(const u32x4_t*)(x + k);
                const f32x4_t g0 = *(const f32x4_t*)(g + k), g1 = *(const f32x4_t*)(g + k + 4);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    a = fmaf(e ? g1[0] : g0[0], __uint_as_float(xv[2 * e] << 16), a);
                    a = fmaf(e ? g1[1] : g0[1], __uint_as_float(xv[2 * e] & 0xffff0000u), a);
                    a = fmaf(e ? g1[2] : g0[2], __uint_as_float(xv[2 * e + 1] << 16), a);
                    a = fmaf(e ? g1[3] : g0[3], __uint_as_float(xv[2 * e + 1] & 0xffff0000u), a);
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
            if (lane == 0) Y[(size_t)r * ncol + ncol - 2 + c] = a;
        }
    }
}

// One workgroup per sequence.  State layout (fp32): [M_c, S_c, M_h, S_h, A_c[D + dI], A_h[D]] (running
// maximum and sum of the open CSA / HCA block's gate exponentials, and its weighted row sums).  Y holds the
// AP_KS partial projections [k][B * T][ncol], added in order k = 0, 1, ...
__global__ __launch_bounds__(AS_TPB) void k_app_state(
    const float* __restrict__ Y, int T, long long* __restrict__ seq_lens, long long L, const float* __restrict__ b_slot,
    const float* __restrict__ b_slot_h, int D, int dI, int m, int mh, int ik_dtype, float* __restrict__ state,
    int state_words, uint16_t* __restrict__ kv, void* __restrict__ ik, uint16_t* __restrict__ kvh, int Nc, int Nh,
    PageMap pm_c, PageMap pm_h, uint16_t* __restrict__ win, int W)
{
    const int b = blockIdx.x, tid = threadIdx.x;
    const int ncol = 2 * D + dI + 2;
    const size_t kstride = (size_t)gridDim.x * T * ncol;   // between the partial sums (gridDim.x = B)
    auto yv = [&](int t, int c) -> float {                 // projection c of the sequence's new token t
        const float* y = Y + ((size_t)b * T + t) * ncol + c;
        float v = y[0];
#pragma unroll
        for (int k = 1; k < AP_KS; ++k) v += y[k * kstride];
        return v;
    };
    // every thread reads the length (a barrier below orders these reads before thread 0 advances it); the
    // first token's projections and gate logits are loaded at once too (T >= 1), before the length is known
    const long long sp0 = seq_lens[b];
    float y0[AS_COLS];
#pragma unroll
    for (int k = 0; k < AS_COLS; ++k) {
        const int c = tid + k * AS_TPB;
        y0[k] = c < 2 * D + dI ? yv(0, c) : 0.f;
    }
    const float zc0 = yv(0, ncol - 2), zh0 = yv(0, ncol - 1);
    const long long p0 = sp0 < 0 ? 0 : (sp0 > L ? L : sp0);
    const int Tn = (int)min((long long)T, L - p0);        // tokens beyond the capacity are dropped

    // The window: row i holds raw position p0 + Tn - W + i; rows of old positions move down by Tn, new
    // positions take the projected KV rows.  Rows go in batches of AS_WG groups in increasing row order: a
    // batch loads all its sources (old rows lie Tn rows further on, past every row written so far), then,
    // after a barrier, stores them.  The first batch's loads are issued before the pools are updated, so
    // that they overlap that work.
    constexpr int AS_WG = 8;
    uint16_t* wb = win + (size_t)b * W * D;
    const int cpr = D / 8;                                  // 16-byte chunks per row
    const int per = AS_TPB / cpr;                           // rows per group
    const int cc = tid % cpr;
    const bool do_win = W > 0 && Tn > 0;
    u32x4_t v[AS_WG];
    auto win_load = [&](int i0) {
#pragma unroll
        for (int gi = 0; gi < AS_WG; ++gi) {
            const int i = i0 + gi * per + tid / cpr;
            v[gi] = u32x4_t{0, 0, 0, 0};
            if (tid < per * cpr && i < W) {
                const long long u = p0 + Tn - W + i;
                if (u >= p0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[gi][e] = pack_bf16x2(yv((int)(u - p0), cc * 8 + 2 * e), yv((int)(u - p0), cc * 8 + 2 * e + 1));
                } else {
                    v[gi] = *(const u32x4_t*)(wb + (size_t)(i + Tn) * D + cc * 8);
                }
            }
        }
    };
    auto win_store = [&](int i0) {
#pragma unroll
        for (int gi = 0; gi < AS_WG; ++gi) {
            const int i = i0 + gi * per + tid / cpr;
            if (tid < per * cpr && i < W) *(u32x4_t*)(wb + (size_t)i * D + cc * 8) = v[gi];
        }
    };
    if (do_win) win_load(0);

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
        // CSA block: slot p mod m (a new block restarts the pool)
        const int sc = (int)(p % m), sh = (int)(p % mh);
        const float zc = (t == 0 ? zc0 : yv(t, ncol - 2)) + (b_slot ? b_slot[sc] : 0.f);
        const float zh = (t == 0 ? zh0 : yv(t, ncol - 1)) + (b_slot_h ? b_slot_h[sh] : 0.f);
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
                A[k] = A[k] * fc_old + fc_new * (t == 0 ? y0[k] : yv(t, c));
                if (wc) {
                    const float val = A[k] / Sc;
                    const size_t row = entry_row(pm_c, b, Nc, jc);
                    if (c < D) kv[row * D + c] = f32_to_bf16(val);
                    else if (ik_dtype == 0) ((uint16_t*)ik)[row * dI + (c - D)] = f32_to_bf16(val);
                    else ((uint8_t*)ik)[row * dI + (c - D)] = f32_to_e4m3(val);
                }
            } else if (c < 2 * D + dI) {
                A[k] = A[k] * fh_old + fh_new * (t == 0 ? y0[k] : yv(t, c));
                if (wh) kvh[entry_row(pm_h, b, Nh, jh) * D + (c - D - dI)] = f32_to_bf16(A[k] / Sh);
            }
        }
    }
    if (do_win) {
        for (int i0 = 0; i0 < W; i0 += AS_WG * per) {
            if (i0 > 0) win_load(i0);
            __syncthreads();
            win_store(i0);
            __syncthreads();
        }
    } else {
        __syncthreads();                                    // every thread has read seq_lens[b]
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
    return ((size_t)AP_KS * B * T * (2 * D + dI + 2) * 4 + 255) / 256 * 256;
}

int append_launch(const void* hidden, int B, int T, int Dh, const void* w_kv, const void* w_ik, const float* w_gate,
                  const float* b_slot, int D, int dI, int m, int ik_dtype, const void* w_kv_h, const float* w_gate_h,
                  const float* b_slot_h, int mh, long long L, long long* seq_lens, void* state, void* kv, void* ik,
                  void* kv_h, void* win, int W, const CacheLayout& lay, void* ws, hipStream_t st) {
    const int R = B * T, ncol = 2 * D + dI + 2;
    float* Y = (float*)ws;
    const int nblk = AP_KS * ((2 * D + dI) / 16 + 1) * ((R + 15) / 16);
    CSA_LAUNCH("k_app_proj", k_app_proj, dim3(nblk), dim3(64 * AP_WAVES), 0, st,
               (const uint16_t*)hidden, R, Dh, (const uint16_t*)w_kv, (const uint16_t*)w_ik,
               (const uint16_t*)w_kv_h, w_gate, w_gate_h, D, dI, Y);
    const int Nc = (int)((L + m - 1) / m), Nh = (int)((L + mh - 1) / mh);
    CSA_LAUNCH("k_app_state", k_app_state, dim3(B), dim3(AS_TPB), 0, st, Y, T, seq_lens, L, b_slot, b_slot_h, D, dI, m,
               mh, ik_dtype, (float*)state, (int)append_state_words(D, dI), (uint16_t*)kv, ik, (uint16_t*)kv_h, Nc, Nh,
               page_map(lay, m), page_map(lay, mh), (uint16_t*)win, W);
    return 0;
}

}  // namespace csa_host

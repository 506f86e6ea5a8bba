// kernels.h -- host-side launchers shared between the translation units of libcsa.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <algorithm>

#include "common.h"

namespace csa_host {

// Optional layout of a batch and its caches (all null: every sequence holds L tokens, batch-major arrays).
struct CacheLayout {
    const long long* seq_lens;   // [B] raw tokens per sequence (variable-length batch) or null
    const int32_t* table;        // [B][max_blocks] page ids of the paged caches or null
    int max_blocks;
    int num_blocks;              // pages in each pool
    int block_tokens;            // raw tokens per page (entries per page = block_tokens / ratio, a power of two)
};
inline int log2_exact(int x) { int e = 0; while ((1 << e) < x) ++e; return e; }
// The page map of a cache of ratio m under this layout (no table: plain batch-major rows).
inline csa::PageMap page_map(const CacheLayout& lay, int m) {
    csa::PageMap pm{lay.table, lay.max_blocks, 0, lay.num_blocks};
    if (lay.table) pm.eshift = log2_exact(lay.block_tokens / m);
    return pm;
}
// workspace of index_topk_launch for these arguments (plain: no seq_lens and no table, so the many-query
// path may apply)
size_t index_topk_ws_bytes(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk, bool plain = true);
int index_topk_launch(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B, int Tq,
                      int HI, int dI, int Nc, long long L, int m, long long pos0, int topk,
                      int32_t* idx_out, int32_t* cnt_out, float* score_out, const CacheLayout& lay,
                      const uint8_t* q_scale, const uint8_t* k_scale, void* ws, hipStream_t st,
                      bool hist_zero = false);   // hist_zero: the workspace's histogram words already hold zeros
int kv_fp8_launch(const void* x, long long n, int D, void* y, hipStream_t st);
int mxfp4_launch(const void* x, long long n, int len, void* codes, void* scales, hipStream_t st);
// many-query (prefill) indexer path: Tq >= 64, topk <= 1024; bf16 / e4m3 rows of dI = 64 or 128 or MXFP4 rows
// of 128, HI = 1, 2, 4 or 8 (all but bf16 8 x 128 widened to it in the workspace first)
bool prefill_index_applicable(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk);
size_t prefill_index_ws_bytes(int dtype, int HI, int dI, int B, int Tq, int Nc);
int prefill_index_launch(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int HI, int dI, int B,
                         int Tq, int Nc, long long L, int m, long long pos0, int topk, int32_t* idx_out,
                         int32_t* cnt_out, float* score_out, const uint8_t* q_scale, const uint8_t* k_scale, void* ws,
                         hipStream_t st);
int fp8_to_bf16_launch(const void* in, void* out, int n, hipStream_t st);
int rope_launch(const void* x, void* y, const long long* pos, long long n, int D, int rd, int group, double theta,
                int inverse, hipStream_t st);

// Row sets of the split-KV attention: dense over a visible prefix (HCA), or
// gathered entries followed by raw window rows (CSA).
struct AttnRows {
    int mode;                 // 0 = dense prefix, 1 = selected + window
    const void* kv;           // [B][N][D]
    int N;                    // entries per sequence in kv
    long long L;              // raw tokens (dense visibility)
    int ratio;                // compression ratio (dense visibility)
    const int32_t* idx;       // [B][Tq][topk] (mode 1)
    int topk;
    const void* kv_raw;       // [B][Lr][D] (mode 1)
    int Lr;
    long long raw0;
    int W;
    const float* sink;        // [H] per-head attention-sink logits (natural log), or null
    const long long* seq_lens;  // [B] raw tokens per sequence (variable-length batch) or null
    csa::PageMap pm;          // entries through a block table (pm.table null: batch-major kv)
    const void* v;            // values of the entries when separate from kv (same rows), or null
    const void* v_raw;        // values of the raw rows when separate from kv_raw, or null
    int kv_fp8;               // entry rows in the FP8 format (D + 80 bytes per row), raw rows bf16
    int rope_rd;              // fused rotary embedding of the last rope_rd dims (0: none)
    double rope_theta;
};
// mode 0: dense over n rows; mode 1: n selected entries + W window rows
size_t attn_ws_bytes(int B, int Tq, int H, int D, int mode, int n, int W);
int attn_launch(const void* q, const AttnRows& rows, int B, int Tq, int H, int D, long long pos0, float scale,
                void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st, const char* tag);
size_t compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W);
size_t hca_compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W, int mh);
int hca_compress_launch(const void* hidden, const void* w_kv, const void* w_ik, const float* w_gate,
                        const float* b_slot, int B, long long L, int Dh, int D, int dI, int m, int W, int ik_dtype,
                        void* kv_out, void* ik_out, void* win_out, const void* w_kv_h, const float* w_gate_h,
                        const float* b_slot_h, int mh, void* kv_h_out, void* ws, hipStream_t st);
size_t append_state_words(int D, int dI);
size_t append_ws_bytes(int B, int T, int D, int dI);
int append_launch(const void* hidden, int B, int T, int Dh, const void* w_kv, const void* w_ik, const float* w_gate,
                  const float* b_slot, int D, int dI, int m, int ik_dtype, const void* w_kv_h, const float* w_gate_h,
                  const float* b_slot_h, int mh, long long L, long long* seq_lens, void* state, void* kv, void* ik,
                  void* kv_h, void* win, int W, const CacheLayout& lay, void* ws, hipStream_t st);
int compress_launch(const void* hidden, const void* w_kv, const void* w_ik, const float* w_gate,
                    const float* b_slot, int B, long long L, int Dh, int D, int dI, int m, int W,
                    int ik_dtype, void* kv_out, void* ik_out, void* win_out, void* ws, hipStream_t st);

}  // namespace csa_host

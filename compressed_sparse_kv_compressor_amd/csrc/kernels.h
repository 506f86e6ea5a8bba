// kernels.h -- host-side launchers shared between the translation units of libcsa.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <algorithm>

namespace csa_host {

// workspace of index_topk_launch for these arguments (the many-query path when it applies)
size_t index_topk_ws_bytes(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk);
int index_topk_launch(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B, int Tq,
                      int HI, int dI, int Nc, long long L, int m, long long pos0, int topk,
                      int32_t* idx_out, int32_t* cnt_out, void* ws, hipStream_t st);
// many-query (prefill) indexer path: bf16, HI = 8, dI = 128, Tq >= 64, topk <= 1024
bool prefill_index_applicable(int dtype, int HI, int dI, int B, int Tq, int Nc, int topk);
size_t prefill_index_ws_bytes(int B, int Tq, int Nc);
int prefill_index_launch(const void* q_idx, const float* w_idx, const void* k_idx, int B, int Tq, int Nc,
                         long long L, int m, long long pos0, int topk, int32_t* idx_out, int32_t* cnt_out, void* ws,
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
int compress_launch(const void* hidden, const void* w_kv, const void* w_ik, const float* w_gate,
                    const float* b_slot, int B, long long L, int Dh, int D, int dI, int m, int W,
                    int ik_dtype, void* kv_out, void* ik_out, void* win_out, void* ws, hipStream_t st);

}  // namespace csa_host

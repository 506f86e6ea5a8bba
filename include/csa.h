/*
 * csa.h -- C ABI of the MI355X (gfx950) hybrid compressed attention library
 *          (libcsa.so): DeepSeek-V4's Compressed Sparse Attention (CSA) and
 *          Heavily Compressed Attention (HCA).
 *
 * Pages this operation set is defined on:
 *  [P1] "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化" (cdjax.com),
 *       section 1.1 "混合注意力：CSA 与 HCA 的协同": the token-level compressor
 *       (m tokens -> one KV entry), the Lightning Indexer, the top-k selector
 *       (Pro keeps 1024), MQA-form core attention, the extra sliding-window
 *       branch, HCA's dense attention over all compressed entries, and the
 *       interleaving of CSA and HCA layers.
 *  [P2] "DeepSeek V4 详解：1M 上下文背后，真正发生了什么", sections
 *       "第一刀：让注意力别再按原价付费" (m, m', per-query top-k, HCA dense),
 *       "第二刀：KV cache 被当成系统在管" (compressed entries + window state),
 *       "mHC、Muon、FP4：这些不是论文装饰" (low-precision indexer QK path).
 *  [P3] "DeepSeek-V4 技术报告解读：百万Token上下文是怎么做到的", section
 *       "三大架构改动" items 1-2 (sequence shrinks to 1/m; m' >> m; window).
 *  [P5] chenxutan.com preface: CSA 4:1, HCA 128:1.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers, 16-byte aligned, dense, row-major
 *    in the index order written next to them.  The caller owns every buffer;
 *    the library keeps no pointer after the call returns and allocates no
 *    device memory: scratch comes from the caller's workspace `ws` of
 *    `ws_bytes` bytes, whose required size the matching *_ws_bytes() call
 *    returns (0 is a valid answer; ws may then be NULL).
 *  - `stream` is a hipStream_t (NULL = the default stream).  On CSA_OK the work
 *    is enqueued on that stream and the call returns without waiting.
 *  - Every argument is validated on the host before anything is enqueued.  On
 *    error nothing is enqueued, a csa_status_t code is returned, and
 *    csa_last_error() (thread-local) holds a one-line explanation.  No
 *    exception or abort crosses the ABI.
 *  - dtypes: CSA_BF16 = bfloat16 (stored as 16-bit patterns), CSA_E4M3 = OCP
 *    8-bit float E4M3 (e4m3fn: bias 7, max 448, 0x7f/0xff NaN).
 *  - Results are deterministic: identical inputs give bitwise identical
 *    outputs (no float atomics; every reduction has a fixed order).
 *  - Inputs must be finite.
 *
 * Positions: raw token positions are absolute, 0-based.  A ratio-m compression
 * of L tokens has N = ceil(L/m) entries; entry j covers raw tokens
 * [j*m, min((j+1)*m, L)) and is visible to a query at position p iff
 * min((j+1)*m, L) - 1 <= p (so visible entries are always a prefix).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 6

typedef enum {
    CSA_OK = 0,
    CSA_ERR_NULL = 1,        /* a required pointer is NULL */
    CSA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
    CSA_ERR_DTYPE = 3,       /* unknown dtype code */
    CSA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    CSA_ERR_WORKSPACE = 5,   /* ws_bytes below the *_ws_bytes() answer */
    CSA_ERR_UNSUPPORTED = 6, /* valid, but outside the sizes this build supports */
    CSA_ERR_HIP = 7          /* a HIP runtime call or launch failed */
} csa_status_t;

typedef enum { CSA_BF16 = 0, CSA_E4M3 = 1, CSA_MXFP4 = 2 } csa_dtype_t;
/* Storage format of compressed KV entry rows (the *_ex attention entry points). */
typedef enum { CSA_KV_BF16 = 0, CSA_KV_FP8 = 1 } csa_kv_format_t;

/* Library identity and error reporting. */
int csa_abi_version(void);                 /* returns CSA_ABI_VERSION */
const char* csa_status_str(int status);    /* static string for a status code */
const char* csa_last_error(void);          /* thread-local detail of the last error ("" if none) */

/* ------------------------------------------------------------------------ */
/* A1. Token-level KV compressor ([P1] 1.1; [P2] first section; [P3] item 1) */
/* ------------------------------------------------------------------------ */
/* Compresses every m raw tokens into one entry.  The pages do not print the
 * pooling weights; this library implements softmax-gated pooling within each
 * block (block mean when w_gate = 0 and b_slot = 0):
 *   z_t = hidden_t . w_gate + b_slot[t - j*m],   a = softmax over the block,
 *   kv_out[j] = bf16( sum_t a_t * (hidden_t . w_kv^T) )
 *   ik_out[j] = bf16 or e4m3( sum_t a_t * (hidden_t . w_ik^T) )   (if w_ik)
 *   win_out[u] = bf16( hidden_{L-W+u} . w_kv^T )   for u in [0, W)  (if win_out;
 *                rows for negative positions are zero)
 * The tail entry j = N-1 pools the L mod m remaining tokens when m does not
 * divide L.  Pooling is applied before the projection (equal to projecting
 * first by linearity; the pooled hidden row is rounded to bf16 once).
 *   hidden [B][L][Dh] bf16       w_kv [D][Dh] bf16     w_ik [dI][Dh] bf16 or NULL
 *   w_gate [Dh] fp32             b_slot [m] fp32 or NULL (= zeros)
 *   kv_out [B][N][D] bf16        ik_out [B][N][dI] (ik_dtype) or NULL
 *   win_out [B][W][D] bf16 or NULL
 * Supported: Dh % 64 == 0 and 64 <= Dh <= 16384; D, dI in {64, 128, 256, 512};
 * 1 <= m <= 1024; 0 <= W <= 1024; 1 <= L; B >= 1. */
/* Workspace of csa_compress: pooled rows [B][N][Dh] bf16, plus fp32 split-K partial sums when a
 * projection has too few output tiles to fill the GPU.  Pass dI = 0 when no indexer keys are
 * requested and W = 0 when no window rows are. */
size_t csa_compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W);
int csa_compress(const void* hidden, const void* w_kv, const void* w_ik,
                 const float* w_gate, const float* b_slot,
                 int B, long long L, int Dh, int D, int dI, int m, int W, int ik_dtype,
                 void* kv_out, void* ik_out, void* win_out,
                 void* ws, size_t ws_bytes, void* stream);

/* Both compressed caches of the same tokens in one call ([P1] 1.1: CSA and HCA side by side;
 * [P3] item 1): the result equals csa_compress with the CSA arguments (m, indexer keys, window)
 * followed by csa_compress(hidden, w_kv_h, NULL, w_gate_h, b_slot_h, ..., m = mh, W = 0,
 * kv_h_out).  Where the shape allows (Dh in {1024, 2048, 4096}, m = 4, mh a multiple of 16) the
 * hidden rows are read once for both caches; otherwise the two poolings run one after the other.
 *   w_kv_h [D][Dh] bf16    w_gate_h [Dh] fp32    b_slot_h [mh] fp32 or NULL
 *   kv_h_out [B][ceil(L/mh)][D] bf16
 * Supported: as csa_compress, and 1 <= mh <= 1024.  Errors and ownership as csa_compress. */
size_t csa_hca_compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W, int mh);
int csa_hca_compress(const void* hidden, int B, long long L, int Dh,
                     const void* w_kv, const void* w_ik, const float* w_gate, const float* b_slot,
                     int D, int dI, int m, int W, int ik_dtype,
                     void* kv_out, void* ik_out, void* win_out,
                     const void* w_kv_h, const float* w_gate_h, const float* b_slot_h, int mh, void* kv_h_out,
                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Batch and cache layouts ([P2] "第二刀：KV cache 被当成系统在管": the      */
/* compressed entries live in a classical cache managed in blocks)          */
/* ------------------------------------------------------------------------ */
/* Optional layout of a batch and of its compressed caches, taken by the *_ex
 * entry points and by the fused decode.  A NULL pointer or NULL fields give the
 * plain layout of the entry points without _ex.
 *  seq_lens     device [B] int64, or NULL.  Variable-length batch: sequence b
 *               holds seq_lens[b] raw tokens.  The call's L is then the
 *               capacity (it sizes the caches: ceil(L / ratio) entries per
 *               sequence), and Tq <= seq_lens[b] <= L is required (values
 *               outside are clamped into it).  The Tq queries of sequence b are
 *               its last Tq tokens and its Lr raw rows its last Lr tokens (raw
 *               row i holds position seq_lens[b] - Lr + i); pos0 and raw0 are
 *               ignored.
 *  block_table  device [B][max_blocks] int32, or NULL.  Paged caches: each
 *               compressed cache is a pool of num_blocks pages, a page holding
 *               the entries of block_tokens consecutive raw tokens (epb =
 *               block_tokens / ratio entries, a power of two; block_tokens =
 *               lcm(m, m') = 128 serves CSA m = 4 and HCA m' = 128 with one
 *               table).  Entry s of sequence b is row
 *               block_table[b][s / epb] * epb + s % epb of the pool, whose rows
 *               have the plain arrays' row layout ([num_blocks * epb][row]).
 *               Page ids outside [0, num_blocks) are clamped into it (wrong
 *               data, never an access out of bounds); the pages that hold a
 *               sequence's visible entries must be valid.  The caller owns the
 *               table and the pools. */
typedef struct csa_cache_layout {
    const long long* seq_lens;
    const int32_t* block_table;
    int max_blocks;
    int num_blocks;
    int block_tokens;
} csa_cache_layout_t;

/* ------------------------------------------------------------------------ */
/* Incremental compression during decode: the per-request state cache       */
/* ([P2] "第二刀：KV cache 被当成系统在管": compressed entries in a classical */
/* cache, plus a fixed-size state per request for the window and the tail)  */
/* ------------------------------------------------------------------------ */
/* Appends T new tokens to every sequence of a batch whose caches were built by
 * csa_hca_compress (or by earlier appends).  For each new token at position
 * p = seq_lens[b] + t, in order: its KV row (w_kv), indexer key (w_ik) and HCA
 * row (w_kv_h) are projected once, with its gate logits; the running
 * softmax-gated pools of the open CSA block (p / m) and HCA block (p / mh)
 * absorb it; the entries of every block it touched are rewritten as the pool
 * so far, rounded once (so after the call the caches hold exactly what
 * csa_hca_compress of the whole prefix gives, within fp32 summation order:
 * complete blocks final, the last entries provisional); the window shifts by
 * T rows (win[b][i] = the raw KV row of position L_b - W + i); and
 * seq_lens[b] advances by T on the device (tokens beyond the capacity L are
 * dropped).  Arguments as csa_hca_compress, plus:
 *   hidden    [B][T][Dh] bf16: the new tokens
 *   L         capacity in raw tokens (caches hold ceil(L/m), ceil(L/mh) entries
 *             per sequence, or their pools through layout->block_table)
 *   seq_lens  device [B] int64, read and advanced
 *   state     device [B][csa_append_state_bytes(D, dI)] fp32, caller-owned:
 *             the open blocks' pools.  It is ignored for a sequence whose
 *             length is a multiple of both m and mh (both blocks start fresh);
 *             otherwise it must be the state the previous append left (a
 *             sequence compressed in bulk should stop at such a multiple, e.g.
 *             of lcm(m, mh) = 128, and append the rest)
 *   win       [B][W][D] bf16, caller-owned (the bulk compressor's win_out)
 *   layout    NULL or a block table for paged caches (its seq_lens field is
 *             not used; the argument above is)
 * Supported: D in {64, 128, 256, 512}, dI in {0, 64, 128, 256, 512},
 * 2 D + dI <= 2048, Dh % 64 == 0, 1 <= m, mh <= 1024, T >= 1, 0 <= W <= 1024.
 * Workspace: csa_decode_append_ws_bytes (the fp32 projections). */
size_t csa_append_state_bytes(int D, int dI);
size_t csa_decode_append_ws_bytes(int B, int T, int D, int dI);
int csa_decode_append(const void* hidden, int B, int T, int Dh,
                      const void* w_kv, const void* w_ik, const float* w_gate, const float* b_slot,
                      int D, int dI, int m, int ik_dtype,
                      const void* w_kv_h, const float* w_gate_h, const float* b_slot_h, int mh,
                      long long L, long long* seq_lens, void* state,
                      void* kv_out, void* ik_out, void* kv_h_out, void* win, int W,
                      const csa_cache_layout_t* layout, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* A2 + A3. Lightning-Indexer scores and per-query top-k                     */
/*          ([P1] 1.1; [P2] first section and "mHC、Muon、FP4")              */
/* ------------------------------------------------------------------------ */
/* For query t of sequence b (absolute position pos0 + t) and every visible
 * compressed entry s, the score is the canonical fp32 value
 *   S = fma-chain over h = 0..HI-1 of  w_idx[h] * ReLU( RN32( exact q_h . k_s ) )
 * (each per-head dot product is the exact sum rounded once to fp32, ReLU maps
 * <= 0 to +0, and S = fmaf(w_h, r_h, S) starting from S = +0).  The selection
 * keeps the first min(topk, n_visible) entries under the total order
 * (S descending, index ascending) -- bit-exact, independent of how the GPU
 * computes its internal approximate scores.
 *   q_idx [B][Tq][HI][dI] dtype     w_idx [B][Tq][HI] fp32
 *   k_idx [B][Nc][dI] dtype         (Nc = ceil(L/m) entries; L raw tokens)
 *   idx_out [B][Tq][topk] int32: selected entry indices in ascending order,
 *           padded with -1 after cnt entries
 *   cnt_out [B][Tq] int32 or NULL: min(topk, n_visible)
 *   score_out [B][Tq][topk] fp32 or NULL: for each returned index, the score
 *           the GPU ranked it by -- the MFMA-path approximate score S~, which
 *           satisfies |S~ - S| <= the certified bound of that entry (entries
 *           whose order was settled on exact scores keep their S~ here too),
 *           or the exact S for rows the exact fallback selected; NaN in the
 *           padding slots and in rows with at most topk visible entries (those
 *           are selected whole, without scoring)
 * Supported: dtype in {CSA_BF16, CSA_E4M3}; HI in {1,2,4,8,16}; dI in {64,128};
 * 1 <= topk <= 4096; 1 <= Tq <= 65536; Nc <= 2^24; pos0 >= 0.
 * Workspace: csa_index_topk_ws_bytes with the call's sizes (the many-query path,
 * used for Tq >= 64, topk <= 1024, HI in {1,2,4,8} and bf16 / e4m3 rows of
 * dI 64 or 128 or MXFP4 rows of 128 on the plain layout, keeps no score matrix:
 * operands other than bf16 8 x 128 are first widened exactly to that format in
 * the workspace -- every e4m3 and scaled E2M1 value is a bf16 value, padded
 * heads carry weight +0 and padded dims are zero, so no score changes; the
 * per-query path holds Tq x Nc fp32 scores and lists).  Returns 0 on invalid
 * sizes. */
size_t csa_index_topk_ws_bytes(int B, int Tq, int HI, int dI, int Nc, int topk, int dtype);
int csa_index_topk(const void* q_idx, const float* w_idx, const void* k_idx, int dtype,
                   int B, int Tq, int HI, int dI, int Nc, long long L, int m, long long pos0,
                   int topk, int32_t* idx_out, int32_t* cnt_out, float* score_out,
                   void* ws, size_t ws_bytes, void* stream);

/* csa_index_topk over a variable-length and/or paged batch (layout above):
 * k_idx is then the pool of indexer-key rows when block_table is given.
 * Results as csa_index_topk (bit-exact to running each sequence on its own
 * contiguous cache).  Such calls always take the per-query path, so the
 * workspace (csa_index_topk_ex_ws_bytes) holds Tq x Nc scores per sequence; a
 * plain layout (NULL, or neither seq_lens nor block_table) routes like
 * csa_index_topk, MXFP4 operands included. */
/* dtype CSA_MXFP4 ([P2] "mHC、Muon、FP4": the indexer's QK path in FP4; see
 * csa_mxfp4_encode for the format): q_idx is then the E2M1 codes
 * [B][Tq][HI][dI/2] and q_scale their E8M0 scales [B][Tq][HI][dI/32], k_idx the
 * codes [B][Nc][dI/2] (or their pool) and k_scale [B][Nc][dI/32] (or their pool,
 * rows alongside k_idx); dI = 128.  The canonical score is taken over the
 * decoded values, so the selection is bit-exact to the oracle's over the same
 * MXFP4 operands.  q_scale and k_scale are NULL for the other dtypes. */
size_t csa_index_topk_ex_ws_bytes(int B, int Tq, int HI, int dI, int Nc, int topk, int dtype,
                                  const csa_cache_layout_t* layout);
int csa_index_topk_ex(const void* q_idx, const float* w_idx, const void* k_idx, int dtype,
                      int B, int Tq, int HI, int dI, int Nc, long long L, int m, long long pos0,
                      int topk, int32_t* idx_out, int32_t* cnt_out, float* score_out,
                      const csa_cache_layout_t* layout, const void* q_scale, const void* k_scale,
                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* A4. CSA core attention: MQA over the selected entries plus a sliding       */
/*     window of raw local tokens ([P1] 1.1; [P3] item 1)                    */
/* ------------------------------------------------------------------------ */
/* For query t of sequence b at p = pos0 + t and every head h, one softmax over
 * the union of {kv[b][j] : j in idx[b][t][*], j >= 0} and the raw window rows
 * {kv_raw[b][u - raw0] : u in [max(0, p-W+1), p]}; each row is both key and
 * value (MQA, one shared KV head):
 *   l_r = scale * (q_h . x_r),  out_h = sum_r softmax(l)_r x_r,
 *   lse_h = log sum_r exp(l_r)   (natural log; -inf and out = 0 if no rows).
 * With sink (device, [H] fp32 natural-log logits, or NULL) every head's softmax has one more denominator
 * term exp(sink[h]) with no value row ([P1] 1.1: a learnable attention-sink logit lets a head send its
 * total attention towards 0): out_h = sum_r exp(l_r) x_r / (exp(sink_h) + sum_r exp(l_r)),
 * lse_h = log(exp(sink_h) + sum_r exp(l_r)) (= sink_h when there are no rows).
 *   q   [B][Tq][H][D] bf16       kv [B][Nc][D] bf16
 *   idx [B][Tq][topk] int32 (entries < 0 are skipped; must be < Nc)
 *   kv_raw [B][Lr][D] bf16, row i = raw position raw0 + i (may be NULL if W = 0)
 *   out [B][Tq][H][D] bf16       lse_out [B][Tq][H] fp32 or NULL
 * Requires raw0 <= max(0, pos0 - W + 1) and pos0 + Tq - 1 < raw0 + Lr when W > 0.
 * Supported: D in {128, 512}; H % 16 == 0, H <= 256; 0 <= topk <= 4096;
 * 0 <= W <= 1024. */
size_t csa_sparse_attn_ws_bytes(int B, int Tq, int H, int D, int topk, int W);
int csa_sparse_attn(const void* q, const void* kv, const int32_t* idx, const void* kv_raw,
                    int B, int Tq, int H, int D, int Nc, int topk, int Lr, long long raw0,
                    long long pos0, int W, float scale, const float* sink, void* out, float* lse_out,
                    void* ws, size_t ws_bytes, void* stream);

/* Partial rotary position embedding fused into the attention ([P1] 1.1: RoPE
 * acts on the last 64 dimensions of the queries and keys, and the core
 * attention's output takes the inverse rotation at the query's position).
 * With a non-NULL csa_rope_t the attention computes
 *   out = R(-p) . attn(R(p) q)
 * for the query at absolute position p (pos0 + t, or its sequence's position
 * with seq_lens), R(a) turning pair j = (D-rd+2j, D-rd+2j+1) by the angle
 * a * theta^(-2j/rd) (as csa_rope; the keys are rotated by the caller when it
 * stores them).  The rotated query is rounded to bf16 like csa_rope's output;
 * the output is rotated in fp32 before its one bf16 rounding.  Supported:
 * rd = 64 (the pages' RoPE width), theta finite and > 1. */
typedef struct csa_rope {
    int rd;          /* rotated dimensions at the end of each row: 64 */
    double theta;    /* frequency base (10000 in the usual reading) */
} csa_rope_t;

/* csa_sparse_attn over a variable-length and/or paged batch (layout above;
 * kv is then the entry pool when block_table is given), and with values that
 * may differ from the keys ([P1] 1.1 reads MQA with one vector per entry as key
 * and value; this variant serves models that keep them apart):
 *   v      [same rows as kv] bf16 or NULL (= kv): the value of entry j
 *   v_raw  [B][Lr][D] bf16 or NULL (= kv_raw): the value of raw row i
 *   out_h = sum_r softmax(l)_r v_r with l_r = scale * q_h . k_r.
 * m is the ratio of the cache kv (it sets the entries per page of a paged
 * pool).  kv_format CSA_KV_FP8: kv (and v) rows are FP8 rows of D + 80 bytes
 * (csa_kv_fp8_encode; the raw rows stay bf16), attended as their exact bf16
 * decoding.  With seq_lens, every sequence's Lr raw rows are its last Lr tokens,
 * so Lr >= Tq + W - 1 is required when W > 0.  rope: the fused rotary
 * embedding above, or NULL (none).  Workspace: csa_sparse_attn_ws_bytes. */
int csa_sparse_attn_ex(const void* q, const void* kv, const void* v, const int32_t* idx, const void* kv_raw,
                       const void* v_raw, int B, int Tq, int H, int D, int Nc, int m, int topk, int Lr,
                       long long raw0, long long pos0, int W, float scale, const float* sink,
                       const csa_cache_layout_t* layout, int kv_format, const csa_rope_t* rope, void* out,
                       float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* No-allocation variant of csa_sparse_attn, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and results as csa_sparse_attn
 * (bitwise: the same kernels and split plan), minus the workspace.  The split
 * partials live in a static device array of CSA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; its device
 * address is looked up once per device (the current device; `stream` must
 * belong to it).  The call allocates nothing.  A call whose partials need more
 * than CSA_NOALLOC_SCRATCH_BYTES (csa_sparse_attn_ws_bytes of the same sizes)
 * returns CSA_ERR_UNSUPPORTED and enqueues nothing.  All calls on one GPU share
 * the one array: calls that overlap in time on one GPU (different streams,
 * threads) race and give undefined results; calls ordered on one stream are
 * safe (every call rewrites the partials it reads). */
#define CSA_NOALLOC_SCRATCH_BYTES (64ull << 20)
int csa_sparse_attn_noalloc(const void* q, const void* kv, const int32_t* idx, const void* kv_raw,
                            int B, int Tq, int H, int D, int Nc, int topk, int Lr, long long raw0,
                            long long pos0, int W, float scale, const float* sink, void* out, float* lse_out,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* A5. HCA attention: dense MQA over every visible compressed entry          */
/*     ([P1] 1.1; [P2] first section; [P3] item 2)                           */
/* ------------------------------------------------------------------------ */
/* As A4 (sink included) but over {kv_h[b][j] : j visible to p} (ratio mh over L
 * raw tokens), with no selection and no window.
 *   q [B][Tq][H][D] bf16    kv_h [B][Nh][D] bf16 (Nh = ceil(L/mh))
 *   out [B][Tq][H][D] bf16  lse_out [B][Tq][H] fp32 or NULL
 * Supported: D in {128, 512}; H % 16 == 0, H <= 256. */
size_t hca_dense_attn_ws_bytes(int B, int Tq, int H, int D, int Nh);
int hca_dense_attn(const void* q, const void* kv_h, int B, int Tq, int H, int D, int Nh,
                   long long L, int mh, long long pos0, float scale, const float* sink,
                   void* out, float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* hca_dense_attn over a variable-length and/or paged batch, with optional
 * separate values v_h (same rows as kv_h, or NULL = kv_h), FP8 entry rows and
 * the fused rotary embedding; as csa_sparse_attn_ex.  With seq_lens, L is the
 * capacity (Nh = ceil(L / mh)). */
int hca_dense_attn_ex(const void* q, const void* kv_h, const void* v_h, int B, int Tq, int H, int D, int Nh,
                      long long L, int mh, long long pos0, float scale, const float* sink,
                      const csa_cache_layout_t* layout, int kv_format, const csa_rope_t* rope, void* out,
                      float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Low-precision cache formats ([P1] 1.1, last paragraph: RoPE dimensions in */
/* BF16, the others in FP8; [P2] "mHC、Muon、FP4": the indexer QK in FP4)    */
/* ------------------------------------------------------------------------ */
/* FP8 KV rows.  x [n][D] bf16 (D in {128, 512}; its last 64 dimensions are the
 * RoPE dimensions) -> y [n][D + 80] bytes: e4m3 codes of dimensions 0..D-65 in
 * groups of 64, each group divided by its smallest power-of-two scale 2^e with
 * max |x| <= 448 * 2^e (0 for an all-zero group; exact division, rounding to
 * nearest even, no saturation), then the 64 RoPE dimensions as bf16, then one
 * byte e + 127 per group (16 bytes, unused ones 0).  A dimension decodes to
 * e4m3(code) * 2^e, exact in bf16 for e >= -126.  Bit-exact. */
int csa_kv_fp8_encode(const void* x, long long n, int D, void* y, void* stream);
/* MXFP4 (the OCP Microscaling FP4 format).  x [n][len] bf16 (len % 32 == 0,
 * len <= 4096) -> codes [n][len/2] (E2M1: sign, 2 exponent bits, 1 mantissa bit;
 * element 2i in the low nibble of byte i) and scales [n][len/32] (E8M0: the
 * byte X + 127 for the scale 2^X of each 32 elements, X = floor(log2 max|x|)
 * - 2 clamped to [-127, 127], -127 for an all-zero block); each element is
 * x / 2^X rounded to the nearest E2M1 value, ties to the even code, saturating
 * at 6.  Bit-exact.  Pointers 16-byte aligned except scales (any). */
int csa_mxfp4_encode(const void* x, long long n, int len, void* codes, void* scales, void* stream);

/* ------------------------------------------------------------------------ */
/* A6. Fused decode of one interleaved CSA layer followed by one HCA layer   */
/*     ([P1] 1.1: the two attention kinds alternate across layers)           */
/* ------------------------------------------------------------------------ */
/* One query token per sequence at position L-1 (decode).  Runs, in stream
 * order and without host synchronisation: csa_index_topk -> csa_sparse_attn
 * (CSA layer), then hca_dense_attn (HCA layer).  The two layers take their own
 * queries; a caller chaining real layers feeds one layer's output into the
 * next layer's projections outside this call. */
typedef struct csa_hca_decode_args {
    int B;                 /* sequences */
    long long L;           /* raw context length of every sequence */
    int H, D;              /* query heads and KV dim of both layers */
    float scale;           /* softmax scale of both layers */
    /* CSA layer */
    const void* csa_q;     /* [B][H][D] bf16 */
    const void* q_idx;     /* [B][HI][dI] idx_dtype */
    const float* w_idx;    /* [B][HI] fp32 */
    const void* k_idx;     /* [B][Nc][dI] idx_dtype, Nc = ceil(L/m) */
    const void* kv;        /* [B][Nc][D] bf16 */
    const void* kv_raw;    /* [B][W][D] bf16: raw positions L-W .. L-1 */
    int idx_dtype, HI, dI, m, topk, W;
    void* csa_out;         /* [B][H][D] bf16 */
    float* csa_lse;        /* [B][H] fp32 or NULL */
    int32_t* idx_out;      /* [B][topk] int32 or NULL (then kept in the workspace) */
    const float* csa_sink; /* [H] fp32 attention-sink logits of the CSA layer or NULL (see A4) */
    /* HCA layer */
    const void* hca_q;     /* [B][H][D] bf16 */
    const void* kv_h;      /* [B][Nh][D] bf16, Nh = ceil(L/mh) */
    int mh;
    void* hca_out;         /* [B][H][D] bf16 */
    float* hca_lse;        /* [B][H] fp32 or NULL */
    const float* hca_sink; /* [H] fp32 attention-sink logits of the HCA layer or NULL */
    /* Batch and cache layout of both layers (see csa_cache_layout_t), or NULL.  With seq_lens, L is the
     * capacity and each sequence decodes its token at seq_lens[b] - 1 (kv_raw holding its last W raw
     * tokens); with block_table, k_idx and kv are the CSA pools (ratio m) and kv_h the HCA pool (ratio
     * mh), all paged by the one table. */
    const csa_cache_layout_t* layout;
    /* With idx_dtype CSA_MXFP4: the E8M0 scales of q_idx [B][HI][dI/32] and of k_idx (rows alongside it). */
    const void* q_idx_scale;
    const void* k_idx_scale;
    /* The fused rotary embedding of each layer's attention (csa_rope_t above) or NULL: each query at its
     * decode position. */
    const csa_rope_t* csa_rope;
    const csa_rope_t* hca_rope;
    /* CSA_KV_BF16 (0), or CSA_KV_FP8: the entry rows of both layers (kv, kv_h) in the FP8 format of
     * csa_kv_fp8_encode, D + 80 bytes per row (the raw window rows kv_raw stay bf16). */
    int kv_format;
    /* 0, or 1 for a workspace the caller keeps across calls with the same sizes (a serving loop): its first
     * csa_hca_decode_ws_bytes(a) bytes must hold zeros before the first such call (allocate it zero-filled)
     * and must not be written by anything else between calls.  Each call then leaves the words the next one
     * counts on (the per-row score histograms) at zero, and skips clearing them itself.  Calls that overlap
     * in time on one workspace race, as with any shared workspace. */
    int ws_persistent;
} csa_hca_decode_args_t;

size_t csa_hca_decode_ws_bytes(const csa_hca_decode_args_t* a);
int csa_hca_decode(const csa_hca_decode_args_t* a, void* ws, size_t ws_bytes, void* stream);

/* C11: partial rotary position embedding [P1 section 1.1]: the rotation acts
 * on the last rd dimensions of a query / KV row only (rd = 64 on the pages),
 * and the core attention output takes the inverse rotation at its query
 * position.  Pair j = (D-rd+2j, D-rd+2j+1) turns by a = pos * theta^(-2j/rd):
 * (u, v) -> (u cos a - v sin a, u sin a + v cos a); inverse = 1 uses -a.  The
 * first D-rd dimensions are copied unchanged.
 *   x, y : device [n][D] bf16, 16-byte aligned; y == x (in place) is allowed,
 *          other overlaps are not.  Caller-owned.
 *   pos  : device [n / group] int64, 8-byte aligned; row r takes pos[r / group]
 *          (group = H for a [rows][H][D] query or output tensor, 1 for KV rows).
 *   D % 8 == 0, rd % 8 == 0, 0 < rd <= D, group >= 1 divides n, theta > 1
 *   (10000 is the usual base), inverse 0 or 1.  n = 0 is a no-op.
 * Angles are formed in fp64, the rotation in fp32, outputs rounded once (RNE).
 * Errors: CSA_ERR_SHAPE, CSA_ERR_NULL, CSA_ERR_ALIGN (nothing launched). */
int csa_rope(const void* x, void* y, const long long* pos, long long n, int D, int rd, int group, double theta,
             int inverse, void* stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */
/* Converts n OCP-e4m3 values (n % 4 == 0) to bf16 with the exact conversion
 * the indexer kernels apply to e4m3 keys and queries (every e4m3 value is a
 * bf16 value, so the result must equal the code's value).  in [n] e4m3,
 * out [n] bf16, both device pointers. */
int csa_debug_fp8_to_bf16(const void* in, void* out, int n, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (measurement aid; not part of the method)                   */
/* ------------------------------------------------------------------------ */
/* While enabled, every kernel the library launches is bracketed by a pair of
 * HIP events recorded on the stream it is launched on.  csa_prof_read() waits
 * for the recorded events and returns the summed duration (ms) and launch
 * count of every kernel whose name equals `kernel`.  csa_prof_reset() drops
 * all records.  Kernel names are the ones rocprofv3 reports. */
int csa_prof_enable(int on);
/* Restrict recording to launches of one kernel (NULL or "" records all), so
 * that timing one kernel adds only its own two events to the stream. */
int csa_prof_only(const char* kernel);
int csa_prof_reset(void);
int csa_prof_read(const char* kernel, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */

/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the hybrid compressed
 * attention that DeepSeek-V4 uses (CSA + HCA), used to check the HIP path.
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * it.  It shares no code with the HIP library and includes none of its headers.
 *
 * Sources (the web pages this method is described on):
 *  [P1] "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化" (cdjax.com),
 *       section 1.1 "混合注意力：CSA 与 HCA 的协同".
 *  [P2] "DeepSeek V4 详解：1M 上下文背后，真正发生了什么" (QianJinGuo wiki copy),
 *       sections "第一刀：让注意力别再按原价付费", "第二刀：KV cache 被当成系统在管",
 *       "mHC、Muon、FP4：这些不是论文装饰".
 *  [P3] "DeepSeek-V4 技术报告解读：百万Token上下文是怎么做到的" (blog.nickys.cn),
 *       section "三大架构改动" items 1 (CSA) and 2 (HCA).
 *  [P5] "1.6万亿参数，1M上下文，仅需27%算力：DeepSeek-V4-Pro 如何重新定义长文本推理"
 *       (chenxutan.com), preface: 4:1 and 128:1 compression ratios.
 *
 * All arithmetic is fp64 unless a step is defined to round (the canonical fp32
 * indexer score, and the final bf16 / e4m3 encodings).  Where the pages leave
 * a step open the reading taken is written next to the code that implements it.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no -ffast-math).
 * OpenMP only splits independent output rows across threads; it never changes
 * the order of any sum.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define ORA_BF16 0
#define ORA_E4M3 1

/* ------------------------------------------------------------------------- */
/* Number formats                                                            */
/* ------------------------------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32. */
double ora_bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit float E4M3 ("e4m3fn"): bias 7, no infinities, S.1111.111 is NaN,
 * subnormals f * 2^-9.  [P1 section 1.1 and P2 "mHC、Muon、FP4" name FP8/FP4
 * storage; the exact encoding is the OCP one that gfx950 implements.] */
double ora_e4m3_value(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, f = b & 7;
    double v;
    if (e == 15 && f == 7) return NAN;
    v = (e == 0) ? ldexp((double)f, -9) : ldexp((double)(8 + f), e - 10);
    return s ? -v : v;
}

/* Round-to-nearest-even of x to a binary format with `p` significant bits and
 * minimum normal exponent `emin` (value quantum 2^(max(e,emin)-(p-1))). */
static double ora_round_rne(double x, int p, int emin)
{
    int ex;
    double ax = fabs(x), q, n;
    if (ax == 0.0) return x;
    frexp(ax, &ex);                 /* ax = fr * 2^ex, fr in [0.5,1) */
    ex -= 1;                        /* ax in [2^ex, 2^(ex+1)) */
    if (ex < emin) ex = emin;
    q = ldexp(1.0, ex - (p - 1));
    n = nearbyint(ax / q);          /* default rounding mode: ties to even */
    return copysign(n * q, x);
}

/* bf16 encoding by round-to-nearest-even (overflow to infinity). */
uint16_t ora_bf16_round(double x)
{
    double r = ora_round_rne(x, 8, -126);
    float f;
    uint32_t u;
    if (fabs(r) >= ldexp(1.0, 128)) r = copysign(INFINITY, x);
    f = (float)r;                   /* exact: r is a bf16 value */
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* e4m3 encoding by round-to-nearest-even, saturating to +-448. */
uint8_t ora_e4m3_round(double x)
{
    double r = ora_round_rne(x, 4, -6);
    int c;
    if (r > 448.0) r = 448.0;
    if (r < -448.0) r = -448.0;
    for (c = 0; c < 0x7f; ++c)
        if (ora_e4m3_value((uint8_t)c) == fabs(r))
            return (uint8_t)((signbit(r) ? 0x80 : 0) | c);
    return 0x7f; /* unreachable for finite x */
}

/* ------------------------------------------------------------------------- */
/* Exact dot product, rounded once to fp32                                  */
/* ------------------------------------------------------------------------- */
/* Each bf16 / e4m3 value is an integer significand times a power of two, so
 * the exact sum of products is an integer multiple of 2^ORA_EMIN.  It is held
 * in a long fixed-point accumulator (Kulisch's exact dot product): digits of
 * 32 bits kept in int64 so that carries can wait until the end. */
#define ORA_EMIN (-300)
#define ORA_NDIG 20

typedef struct { int64_t d[ORA_NDIG]; } ora_acc;

/* value = (-1)^neg * M * 2^e; returns -1 for NaN / infinity. */
static int ora_decode(const void* base, int i, int dtype, int* neg, uint32_t* M, int* e)
{
    if (dtype == ORA_BF16) {
        uint16_t h = ((const uint16_t*)base)[i];
        int E = (h >> 7) & 0xff, f = h & 0x7f;
        *neg = h >> 15;
        if (E == 0xff) return -1;
        if (E == 0) { *M = (uint32_t)f; *e = -133; }
        else { *M = 128u + (uint32_t)f; *e = E - 134; }
    } else {
        uint8_t b = ((const uint8_t*)base)[i];
        int E = (b >> 3) & 15, f = b & 7;
        *neg = b >> 7;
        if (E == 15 && f == 7) return -1;
        if (E == 0) { *M = (uint32_t)f; *e = -9; }
        else { *M = 8u + (uint32_t)f; *e = E - 10; }
    }
    return 0;
}

static void ora_acc_add(ora_acc* a, int neg, uint64_t M, int e)
{
    int pos, j, b;
    uint64_t v;
    int64_t lo, hi;
    if (M == 0) return;
    pos = e - ORA_EMIN;             /* >= 0 for all bf16 / e4m3 products */
    j = pos >> 5;
    b = pos & 31;
    v = M << b;                     /* M < 2^16, so v < 2^47 */
    lo = (int64_t)(v & 0xffffffffu);
    hi = (int64_t)(v >> 32);
    if (neg) { lo = -lo; hi = -hi; }
    a->d[j] += lo;
    a->d[j + 1] += hi;
}

static void ora_acc_normalize(ora_acc* a)
{
    int j;
    for (j = 0; j < ORA_NDIG - 1; ++j) {
        int64_t c = a->d[j] >> 32;              /* floor division by 2^32 */
        a->d[j] -= c * 4294967296LL;
        a->d[j + 1] += c;
    }
}

static int ora_acc_bit(const ora_acc* a, int i)
{
    return (int)((a->d[i >> 5] >> (i & 31)) & 1);
}

/* Round the accumulated exact value to fp32, ties to even. */
static float ora_acc_to_f32(ora_acc* a)
{
    int neg, j, P = -1, R, i, rnd, sticky;
    uint64_t T = 0;
    double v;
    ora_acc_normalize(a);
    neg = a->d[ORA_NDIG - 1] < 0;
    if (neg) {
        for (j = 0; j < ORA_NDIG; ++j) a->d[j] = -a->d[j];
        ora_acc_normalize(a);
    }
    for (i = 32 * ORA_NDIG - 1; i >= 0; --i)
        if (ora_acc_bit(a, i)) { P = i; break; }
    if (P < 0) return 0.0f;                    /* exact zero -> +0 */
    /* keep bits P..R: 24 bits, or fewer below the fp32 subnormal quantum */
    R = P - 23;
    if (R < -149 - ORA_EMIN) R = -149 - ORA_EMIN;
    if (R <= 0) {
        for (i = P; i >= 0; --i) T = (T << 1) | (uint64_t)ora_acc_bit(a, i);
        v = ldexp((double)T, ORA_EMIN);
    } else {
        for (i = P; i >= R; --i) T = (T << 1) | (uint64_t)ora_acc_bit(a, i);
        rnd = ora_acc_bit(a, R - 1);
        sticky = 0;
        for (i = R - 2; i >= 0 && !sticky; --i) sticky = ora_acc_bit(a, i);
        if (rnd && (sticky || (T & 1))) T += 1;
        v = ldexp((double)T, R + ORA_EMIN);
    }
    if (v >= ldexp(1.0, 128)) return neg ? -INFINITY : INFINITY;
    return neg ? -(float)v : (float)v;
}

/* Exact sum_i a[i]*b[i] of n bf16 / e4m3 values, rounded once to fp32.
 * Returns NaN if any input is NaN or infinite (inputs are assumed finite). */
float ora_exact_dot_f32(const void* a, const void* b, int n, int dtype)
{
    ora_acc acc;
    int i;
    memset(&acc, 0, sizeof acc);
    for (i = 0; i < n; ++i) {
        int na, nb, ea, eb;
        uint32_t Ma, Mb;
        if (ora_decode(a, i, dtype, &na, &Ma, &ea) || ora_decode(b, i, dtype, &nb, &Mb, &eb))
            return NAN;
        ora_acc_add(&acc, na ^ nb, (uint64_t)Ma * Mb, ea + eb);
    }
    return ora_acc_to_f32(&acc);
}

/* ------------------------------------------------------------------------- */
/* Visibility of compressed entries                                          */
/* ------------------------------------------------------------------------- */
/* Entry j of a ratio-m compression of L tokens covers raw tokens
 * [j*m, min((j+1)*m, L)) [P3 item 1: the sequence shrinks to 1/m; P2 first
 * section: every m tokens become one entry].  A query at absolute position p
 * may use entry j only once all of its tokens are at or before p (causal at
 * block granularity).  Counted literally. */
int ora_n_visible(long long p, long long L, int m)
{
    long long Nc = (L + m - 1) / m, j;
    int n = 0;
    for (j = 0; j < Nc; ++j) {
        long long last = ((j + 1) * m < L ? (j + 1) * m : L) - 1;
        if (last <= p) ++n;
    }
    return n;
}

/* ------------------------------------------------------------------------- */
/* A1: token-level compressor                                                */
/* ------------------------------------------------------------------------- */
/* [P1 section 1.1]: a token-level compressor merges the KV of every m tokens
 * into one entry; [P2 first section] and [P3 item 1] say the same for CSA,
 * and HCA does it with a much larger m'.  The pages do not print the pooling
 * weights.  Reading taken: softmax-gated pooling within the block,
 *   z_t = X_t . w_gate + b_slot[t - j*m],   a = softmax_{t in block}(z),
 *   kv_j = sum_t a_t (X_t W_kv^T),  ik_j = sum_t a_t (X_t W_ik^T),
 * which is the block mean when w_gate = 0 and b_slot = 0.  Projection first,
 * then pooling, exactly as the sentence reads ("compress the KV").
 * Layouts: hidden[B][L][Dh], w_kv[D][Dh], w_ik[dI][Dh] (output-major, like a
 * linear layer's weight), w_gate[Dh], b_slot[m] (NULL = zeros).
 * Only entries j0..j1-1 are computed: kv_out[B][j1-j0][D], ik_out[B][j1-j0][dI].
 * The window rows are the un-pooled projected KV of the last W tokens,
 * win_out[B][W][D], row u <-> raw token L-W+u (zero rows for negative
 * positions).  Any output pointer may be NULL. */
void ora_compress(int B, int L, int Dh, int D, int dI, int m, int W,
                  const uint16_t* hidden, const uint16_t* w_kv, const uint16_t* w_ik,
                  const float* w_gate, const float* b_slot,
                  int j0, int j1, double* kv_out, double* ik_out, double* win_out)
{
    int b;
    int nj = j1 - j0;
    for (b = 0; b < B; ++b) {
        const uint16_t* X = hidden + (size_t)b * L * Dh;
        int jj;
        #pragma omp parallel for schedule(dynamic)
        for (jj = 0; jj < nj; ++jj) {
            int j = j0 + jj, t0 = j * m, t1 = (j + 1) * m < L ? (j + 1) * m : L;
            int nt = t1 - t0, t, i, n;
            double* z = (double*)malloc(sizeof(double) * nt);
            double zmax = -INFINITY, zsum = 0.0;
            for (t = 0; t < nt; ++t) {
                double s = 0.0;
                for (i = 0; i < Dh; ++i)
                    s += ora_bf16_value(X[(size_t)(t0 + t) * Dh + i]) * (double)w_gate[i];
                z[t] = s + (b_slot ? (double)b_slot[t] : 0.0);
                if (z[t] > zmax) zmax = z[t];
            }
            for (t = 0; t < nt; ++t) { z[t] = exp(z[t] - zmax); zsum += z[t]; }
            for (t = 0; t < nt; ++t) z[t] /= zsum;        /* a_t */
            if (kv_out) {
                for (n = 0; n < D; ++n) {
                    double acc = 0.0;
                    for (t = 0; t < nt; ++t) {
                        double y = 0.0;                    /* (X_t W_kv^T)[n] */
                        for (i = 0; i < Dh; ++i)
                            y += ora_bf16_value(X[(size_t)(t0 + t) * Dh + i]) *
                                 ora_bf16_value(w_kv[(size_t)n * Dh + i]);
                        acc += z[t] * y;
                    }
                    kv_out[((size_t)b * nj + jj) * D + n] = acc;
                }
            }
            if (ik_out && w_ik) {
                for (n = 0; n < dI; ++n) {
                    double acc = 0.0;
                    for (t = 0; t < nt; ++t) {
                        double y = 0.0;
                        for (i = 0; i < Dh; ++i)
                            y += ora_bf16_value(X[(size_t)(t0 + t) * Dh + i]) *
                                 ora_bf16_value(w_ik[(size_t)n * Dh + i]);
                        acc += z[t] * y;
                    }
                    ik_out[((size_t)b * nj + jj) * dI + n] = acc;
                }
            }
            free(z);
        }
        if (win_out) {
            int u;
            #pragma omp parallel for
            for (u = 0; u < W; ++u) {
                int t = L - W + u, n, i;
                for (n = 0; n < D; ++n) {
                    double y = 0.0;
                    if (t >= 0)
                        for (i = 0; i < Dh; ++i)
                            y += ora_bf16_value(X[(size_t)t * Dh + i]) *
                                 ora_bf16_value(w_kv[(size_t)n * Dh + i]);
                    win_out[((size_t)b * W + u) * D + n] = y;
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* A2: Lightning-Indexer scores                                              */
/* ------------------------------------------------------------------------- */
/* [P1 section 1.1]: a light "Lightning Indexer" scores each compressed entry
 * against the query; [P2 "mHC、Muon、FP4"] runs its QK path in low precision.
 * The score formula is not printed on the pages.  Reading taken: one indexer
 * key per entry shared by HI indexer heads, per-query head weights w_h, and
 *   S = sum_h w_h * ReLU(q_h . k),
 * made bit-reproducible ("canonical"): each q_h . k is the exact dot product
 * rounded once to fp32, ReLU maps <= 0 to +0, and the head sum is the fp32
 * fused-multiply-add chain S = fma(w_h, r_h, S) over h = 0..HI-1 from S = +0.
 * q_idx[B][Tq][HI][dI], w_idx[B][Tq][HI], k_idx[B][Nc][dI]; query t sits at
 * absolute position pos0+t.  Invisible entries get NaN.  n_vis[B][Tq] gets the
 * number of visible entries (always a prefix 0..n_vis-1). */
float ora_index_score(const void* q, const float* w, const void* k, int HI, int dI, int dtype)
{
    float S = 0.0f;
    int h;
    size_t es = dtype == ORA_BF16 ? 2 : 1;
    for (h = 0; h < HI; ++h) {
        float d = ora_exact_dot_f32((const char*)q + (size_t)h * dI * es, k, dI, dtype);
        float r = d > 0.0f ? d : 0.0f;
        S = fmaf(w[h], r, S);
    }
    return S;
}

void ora_index_scores(int B, int Tq, int HI, int dI, int Nc, long long L, int m, long long pos0,
                      int dtype, const void* q_idx, const float* w_idx, const void* k_idx,
                      float* S_out, int* n_vis_out)
{
    size_t es = dtype == ORA_BF16 ? 2 : 1;
    int b, t;
    for (b = 0; b < B; ++b)
        for (t = 0; t < Tq; ++t) {
            int nv = ora_n_visible(pos0 + t, L, m), j;
            const char* q = (const char*)q_idx + ((size_t)b * Tq + t) * HI * dI * es;
            const float* w = w_idx + ((size_t)b * Tq + t) * HI;
            float* S = S_out + ((size_t)b * Tq + t) * Nc;
            if (nv > Nc) nv = Nc;
            n_vis_out[(size_t)b * Tq + t] = nv;
            #pragma omp parallel for schedule(static)
            for (j = 0; j < Nc; ++j) {
                if (j < nv)
                    S[j] = ora_index_score(q, w, (const char*)k_idx + ((size_t)b * Nc + j) * dI * es,
                                           HI, dI, dtype);
                else
                    S[j] = NAN;
            }
        }
}

/* ------------------------------------------------------------------------- */
/* A3: per-query top-k                                                       */
/* ------------------------------------------------------------------------- */
/* [P1 section 1.1]: a top-k selector keeps the k most relevant compressed
 * entries (Pro keeps 1024); [P2 first section]: each query looks only at its
 * own top-k.  Order: score descending, ties by lower index (+0 == -0 as IEEE
 * values).  Output: the first min(k, n_vis) entries in that order, written in
 * ascending index order and padded with -1; cnt = min(k, n_vis). */
typedef struct { float s; int j; } ora_sj;

static int ora_cmp_sj(const void* x, const void* y)
{
    const ora_sj* a = (const ora_sj*)x;
    const ora_sj* b = (const ora_sj*)y;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int ora_cmp_int(const void* x, const void* y)
{
    int a = *(const int*)x, b = *(const int*)y;
    return (a > b) - (a < b);
}

void ora_topk(int rows, int Nc, int k, const float* S, const int* n_vis, int* idx_out, int* cnt_out)
{
    int r;
    #pragma omp parallel for schedule(dynamic)
    for (r = 0; r < rows; ++r) {
        int nv = n_vis[r], j, c;
        ora_sj* v = (ora_sj*)malloc(sizeof(ora_sj) * (nv > 0 ? nv : 1));
        int* sel = idx_out + (size_t)r * k;
        for (j = 0; j < nv; ++j) { v[j].s = S[(size_t)r * Nc + j]; v[j].j = j; }
        qsort(v, (size_t)nv, sizeof(ora_sj), ora_cmp_sj);
        c = nv < k ? nv : k;
        for (j = 0; j < c; ++j) sel[j] = v[j].j;
        qsort(sel, (size_t)c, sizeof(int), ora_cmp_int);
        for (j = c; j < k; ++j) sel[j] = -1;
        if (cnt_out) cnt_out[r] = c;
        free(v);
    }
}

/* ------------------------------------------------------------------------- */
/* A4 / A5: MQA attention over a key set                                     */
/* ------------------------------------------------------------------------- */
/* [P1 section 1.1]: core attention is Multi-Query Attention (all query heads
 * share one KV head).  Reading taken: one vector per entry is both key and
 * value.  For head h: l_r = scale * (q_h . x_r), o_h = sum_r softmax(l)_r x_r,
 * lse_h = log sum_r exp(l_r).  An empty key set gives o = 0, lse = -inf. */
/* One softmax per head over the rows' logits l_r = scale (q_h . x_r) and, when sink is given, the head's
 * attention-sink logit sink[h] (a term of the denominator with no value row): [P1 section 1.1] gives
 * every query head a learnable sink logit that lets it send its total attention towards 0.
 * out_h = sum_r e^{l_r} y_r / (e^{sink_h} + sum_r e^{l_r}),  lse_h = log(e^{sink_h} + sum_r e^{l_r}),
 * where y_r = vals[r] when vals is given (separate values) and y_r = x_r otherwise. */
static void ora_attend(const uint16_t* q, int H, int D, const uint16_t** rows, const uint16_t** vals, int nr,
                       double scale, const double* sink, double* out, double* lse)
{
    int h, r, d;
    double* l = (double*)malloc(sizeof(double) * (nr > 0 ? nr : 1));
    for (h = 0; h < H; ++h) {
        double mx = sink ? sink[h] : -INFINITY, s = 0.0;
        for (r = 0; r < nr; ++r) {
            double dot = 0.0;
            for (d = 0; d < D; ++d)
                dot += ora_bf16_value(q[(size_t)h * D + d]) * ora_bf16_value(rows[r][d]);
            l[r] = scale * dot;
            if (l[r] > mx) mx = l[r];
        }
        for (d = 0; d < D; ++d) out[(size_t)h * D + d] = 0.0;
        if (mx == -INFINITY) { lse[h] = -INFINITY; continue; }     /* no row and no sink */
        for (r = 0; r < nr; ++r) { l[r] = exp(l[r] - mx); s += l[r]; }
        if (sink) s += exp(sink[h] - mx);
        for (r = 0; r < nr; ++r) {
            const uint16_t* y = vals ? vals[r] : rows[r];
            for (d = 0; d < D; ++d)
                out[(size_t)h * D + d] += l[r] * ora_bf16_value(y[d]);
        }
        for (d = 0; d < D; ++d) out[(size_t)h * D + d] /= s;
        lse[h] = mx + log(s);
    }
    free(l);
}

/* A4: CSA core attention.  [P1 section 1.1]: attention runs over the top-k
 * compressed entries, plus an extra sliding-window branch over raw local
 * tokens (window length not printed; taken as a parameter W); [P3 item 1]
 * keeps "a few sliding-window local KV entries".  Reading taken: one softmax
 * over the union of the selected entries and the raw window tokens
 * [max(0, p-W+1), p] (the current token included, no de-duplication).
 * q[B][Tq][H][D], kv[B][Nc][D], idx[B][Tq][topk] (-1 = unused),
 * kv_raw[B][Lr][D] holds raw positions raw0..raw0+Lr-1.
 * v[B][Nc][D] and v_raw[B][Lr][D], when given (both or neither), are separate values of the entries and raw
 * rows (the variant that keeps keys and values apart; NULL: each row is its own value).
 * out[B][Tq][H][D], lse[B][Tq][H].  Returns -1 on an out-of-range index. */
int ora_sparse_attn(int B, int Tq, int H, int D, int Nc, int topk, int Lr, long long raw0,
                    long long pos0, int W, double scale,
                    const uint16_t* q, const uint16_t* kv, const int* idx, const uint16_t* kv_raw,
                    const uint16_t* v, const uint16_t* v_raw,
                    const double* sink, double* out, double* lse)
{
    int bt, bad = 0;
    #pragma omp parallel for schedule(dynamic) reduction(|:bad)
    for (bt = 0; bt < B * Tq; ++bt) {
        int b = bt / Tq, t = bt % Tq, i, nr = 0;
        long long p = pos0 + t, u, w0 = p - W + 1 < 0 ? 0 : p - W + 1;
        const uint16_t** rows = (const uint16_t**)malloc(sizeof(void*) * (topk + W + 1));
        const uint16_t** vals = (const uint16_t**)malloc(sizeof(void*) * (topk + W + 1));
        for (i = 0; i < topk; ++i) {
            int j = idx[(size_t)bt * topk + i];
            if (j < 0) continue;
            if (j >= Nc) { bad = 1; continue; }
            rows[nr] = kv + ((size_t)b * Nc + j) * D;
            vals[nr++] = v ? v + ((size_t)b * Nc + j) * D : NULL;
        }
        for (u = w0; W > 0 && u <= p; ++u) {
            if (u < raw0 || u >= raw0 + Lr) { bad = 1; continue; }
            rows[nr] = kv_raw + ((size_t)b * Lr + (size_t)(u - raw0)) * D;
            vals[nr++] = v_raw ? v_raw + ((size_t)b * Lr + (size_t)(u - raw0)) * D : NULL;
        }
        ora_attend(q + (size_t)bt * H * D, H, D, rows, v ? vals : NULL, nr, scale, sink,
                   out + (size_t)bt * H * D, lse + (size_t)bt * H);
        free(rows);
        free(vals);
    }
    return bad ? -1 : 0;
}

/* A5: HCA attention.  [P1 section 1.1], [P3 item 2]: every m' tokens become
 * one entry and attention is dense over all compressed entries, with no
 * selection.  Reading taken: no sliding window in HCA.  Entries visible to the
 * query at p as defined above.  q[B][Tq][H][D], kv_h[B][Nh][D]; v_h[B][Nh][D] separate values or NULL. */
void ora_dense_attn(int B, int Tq, int H, int D, int Nh, long long L, int mh, long long pos0,
                    double scale, const uint16_t* q, const uint16_t* kv_h, const uint16_t* v_h, const double* sink,
                    double* out, double* lse)
{
    int bt;
    #pragma omp parallel for schedule(dynamic)
    for (bt = 0; bt < B * Tq; ++bt) {
        int b = bt / Tq, t = bt % Tq, j;
        int nv = ora_n_visible(pos0 + t, L, mh);
        const uint16_t** rows = (const uint16_t**)malloc(sizeof(void*) * (nv > 0 ? nv : 1));
        const uint16_t** vals = (const uint16_t**)malloc(sizeof(void*) * (nv > 0 ? nv : 1));
        if (nv > Nh) nv = Nh;
        for (j = 0; j < nv; ++j) {
            rows[j] = kv_h + ((size_t)b * Nh + j) * D;
            vals[j] = v_h ? v_h + ((size_t)b * Nh + j) * D : NULL;
        }
        ora_attend(q + (size_t)bt * H * D, H, D, rows, v_h ? vals : NULL, nv, scale, sink,
                   out + (size_t)bt * H * D, lse + (size_t)bt * H);
        free(rows);
        free(vals);
    }
}

/* ---- C11: partial rotary position embedding ----------------------------------------------------------
 * [P1 section 1.1]: the rotary position embedding acts only on the last 64 dimensions of a query / KV
 * vector, and the core attention output receives the inverse rotation at the query's position, which
 * restores the relative-position structure.  The pages print no formula; the rotation is the standard
 * rotary embedding with adjacent-pair (interleaved) pairing over the last rd dimensions:
 *   pair j = (D-rd+2j, D-rd+2j+1), frequency f_j = theta^(-2j/rd), angle a = pos * f_j,
 *   (u, v) -> (u cos a - v sin a, u sin a + v cos a); the inverse uses -a.
 * Row r of x (bf16 [n][D]) takes position pos[r / group]; the first D-rd dimensions pass unchanged.
 * y is fp64 [n][D]. */
void ora_rope(int n, int D, int rd, int group, double theta, int inverse, const uint16_t* x,
              const long long* pos, double* y)
{
    for (int r = 0; r < n; ++r) {
        const double p = (double)pos[r / group];
        const uint16_t* xr = x + (size_t)r * D;
        double* yr = y + (size_t)r * D;
        for (int d = 0; d < D - rd; ++d) yr[d] = ora_bf16_value(xr[d]);
        for (int j = 0; j < rd / 2; ++j) {
            const double f = pow(theta, -2.0 * j / rd);
            const double a = (inverse ? -p : p) * f;
            const double u = ora_bf16_value(xr[D - rd + 2 * j]), v = ora_bf16_value(xr[D - rd + 2 * j + 1]);
            yr[D - rd + 2 * j] = u * cos(a) - v * sin(a);
            yr[D - rd + 2 * j + 1] = u * sin(a) + v * cos(a);
        }
    }
}

/* ---- C12: FP8 storage of the non-RoPE KV dimensions ----------------------------------------------------
 * [P1 section 1.1, last paragraph]: the KV cache keeps its RoPE dimensions in BF16 and the other dimensions
 * in FP8.  The pages print no scale scheme.  Reading taken: a D-wide KV row (its first D - 64 dimensions,
 * then the 64 RoPE dimensions of C11) is stored in D + 80 bytes:
 *   bytes [0, D-64)        OCP e4m3 codes of x_i / 2^e_g, group g = i / 64 of the non-RoPE dimensions,
 *   bytes [D-64, D+64)     the 64 RoPE dimensions as they were (bf16),
 *   bytes [D+64, D+80)     e_g + 127 for each group (one byte each, the unused bytes 0),
 * where e_g is the smallest integer with max_{i in g} |x_i| <= 448 * 2^e_g (0 for an all-zero group): no code
 * saturates and the division by 2^e_g is exact, so each code is the e4m3 rounding (to nearest, ties to
 * even) of its value.  A dimension decodes to e4m3(code) * 2^e_g. */
int ora_kv_fp8_row_bytes(int D) { return D + 80; }

void ora_kv_fp8_encode(int n, int D, const uint16_t* x, uint8_t* y)
{
    const int nope = D - 64, rb = D + 80;
    for (int r = 0; r < n; ++r) {
        const uint16_t* xr = x + (size_t)r * D;
        uint8_t* yr = y + (size_t)r * rb;
        memset(yr, 0, (size_t)rb);
        for (int g = 0; g < nope / 64; ++g) {
            double amax = 0.0;
            for (int i = 64 * g; i < 64 * g + 64; ++i) {
                const double a = fabs(ora_bf16_value(xr[i]));
                if (a > amax) amax = a;
            }
            int e = 0;
            if (amax > 0.0) {
                e = -200;
                while (amax > ldexp(448.0, e)) ++e;            /* the smallest e with amax <= 448 * 2^e */
            }
            yr[D + 64 + g] = (uint8_t)(e + 127);
            for (int i = 64 * g; i < 64 * g + 64; ++i)
                yr[i] = ora_e4m3_round(ldexp(ora_bf16_value(xr[i]), -e));
        }
        memcpy(yr + nope, xr + nope, 128);
    }
}

void ora_kv_fp8_decode(int n, int D, const uint8_t* y, double* x)
{
    const int nope = D - 64, rb = D + 80;
    for (int r = 0; r < n; ++r) {
        const uint8_t* yr = y + (size_t)r * rb;
        double* xr = x + (size_t)r * D;
        for (int i = 0; i < nope; ++i) xr[i] = ldexp(ora_e4m3_value(yr[i]), (int)yr[D + 64 + i / 64] - 127);
        for (int i = 0; i < 64; ++i) {
            uint16_t h;
            memcpy(&h, yr + nope + 2 * i, 2);
            xr[nope + i] = ora_bf16_value(h);
        }
    }
}

/* ---- C13: MXFP4 operands of the Lightning Indexer ------------------------------------------------------
 * [P2 "mHC、Muon、FP4：这些不是论文装饰"]: the indexer's QK path runs in FP4.  The pages print no format.
 * Reading taken: the OCP Microscaling (MX) FP4 format -- blocks of 32 consecutive elements share a
 * power-of-two scale 2^X stored as the byte X + 127 (E8M0); each element is an E2M1 code (sign, 2 exponent
 * bits, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte, element 2i in the low nibble.
 * Encoding follows the MX specification: X = floor(log2(max |x|)) - 2 (2 = the largest E2M1 exponent),
 * clamped to [-127, 127] (X = -127 for an all-zero block); each x / 2^X rounds to the nearest E2M1 magnitude,
 * ties to the even code, saturating at 6.  Scores are the canonical scores of A2 over the decoded values. */
static const double ora_e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static uint8_t ora_e2m1_round(double v)
{
    const double a = fabs(v);
    int best = 0;
    for (int k = 1; k < 8; ++k) {
        const double dk = fabs(a - ora_e2m1_mag[k]), db = fabs(a - ora_e2m1_mag[best]);
        if (dk < db || (dk == db && (k & 1) == 0)) best = k;
    }
    if (a >= 6.0) best = 7;
    return (uint8_t)((v < 0.0 && best != 0 ? 8 : 0) | best);
}

void ora_mxfp4_encode(int n, int len, const uint16_t* x, uint8_t* codes, uint8_t* scales)
{
    for (int r = 0; r < n; ++r) {
        const uint16_t* xr = x + (size_t)r * len;
        uint8_t* cr = codes + (size_t)r * (len / 2);
        uint8_t* sr = scales + (size_t)r * (len / 32);
        memset(cr, 0, (size_t)len / 2);
        for (int blk = 0; blk < len / 32; ++blk) {
            double amax = 0.0;
            for (int i = 32 * blk; i < 32 * blk + 32; ++i) {
                const double a = fabs(ora_bf16_value(xr[i]));
                if (a > amax) amax = a;
            }
            int X = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);                          /* amax in [2^(ex-1), 2^ex) */
                X = (ex - 1) - 2;
                if (X < -127) X = -127;
                if (X > 127) X = 127;
            }
            sr[blk] = (uint8_t)(X + 127);
            for (int i = 32 * blk; i < 32 * blk + 32; ++i) {
                const uint8_t c = ora_e2m1_round(ldexp(ora_bf16_value(xr[i]), -X));
                cr[i / 2] |= (uint8_t)(i & 1 ? c << 4 : c);
            }
        }
    }
}

/* element i of an MXFP4 vector as (-1)^neg M 2^e */
static void ora_mx_decode(const uint8_t* codes, const uint8_t* scales, int i, int* neg, uint32_t* M, int* e)
{
    const uint8_t c = (uint8_t)((codes[i / 2] >> (4 * (i & 1))) & 15);
    const int k = c & 7, E = k >> 1, mb = k & 1;
    *neg = c >> 3;
    if (E == 0) { *M = (uint32_t)mb; *e = -1; }
    else { *M = 2u + (uint32_t)mb; *e = E - 2; }
    *e += (int)scales[i / 32] - 127;
}

double ora_mxfp4_value(const uint8_t* codes, const uint8_t* scales, int i)
{
    int neg, e;
    uint32_t M;
    ora_mx_decode(codes, scales, i, &neg, &M, &e);
    return (neg ? -1.0 : 1.0) * ldexp((double)M, e);
}

/* exact sum_i a_i b_i of two MXFP4 vectors of n elements, rounded once to fp32 */
float ora_exact_dot_mxfp4(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs, int n)
{
    ora_acc acc;
    memset(&acc, 0, sizeof acc);
    for (int i = 0; i < n; ++i) {
        int na, nb, ea, eb;
        uint32_t Ma, Mb;
        ora_mx_decode(ac, as, i, &na, &Ma, &ea);
        ora_mx_decode(bc, bs, i, &nb, &Mb, &eb);
        ora_acc_add(&acc, na ^ nb, (uint64_t)Ma * Mb, ea + eb);
    }
    return ora_acc_to_f32(&acc);
}

/* Canonical scores (A2) over MXFP4 operands: q codes [B][Tq][HI][dI/2] and scales [B][Tq][HI][dI/32], k codes
 * [B][Nc][dI/2] and scales [B][Nc][dI/32]; the rest as ora_index_scores. */
void ora_index_scores_mxfp4(int B, int Tq, int HI, int dI, int Nc, long long L, int m, long long pos0,
                            const uint8_t* qc, const uint8_t* qs, const float* w_idx, const uint8_t* kc,
                            const uint8_t* ks, float* S_out, int* n_vis_out)
{
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < Tq; ++t) {
            int nv = ora_n_visible(pos0 + t, L, m), j;
            const size_t r = (size_t)b * Tq + t;
            const float* w = w_idx + r * HI;
            float* S = S_out + r * Nc;
            if (nv > Nc) nv = Nc;
            n_vis_out[r] = nv;
            #pragma omp parallel for schedule(static)
            for (j = 0; j < Nc; ++j) {
                if (j >= nv) { S[j] = NAN; continue; }
                float Sx = 0.0f;
                const size_t kr = (size_t)b * Nc + j;
                for (int h = 0; h < HI; ++h) {
                    const size_t qr = r * HI + h;
                    const float d = ora_exact_dot_mxfp4(qc + qr * (dI / 2), qs + qr * (dI / 32), kc + kr * (dI / 2),
                                                        ks + kr * (dI / 32), dI);
                    Sx = fmaf(w[h], d > 0.0f ? d : 0.0f, Sx);
                }
                S[j] = Sx;
            }
        }
}

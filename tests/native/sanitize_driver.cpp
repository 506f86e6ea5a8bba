// Host build under AddressSanitizer + UndefinedBehaviorSanitizer of the two pieces of plain C/C++ in this
// repository: the CPU oracle (oracle/oracle.c, test infrastructure) and the library's exact-rescoring header
// (csrc/exact_dot.h).  Every oracle routine runs on small seeded inputs (memory errors and undefined behaviour
// abort the run), and the header's exact dot products are compared bit for bit with the oracle's on random,
// cancelling and wide-span inputs.  Exit status 0 = clean and equal.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "exact_dot.h"

extern "C" {
double ora_bf16_value(uint16_t h);
uint16_t ora_bf16_round(double x);
uint8_t ora_e4m3_round(double x);
float ora_exact_dot_f32(const void* a, const void* b, int n, int dtype);
int ora_n_visible(long long p, long long L, int m);
void ora_compress(int B, int L, int Dh, int D, int dI, int m, int W, const uint16_t* hidden, const uint16_t* w_kv,
                  const uint16_t* w_ik, const float* w_gate, const float* b_slot, int j0, int j1, double* kv_out,
                  double* ik_out, double* win_out);
float ora_index_score(const void* q, const float* w, const void* k, int HI, int dI, int dtype);
void ora_index_scores(int B, int Tq, int HI, int dI, int Nc, long long L, int m, long long pos0, int dtype,
                      const void* q_idx, const float* w_idx, const void* k_idx, float* S_out, int* n_vis_out);
void ora_topk(int rows, int Nc, int k, const float* S, const int* n_vis, int* idx_out, int* cnt_out);
int ora_sparse_attn(int B, int Tq, int H, int D, int Nc, int topk, int Lr, long long raw0, long long pos0, int W,
                    double scale, const uint16_t* q, const uint16_t* kv, const int* idx, const uint16_t* kv_raw,
                    const uint16_t* v, const uint16_t* v_raw, const double* sink, double* out, double* lse);
void ora_dense_attn(int B, int Tq, int H, int D, int Nh, long long L, int mh, long long pos0, double scale,
                    const uint16_t* q, const uint16_t* kv_h, const uint16_t* v_h, const double* sink, double* out,
                    double* lse);
void ora_rope(int n, int D, int rd, int group, double theta, int inverse, const uint16_t* x, const long long* pos,
              double* y);
void ora_kv_fp8_encode(int n, int D, const uint16_t* x, uint8_t* y);
void ora_kv_fp8_decode(int n, int D, const uint8_t* y, double* x);
void ora_mxfp4_encode(int n, int len, const uint16_t* x, uint8_t* codes, uint8_t* scales);
float ora_exact_dot_mxfp4(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs, int n);
}

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64() {                       // splitmix64
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static double uniform() { return (double)(next_u64() >> 11) * 0x1.0p-53; }
static double normal() {
    const double u = uniform() + 1e-300, v = uniform();
    return std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v);
}
static std::vector<uint16_t> bf16_vec(size_t n, double s) {
    std::vector<uint16_t> x(n);
    for (auto& e : x) e = ora_bf16_round(normal() * s);
    return x;
}

static int g_fail = 0;
static void check(bool ok, const char* what, int i) {
    if (!ok && g_fail++ < 20) std::fprintf(stderr, "mismatch: %s (case %d)\n", what, i);
}
static uint32_t bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

int main() {
    // 1. exact dot products: header vs oracle, bf16 and e4m3, several magnitudes and spans
    for (int it = 0; it < 400; ++it) {
        const int n = 1 + (int)(next_u64() % 256);
        const double span = (it % 4 == 0) ? 40.0 : 3.0;
        std::vector<uint16_t> a(n), b(n);
        std::vector<uint8_t> a8(n), b8(n);
        for (int i = 0; i < n; ++i) {
            const double sa = std::ldexp(1.0, (int)((uniform() - 0.5) * span));
            const double sb = std::ldexp(1.0, (int)((uniform() - 0.5) * span));
            a[i] = ora_bf16_round(normal() * sa);
            b[i] = ora_bf16_round(normal() * sb);
            a8[i] = ora_e4m3_round(normal() * 8.0);
            b8[i] = ora_e4m3_round(normal() * 8.0);
        }
        if (it % 7 == 0) for (int i = 0; i + 1 < n; i += 2) { a[i + 1] = a[i]; b[i + 1] = b[i] ^ 0x8000u; }
        const float o16 = ora_exact_dot_f32(a.data(), b.data(), n, 0);
        const float o8 = ora_exact_dot_f32(a8.data(), b8.data(), n, 1);
        check(bits(csa_exact::exact_dot<0>(a.data(), b.data(), n)) == bits(o16), "exact_dot bf16", it);
        check(bits(csa_exact::exact_dot_wide<0>(a.data(), b.data(), n)) == bits(o16), "exact_dot_wide bf16", it);
        check(bits(csa_exact::exact_dot<1>(a8.data(), b8.data(), n)) == bits(o8), "exact_dot e4m3", it);
        check(bits(csa_exact::exact_dot_wide<1>(a8.data(), b8.data(), n)) == bits(o8), "exact_dot_wide e4m3", it);
    }
    // 2. indexer scores: header vs oracle
    {
        const int HI = 8, dI = 128;
        for (int it = 0; it < 50; ++it) {
            auto q = bf16_vec((size_t)HI * dI, 1.0 / 11.3), k = bf16_vec(dI, 1.0 / 11.3);
            std::vector<float> w(HI);
            for (auto& e : w) e = (float)std::fabs(normal()) / 2.83f;
            check(bits(csa_exact::exact_score<0>(q.data(), w.data(), k.data(), HI, dI)) ==
                      bits(ora_index_score(q.data(), w.data(), k.data(), HI, dI, 0)), "exact_score", it);
        }
    }
    // 3. every oracle routine on small inputs (the sanitizers watch the memory accesses)
    {
        const int B = 2, L = 37, Dh = 64, D = 32, dI = 16, m = 4, W = 5, Nc = (L + m - 1) / m;
        auto X = bf16_vec((size_t)B * L * Dh, 1.0), wkv = bf16_vec((size_t)D * Dh, 0.125), wik = bf16_vec((size_t)dI * Dh, 0.125);
        std::vector<float> wg(Dh), bs(m);
        for (auto& e : wg) e = (float)(normal() * 0.125);
        for (auto& e : bs) e = (float)(normal() * 0.5);
        std::vector<double> kv((size_t)B * Nc * D), ik((size_t)B * Nc * dI), win((size_t)B * W * D);
        ora_compress(B, L, Dh, D, dI, m, W, X.data(), wkv.data(), wik.data(), wg.data(), bs.data(), 0, Nc, kv.data(),
                     ik.data(), win.data());
        check(std::isfinite(kv[0]) && std::isfinite(ik.back()) && std::isfinite(win.back()), "compress finite", 0);
        check(ora_n_visible(L - 1, L, m) == Nc && ora_n_visible(2, L, m) == 0, "n_visible", 0);

        const int Tq = 2, HI = 4, topk = 5;
        auto qi = bf16_vec((size_t)B * Tq * HI * dI, 0.25), ki = bf16_vec((size_t)B * Nc * dI, 0.25);
        std::vector<float> wi((size_t)B * Tq * HI, 0.5f), S((size_t)B * Tq * Nc);
        std::vector<int> nv((size_t)B * Tq), idx((size_t)B * Tq * topk), cnt((size_t)B * Tq);
        ora_index_scores(B, Tq, HI, dI, Nc, L, m, L - Tq, 0, qi.data(), wi.data(), ki.data(), S.data(), nv.data());
        ora_topk(B * Tq, Nc, topk, S.data(), nv.data(), idx.data(), cnt.data());
        check(cnt[0] == topk, "topk count", 0);

        const int H = 4, Lr = W + Tq;
        auto q = bf16_vec((size_t)B * Tq * H * D, 0.2), kvb = bf16_vec((size_t)B * Nc * D, 0.2);
        auto raw = bf16_vec((size_t)B * Lr * D, 0.2);
        std::vector<double> out((size_t)B * Tq * H * D), lse((size_t)B * Tq * H), sink(H, 0.3);
        const long long pos0 = L - Tq;
        check(ora_sparse_attn(B, Tq, H, D, Nc, topk, Lr, pos0 + Tq - Lr, pos0, W, 0.17, q.data(), kvb.data(),
                              idx.data(), raw.data(), nullptr, nullptr, sink.data(), out.data(), lse.data()) == 0,
              "sparse_attn", 0);
        ora_dense_attn(B, Tq, H, D, Nc, L, m, pos0, 0.17, q.data(), kvb.data(), nullptr, nullptr, out.data(), lse.data());
        check(std::isfinite(out[0]) && std::isfinite(lse.back()), "dense_attn finite", 0);

        std::vector<long long> pos = {0, 5, 1 << 20, 77};
        std::vector<double> y((size_t)4 * 3 * D);
        auto xr = bf16_vec((size_t)4 * 3 * D, 1.0);
        ora_rope(4 * 3, D, 16, 3, 10000.0, 0, xr.data(), pos.data(), y.data());
        check(std::isfinite(y.back()), "rope", 0);

        const int n8 = 9, D8 = 128;
        auto x8 = bf16_vec((size_t)n8 * D8, 0.5);
        std::vector<uint8_t> y8((size_t)n8 * (D8 + 80));
        std::vector<double> d8((size_t)n8 * D8);
        ora_kv_fp8_encode(n8, D8, x8.data(), y8.data());
        ora_kv_fp8_decode(n8, D8, y8.data(), d8.data());
        for (int i = D8 - 64; i < D8; ++i) check(d8[i] == ora_bf16_value(x8[i]), "fp8 rows keep the RoPE dims", i);

        const int nm = 5, len = 64;
        auto xm = bf16_vec((size_t)nm * len, 1.0);
        std::vector<uint8_t> codes((size_t)nm * len / 2), scales((size_t)nm * len / 32);
        ora_mxfp4_encode(nm, len, xm.data(), codes.data(), scales.data());
        check(std::isfinite(ora_exact_dot_mxfp4(codes.data(), scales.data(), codes.data() + len / 2,
                                                scales.data() + len / 32, len)), "mxfp4 dot", 0);
    }
    if (g_fail) std::fprintf(stderr, "%d mismatches\n", g_fail);
    else std::printf("sanitized host build: clean and equal\n");
    return g_fail ? 1 : 0;
}

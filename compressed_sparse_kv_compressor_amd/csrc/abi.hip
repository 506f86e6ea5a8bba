// abi.hip -- the C ABI of libcsa (include/csa.h): argument validation, workspace
// sizing and launch sequencing.  Nothing here computes; every step of the method
// runs in the kernels of index_topk.hip, attn.hip and compress.hip.
#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/csa.h"
#include "common.h"
#include "kernels.h"

namespace csa_host {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

// ---------------------------------------------------------------------------
// timing registry
// ---------------------------------------------------------------------------
struct ProfRec {
    std::string name;
    hipEvent_t a, b;
};
static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::string g_prof_only;          // non-empty: record only launches of this kernel
static std::vector<ProfRec> g_prof;
static std::vector<hipEvent_t> g_ev_pool;

static hipEvent_t take_event() {
    if (!g_ev_pool.empty()) {
        hipEvent_t e = g_ev_pool.back();
        g_ev_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void* prof_begin(const char* name, hipStream_t s) {
    if (!g_prof_on) return nullptr;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_only.empty() && g_prof_only != name) return nullptr;
    ProfRec r;
    r.name = name;
    r.a = take_event();
    r.b = take_event();
    if (!r.a || !r.b) return nullptr;
    (void)hipEventRecord(r.a, s);
    g_prof.push_back(r);
    return (void*)(uintptr_t)g_prof.size();
}

void prof_end(void* token, hipStream_t s) {
    if (!token) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    size_t i = (size_t)(uintptr_t)token - 1;
    if (i < g_prof.size()) (void)hipEventRecord(g_prof[i].b, s);
}

}  // namespace csa_host

using csa_host::fail;

// ---------------------------------------------------------------------------
// scratch of the no-allocation entry point (csa_sparse_attn_noalloc)
// ---------------------------------------------------------------------------
// One file-scope device array per GPU, loaded with the library's code object and held until the process
// ends.  Host code never passes `scratch` itself to a kernel (in host code the name is a host-side stand-in,
// not a device address): the device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept below.
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace csa_host {
constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[MAX_DEVICES];

// The current device's copy of `scratch` (looked up on the first call on each device).
static int scratch_ptr(const char* fn, void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CSA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(CSA_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r != hipSuccess || !p)
            return fail(CSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                        hipGetErrorString(r));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CSA_OK;
}
}  // namespace csa_host

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------
namespace {

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

#define REQ_PTR(p)                                                                     \
    do {                                                                               \
        if (!(p)) return fail(CSA_ERR_NULL, "%s: %s is NULL", fn, #p);                 \
        if (misaligned(p)) return fail(CSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)
#define OPT_PTR(p)                                                                     \
    do {                                                                               \
        if ((p) && misaligned(p)) return fail(CSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)
#define REQ(cond, code, ...)                                                           \
    do {                                                                               \
        if (!(cond)) return fail(code, __VA_ARGS__);                                   \
    } while (0)

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

int check_ws(const char* fn, void* ws, size_t have, size_t need) {
    if (have < need) return fail(CSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, have, need);
    if (need && !ws) return fail(CSA_ERR_NULL, "%s: ws is NULL but %zu bytes are required", fn, need);
    if (ws && misaligned(ws)) return fail(CSA_ERR_ALIGN, "%s: ws is not 16-byte aligned", fn);
    return CSA_OK;
}

int validate_index(const char* fn, const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B,
                   int Tq, int HI, int dI, int Nc, long long L, int m, long long pos0, int topk,
                   const int32_t* idx_out, const int32_t* cnt_out) {
    REQ_PTR(q_idx);
    REQ_PTR(w_idx);
    REQ_PTR(k_idx);
    REQ_PTR(idx_out);
    OPT_PTR(cnt_out);
    REQ(dtype == CSA_BF16 || dtype == CSA_E4M3 || dtype == CSA_MXFP4, CSA_ERR_DTYPE, "%s: dtype %d unknown", fn,
        dtype);
    REQ(B >= 1 && Tq >= 1 && L >= 1 && m >= 1 && pos0 >= 0, CSA_ERR_SHAPE,
        "%s: need B, Tq, L, m >= 1 and pos0 >= 0 (B=%d Tq=%d L=%lld m=%d pos0=%lld)", fn, B, Tq, L, m, pos0);
    REQ((long long)Nc == (L + m - 1) / m, CSA_ERR_SHAPE, "%s: Nc=%d but ceil(L/m)=%lld", fn, Nc, (L + m - 1) / m);
    REQ(pos0 + Tq - 1 <= L - 1, CSA_ERR_SHAPE, "%s: query positions pos0..pos0+Tq-1 exceed L-1", fn);
    REQ(topk >= 1, CSA_ERR_SHAPE, "%s: topk=%d must be >= 1", fn, topk);
    REQ(topk <= 4096 && Tq <= 65536 && Nc <= (1 << 24), CSA_ERR_UNSUPPORTED,
        "%s: topk <= 4096, Tq <= 65536, Nc <= 2^24 supported", fn);
    REQ(pow2_in(HI, 1, 16), CSA_ERR_UNSUPPORTED, "%s: HI=%d (supported 1,2,4,8,16)", fn, HI);
    REQ(dI == 64 || dI == 128, CSA_ERR_UNSUPPORTED, "%s: dI=%d (supported 64, 128)", fn, dI);
    return CSA_OK;
}

// Checks an optional batch / cache layout for caches of ratios r1 (N1 entries per sequence) and, if r2 > 0,
// r2 (N2 entries), and converts it to the launchers' form.
int read_layout(const char* fn, const csa_cache_layout_t* lay, int r1, int N1, int r2, int N2,
                csa_host::CacheLayout* out) {
    *out = csa_host::CacheLayout{nullptr, nullptr, 0, 0, 0};
    if (!lay) return CSA_OK;
    if (lay->seq_lens)
        REQ(((uintptr_t)lay->seq_lens & 7u) == 0, CSA_ERR_ALIGN, "%s: seq_lens is not 8-byte aligned", fn);
    if (lay->block_table) {
        REQ(((uintptr_t)lay->block_table & 3u) == 0, CSA_ERR_ALIGN, "%s: block_table is not 4-byte aligned", fn);
        REQ(lay->max_blocks >= 1 && lay->num_blocks >= 1 && lay->block_tokens >= 1, CSA_ERR_SHAPE,
            "%s: max_blocks, num_blocks and block_tokens must be >= 1", fn);
        const int rs[2] = {r1, r2}, ns[2] = {N1, N2};
        for (int i = 0; i < 2; ++i) {
            if (rs[i] <= 0) continue;
            const int epb = lay->block_tokens / rs[i];
            REQ(lay->block_tokens % rs[i] == 0 && epb >= 1 && (epb & (epb - 1)) == 0, CSA_ERR_UNSUPPORTED,
                "%s: block_tokens=%d must be a multiple of the ratio %d with a power-of-two quotient", fn,
                lay->block_tokens, rs[i]);
            REQ((long long)lay->max_blocks * epb >= ns[i], CSA_ERR_SHAPE,
                "%s: %d table columns of %d entries cover fewer than the %d entries of the cache", fn,
                lay->max_blocks, epb, ns[i]);
            REQ((long long)lay->num_blocks * epb < (1LL << 31), CSA_ERR_UNSUPPORTED, "%s: pool too large", fn);
        }
    }
    *out = csa_host::CacheLayout{lay->seq_lens, lay->block_table, lay->max_blocks, lay->num_blocks,
                                 lay->block_tokens};
    return CSA_OK;
}

int validate_attn_common(const char* fn, const void* q, int B, int Tq, int H, int D, float scale, const void* out,
                         const float* lse) {
    REQ_PTR(q);
    REQ_PTR(out);
    OPT_PTR(lse);
    REQ(B >= 1 && Tq >= 1 && H >= 1, CSA_ERR_SHAPE, "%s: need B, Tq, H >= 1", fn);
    REQ(D == 128 || D == 512, CSA_ERR_UNSUPPORTED, "%s: D=%d (supported 128, 512)", fn, D);
    REQ(H % 16 == 0 && H <= 256, CSA_ERR_UNSUPPORTED, "%s: H=%d (supported multiples of 16 up to 256)", fn, H);
    REQ(scale == scale && scale > -1e30f && scale < 1e30f, CSA_ERR_SHAPE, "%s: scale must be finite", fn);
    return CSA_OK;
}

int validate_sparse(const char* fn, const void* q, const void* kv, const int32_t* idx, const void* kv_raw, int B,
                    int Tq, int H, int D, int Nc, int topk, int Lr, long long raw0, long long pos0, int W,
                    float scale, const void* out, const float* lse, bool varlen = false) {
    int rc = validate_attn_common(fn, q, B, Tq, H, D, scale, out, lse);
    if (rc) return rc;
    REQ(topk >= 0 && W >= 0 && pos0 >= 0 && Nc >= 0, CSA_ERR_SHAPE, "%s: topk, W, pos0, Nc must be >= 0", fn);
    REQ(topk <= 4096 && W <= 1024, CSA_ERR_UNSUPPORTED, "%s: topk <= 4096 and W <= 1024 supported", fn);
    REQ(topk + W >= 0, CSA_ERR_SHAPE, "%s: bad sizes", fn);
    if (topk > 0) {
        REQ_PTR(kv);
        REQ_PTR(idx);
        REQ(Nc >= 1, CSA_ERR_SHAPE, "%s: Nc must be >= 1 when topk > 0", fn);
    }
    if (W > 0 && varlen) {           // every sequence's raw rows are its last Lr tokens
        REQ_PTR(kv_raw);
        REQ((long long)Lr >= (long long)Tq + W - 1, CSA_ERR_SHAPE,
            "%s: Lr=%d raw rows per sequence cannot hold the windows of %d queries (W=%d)", fn, Lr, Tq, W);
    } else if (W > 0) {
        REQ_PTR(kv_raw);
        REQ(Lr >= 1, CSA_ERR_SHAPE, "%s: Lr must be >= 1 when W > 0", fn);
        const long long first = pos0 - W + 1 < 0 ? 0 : pos0 - W + 1;
        REQ(raw0 <= first, CSA_ERR_SHAPE, "%s: raw rows start at %lld, window needs %lld", fn, raw0, first);
        REQ(pos0 + Tq - 1 < raw0 + Lr, CSA_ERR_SHAPE, "%s: raw rows end at %lld, window needs %lld", fn,
            raw0 + Lr - 1, pos0 + Tq - 1);
    }
    return CSA_OK;
}

int validate_dense(const char* fn, const void* q, const void* kv_h, int B, int Tq, int H, int D, int Nh, long long L,
                   int mh, long long pos0, float scale, const void* out, const float* lse) {
    int rc = validate_attn_common(fn, q, B, Tq, H, D, scale, out, lse);
    if (rc) return rc;
    REQ_PTR(kv_h);
    REQ(L >= 1 && mh >= 1 && pos0 >= 0, CSA_ERR_SHAPE, "%s: need L, mh >= 1 and pos0 >= 0", fn);
    REQ((long long)Nh == (L + mh - 1) / mh, CSA_ERR_SHAPE, "%s: Nh=%d but ceil(L/mh)=%lld", fn, Nh, (L + mh - 1) / mh);
    REQ(pos0 + Tq - 1 <= L - 1, CSA_ERR_SHAPE, "%s: query positions exceed L-1", fn);
    return CSA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// exported entry points
// ---------------------------------------------------------------------------
extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_str(int s) {
    switch (s) {
        case CSA_OK: return "CSA_OK";
        case CSA_ERR_NULL: return "CSA_ERR_NULL";
        case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE";
        case CSA_ERR_DTYPE: return "CSA_ERR_DTYPE";
        case CSA_ERR_ALIGN: return "CSA_ERR_ALIGN";
        case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
        case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
        case CSA_ERR_HIP: return "CSA_ERR_HIP";
        default: return "CSA_ERR_UNKNOWN";
    }
}

const char* csa_last_error(void) { return csa_host::g_err; }

size_t csa_compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W) {
    if (B < 1 || L < 1 || Dh < 1 || D < 1 || dI < 0 || m < 1 || W < 0) return 0;
    return csa_host::compress_ws_bytes(B, L, Dh, D, dI, m, W);
}

int csa_compress(const void* hidden, const void* w_kv, const void* w_ik, const float* w_gate, const float* b_slot,
                 int B, long long L, int Dh, int D, int dI, int m, int W, int ik_dtype, void* kv_out, void* ik_out,
                 void* win_out, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa_compress";
    csa_host::g_err[0] = 0;
    REQ_PTR(hidden);
    REQ_PTR(w_kv);
    REQ_PTR(w_gate);
    REQ_PTR(kv_out);
    OPT_PTR(w_ik);
    OPT_PTR(b_slot);
    OPT_PTR(ik_out);
    OPT_PTR(win_out);
    REQ(B >= 1 && L >= 1 && m >= 1 && W >= 0, CSA_ERR_SHAPE, "%s: need B, L, m >= 1 and W >= 0", fn);
    REQ(ik_dtype == CSA_BF16 || ik_dtype == CSA_E4M3, CSA_ERR_DTYPE, "%s: ik_dtype %d unknown", fn, ik_dtype);
    REQ(Dh % 64 == 0 && Dh >= 64 && Dh <= 16384, CSA_ERR_UNSUPPORTED, "%s: Dh=%d (multiple of 64 in [64,16384])", fn, Dh);
    REQ(D == 64 || D == 128 || D == 256 || D == 512, CSA_ERR_UNSUPPORTED, "%s: D=%d unsupported", fn, D);
    REQ(m <= 1024 && W <= 1024, CSA_ERR_UNSUPPORTED, "%s: m <= 1024 and W <= 1024 supported", fn);
    REQ((L + m - 1) / m <= (1LL << 24) && (long long)B * L * Dh < (1LL << 40), CSA_ERR_UNSUPPORTED, "%s: sizes too large", fn);
    if (w_ik || ik_out) {
        REQ(w_ik && ik_out, CSA_ERR_NULL, "%s: w_ik and ik_out must both be given or both be NULL", fn);
        REQ(dI == 64 || dI == 128 || dI == 256 || dI == 512, CSA_ERR_UNSUPPORTED, "%s: dI=%d unsupported", fn, dI);
    }
    if (W > 0) REQ(win_out != nullptr, CSA_ERR_NULL, "%s: win_out is NULL but W > 0", fn);
    int rc = check_ws(fn, ws, ws_bytes, csa_host::compress_ws_bytes(B, L, Dh, D, (w_ik && ik_out) ? dI : 0, m,
                                                                 win_out ? W : 0));
    if (rc) return rc;
    return csa_host::compress_launch(hidden, w_kv, w_ik, w_gate, b_slot, B, L, Dh, D, dI, m, W, ik_dtype, kv_out,
                                     ik_out, W > 0 ? win_out : nullptr, ws, (hipStream_t)stream);
}

size_t csa_hca_compress_ws_bytes(int B, long long L, int Dh, int D, int dI, int m, int W, int mh) {
    if (B < 1 || L < 1 || Dh < 1 || D < 1 || dI < 0 || m < 1 || W < 0 || mh < 1) return 0;
    return csa_host::hca_compress_ws_bytes(B, L, Dh, D, dI, m, W, mh);
}

int csa_hca_compress(const void* hidden, int B, long long L, int Dh, const void* w_kv, const void* w_ik,
                     const float* w_gate, const float* b_slot, int D, int dI, int m, int W, int ik_dtype, void* kv_out,
                     void* ik_out, void* win_out, const void* w_kv_h, const float* w_gate_h, const float* b_slot_h,
                     int mh, void* kv_h_out, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa_hca_compress";
    csa_host::g_err[0] = 0;
    REQ_PTR(hidden);
    REQ_PTR(w_kv);
    REQ_PTR(w_gate);
    REQ_PTR(kv_out);
    REQ_PTR(w_kv_h);
    REQ_PTR(w_gate_h);
    REQ_PTR(kv_h_out);
    OPT_PTR(w_ik);
    OPT_PTR(b_slot);
    OPT_PTR(ik_out);
    OPT_PTR(win_out);
    OPT_PTR(b_slot_h);
    REQ(B >= 1 && L >= 1 && m >= 1 && mh >= 1 && W >= 0, CSA_ERR_SHAPE, "%s: need B, L, m, mh >= 1 and W >= 0", fn);
    REQ(ik_dtype == CSA_BF16 || ik_dtype == CSA_E4M3, CSA_ERR_DTYPE, "%s: ik_dtype %d unknown", fn, ik_dtype);
    REQ(Dh % 64 == 0 && Dh >= 64 && Dh <= 16384, CSA_ERR_UNSUPPORTED, "%s: Dh=%d (multiple of 64 in [64,16384])", fn, Dh);
    REQ(D == 64 || D == 128 || D == 256 || D == 512, CSA_ERR_UNSUPPORTED, "%s: D=%d unsupported", fn, D);
    REQ(m <= 1024 && mh <= 1024 && W <= 1024, CSA_ERR_UNSUPPORTED, "%s: m, mh <= 1024 and W <= 1024 supported", fn);
    REQ((L + m - 1) / m <= (1LL << 24) && (long long)B * L * Dh < (1LL << 40), CSA_ERR_UNSUPPORTED, "%s: sizes too large", fn);
    if (w_ik || ik_out) {
        REQ(w_ik && ik_out, CSA_ERR_NULL, "%s: w_ik and ik_out must both be given or both be NULL", fn);
        REQ(dI == 64 || dI == 128 || dI == 256 || dI == 512, CSA_ERR_UNSUPPORTED, "%s: dI=%d unsupported", fn, dI);
    }
    if (W > 0) REQ(win_out != nullptr, CSA_ERR_NULL, "%s: win_out is NULL but W > 0", fn);
    int rc = check_ws(fn, ws, ws_bytes, csa_host::hca_compress_ws_bytes(B, L, Dh, D, (w_ik && ik_out) ? dI : 0, m,
                                                                     win_out ? W : 0, mh));
    if (rc) return rc;
    return csa_host::hca_compress_launch(hidden, w_kv, w_ik, w_gate, b_slot, B, L, Dh, D, dI, m, W, ik_dtype, kv_out,
                                         ik_out, W > 0 ? win_out : nullptr, w_kv_h, w_gate_h, b_slot_h, mh, kv_h_out,
                                         ws, (hipStream_t)stream);
}

static bool plain_layout(const csa_cache_layout_t* lay) { return !lay || (!lay->seq_lens && !lay->block_table); }

size_t csa_append_state_bytes(int D, int dI) {
    if (D < 1 || dI < 0) return 0;
    return csa_host::append_state_words(D, dI) * 4;
}

size_t csa_decode_append_ws_bytes(int B, int T, int D, int dI) {
    if (B < 1 || T < 1 || D < 1 || dI < 0) return 0;
    return csa_host::append_ws_bytes(B, T, D, dI);
}

int csa_decode_append(const void* hidden, int B, int T, int Dh, const void* w_kv, const void* w_ik, const float* w_gate,
                      const float* b_slot, int D, int dI, int m, int ik_dtype, const void* w_kv_h,
                      const float* w_gate_h, const float* b_slot_h, int mh, long long L, long long* seq_lens,
                      void* state, void* kv_out, void* ik_out, void* kv_h_out, void* win, int W,
                      const csa_cache_layout_t* layout, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa_decode_append";
    csa_host::g_err[0] = 0;
    REQ_PTR(hidden);
    REQ_PTR(w_kv);
    REQ_PTR(w_gate);
    REQ_PTR(w_kv_h);
    REQ_PTR(w_gate_h);
    REQ_PTR(state);
    REQ_PTR(kv_out);
    REQ_PTR(kv_h_out);
    OPT_PTR(b_slot);
    OPT_PTR(b_slot_h);
    REQ(seq_lens != nullptr, CSA_ERR_NULL, "%s: seq_lens is NULL", fn);
    REQ(((uintptr_t)seq_lens & 7u) == 0, CSA_ERR_ALIGN, "%s: seq_lens is not 8-byte aligned", fn);
    REQ(B >= 1 && T >= 1 && L >= 1 && m >= 1 && mh >= 1 && W >= 0 && dI >= 0, CSA_ERR_SHAPE,
        "%s: need B, T, L, m, mh >= 1 and W, dI >= 0", fn);
    REQ(ik_dtype == CSA_BF16 || ik_dtype == CSA_E4M3, CSA_ERR_DTYPE, "%s: ik_dtype %d unknown", fn, ik_dtype);
    REQ(Dh % 64 == 0 && Dh >= 64 && Dh <= 16384, CSA_ERR_UNSUPPORTED, "%s: Dh=%d (multiple of 64 in [64,16384])", fn, Dh);
    REQ(D == 64 || D == 128 || D == 256 || D == 512, CSA_ERR_UNSUPPORTED, "%s: D=%d unsupported", fn, D);
    REQ(dI == 0 || dI == 64 || dI == 128 || dI == 256 || dI == 512, CSA_ERR_UNSUPPORTED, "%s: dI=%d unsupported", fn, dI);
    REQ(2 * D + dI <= 2048 && m <= 1024 && mh <= 1024 && W <= 1024, CSA_ERR_UNSUPPORTED,
        "%s: 2 D + dI <= 2048, m, mh, W <= 1024 supported", fn);
    REQ((long long)B * T <= (1LL << 24) && (L + m - 1) / m <= (1LL << 24), CSA_ERR_UNSUPPORTED, "%s: sizes too large", fn);
    if (dI) {
        REQ_PTR(w_ik);
        REQ_PTR(ik_out);
    }
    if (W > 0) REQ_PTR(win);
    const int Nc = (int)((L + m - 1) / m), Nh = (int)((L + mh - 1) / mh);
    csa_host::CacheLayout lay;
    int rc = read_layout(fn, layout, m, Nc, mh, Nh, &lay);
    if (rc) return rc;
    lay.seq_lens = nullptr;
    rc = check_ws(fn, ws, ws_bytes, csa_host::append_ws_bytes(B, T, D, dI));
    if (rc) return rc;
    return csa_host::append_launch(hidden, B, T, Dh, w_kv, dI ? w_ik : nullptr, w_gate, b_slot, D, dI, m, ik_dtype,
                                   w_kv_h, w_gate_h, b_slot_h, mh, L, seq_lens, state, kv_out, dI ? ik_out : nullptr,
                                   kv_h_out, W > 0 ? win : nullptr, W, lay, ws, (hipStream_t)stream);
}

size_t csa_index_topk_ws_bytes(int B, int Tq, int HI, int dI, int Nc, int topk, int dtype) {
    if (B < 1 || Tq < 1 || Nc < 1 || HI < 1 || dI < 1 || topk < 1) return 0;
    return csa_host::index_topk_ws_bytes(dtype, HI, dI, B, Tq, Nc, topk);
}

size_t csa_index_topk_ex_ws_bytes(int B, int Tq, int HI, int dI, int Nc, int topk, int dtype,
                                  const csa_cache_layout_t* layout) {
    if (B < 1 || Tq < 1 || Nc < 1 || HI < 1 || dI < 1 || topk < 1) return 0;
    return csa_host::index_topk_ws_bytes(dtype, HI, dI, B, Tq, Nc, topk, plain_layout(layout));
}

static int index_topk_impl(const char* fn, const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B,
                           int Tq, int HI, int dI, int Nc, long long L, int m, long long pos0, int topk,
                           int32_t* idx_out, int32_t* cnt_out, float* score_out, const csa_cache_layout_t* layout,
                           const uint8_t* q_scale, const uint8_t* k_scale, void* ws, size_t ws_bytes, void* stream) {
    csa_host::g_err[0] = 0;
    int rc = validate_index(fn, q_idx, w_idx, k_idx, dtype, B, Tq, HI, dI, Nc, L, m, pos0, topk, idx_out, cnt_out);
    if (rc) return rc;
    if (dtype == CSA_MXFP4) {
        REQ(q_scale && k_scale, CSA_ERR_NULL, "%s: MXFP4 operands need q_scale and k_scale", fn);
        REQ(dI == 128, CSA_ERR_UNSUPPORTED, "%s: MXFP4 indexer rows of dI = 128 supported (got %d)", fn, dI);
    }
    OPT_PTR(score_out);
    csa_host::CacheLayout lay;
    rc = read_layout(fn, layout, m, Nc, 0, 0, &lay);
    if (rc) return rc;
    rc = check_ws(fn, ws, ws_bytes, csa_host::index_topk_ws_bytes(dtype, HI, dI, B, Tq, Nc, topk, plain_layout(layout)));
    if (rc) return rc;
    return csa_host::index_topk_launch(q_idx, w_idx, k_idx, dtype, B, Tq, HI, dI, Nc, L, m, pos0, topk, idx_out,
                                       cnt_out, score_out, lay, q_scale, k_scale, ws, (hipStream_t)stream);
}

int csa_index_topk(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B, int Tq, int HI, int dI,
                   int Nc, long long L, int m, long long pos0, int topk, int32_t* idx_out, int32_t* cnt_out,
                   float* score_out, void* ws, size_t ws_bytes, void* stream) {
    if (dtype == CSA_MXFP4)
        return fail(CSA_ERR_DTYPE, "csa_index_topk: MXFP4 operands carry scales: call csa_index_topk_ex");
    return index_topk_impl("csa_index_topk", q_idx, w_idx, k_idx, dtype, B, Tq, HI, dI, Nc, L, m, pos0, topk, idx_out,
                           cnt_out, score_out, nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

int csa_index_topk_ex(const void* q_idx, const float* w_idx, const void* k_idx, int dtype, int B, int Tq, int HI,
                      int dI, int Nc, long long L, int m, long long pos0, int topk, int32_t* idx_out, int32_t* cnt_out,
                      float* score_out, const csa_cache_layout_t* layout, const void* q_scale, const void* k_scale,
                      void* ws, size_t ws_bytes, void* stream) {
    return index_topk_impl("csa_index_topk_ex", q_idx, w_idx, k_idx, dtype, B, Tq, HI, dI, Nc, L, m, pos0, topk,
                           idx_out, cnt_out, score_out, layout, (const uint8_t*)q_scale, (const uint8_t*)k_scale, ws,
                           ws_bytes, stream);
}

size_t csa_sparse_attn_ws_bytes(int B, int Tq, int H, int D, int topk, int W) {
    if (B < 1 || Tq < 1 || H < 1 || topk < 0 || W < 0) return 0;
    return csa_host::attn_ws_bytes(B, Tq, H, D, 1, topk, W);
}

// The fused rotary embedding (csa_rope_t) of an attention call: NULL = none.
static int read_rope(const char* fn, const csa_rope_t* rope, int D, csa_host::AttnRows& r) {
    r.rope_rd = 0;
    r.rope_theta = 0.0;
    if (!rope) return CSA_OK;
    REQ(rope->rd == 64 && D >= 64, CSA_ERR_UNSUPPORTED, "%s: the fused rotary embedding covers rd = 64 (got %d)", fn,
        rope->rd);
    REQ(std::isfinite(rope->theta) && rope->theta > 1.0, CSA_ERR_SHAPE, "%s: rope theta must be finite and > 1", fn);
    r.rope_rd = rope->rd;
    r.rope_theta = rope->theta;
    return CSA_OK;
}

static int sparse_impl(const char* fn, const void* q, const void* kv, const void* v, const int32_t* idx,
                       const void* kv_raw, const void* v_raw, int B, int Tq, int H, int D, int Nc, int m, int topk,
                       int Lr, long long raw0, long long pos0, int W, float scale, const float* sink,
                       const csa_cache_layout_t* layout, int kv_format, const csa_rope_t* rope, void* out,
                       float* lse_out, void* ws, size_t ws_bytes, void* stream) {
    csa_host::g_err[0] = 0;
    const bool varlen = layout && layout->seq_lens;
    int rc = validate_sparse(fn, q, kv, idx, kv_raw, B, Tq, H, D, Nc, topk, Lr, raw0, pos0, W, scale, out, lse_out,
                             varlen);
    if (rc) return rc;
    OPT_PTR(v);
    OPT_PTR(v_raw);
    csa_host::CacheLayout lay;
    REQ(m >= 1, CSA_ERR_SHAPE, "%s: m must be >= 1", fn);
    rc = read_layout(fn, layout, m, Nc, 0, 0, &lay);
    if (rc) return rc;
    rc = check_ws(fn, ws, ws_bytes, csa_host::attn_ws_bytes(B, Tq, H, D, 1, topk, W));
    if (rc) return rc;
    csa_host::AttnRows r{1, kv, Nc, 0, 1, idx, topk, kv_raw, Lr, raw0, W, sink};
    r.seq_lens = lay.seq_lens;
    r.v = v;
    r.v_raw = W > 0 ? v_raw : nullptr;
    r.pm = csa_host::page_map(lay, m);
    REQ(kv_format == CSA_KV_BF16 || kv_format == CSA_KV_FP8, CSA_ERR_DTYPE, "%s: kv_format %d unknown", fn, kv_format);
    r.kv_fp8 = kv_format == CSA_KV_FP8;
    rc = read_rope(fn, rope, D, r);
    if (rc) return rc;
    return csa_host::attn_launch(q, r, B, Tq, H, D, pos0, scale, out, lse_out, ws, ws_bytes, (hipStream_t)stream,
                                 "k_attn_sparse");
}

int csa_sparse_attn(const void* q, const void* kv, const int32_t* idx, const void* kv_raw, int B, int Tq, int H, int D,
                    int Nc, int topk, int Lr, long long raw0, long long pos0, int W, float scale, const float* sink,
                    void* out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
    return sparse_impl("csa_sparse_attn", q, kv, nullptr, idx, kv_raw, nullptr, B, Tq, H, D, Nc, 1, topk, Lr, raw0, pos0,
                       W, scale, sink, nullptr, CSA_KV_BF16, nullptr, out, lse_out, ws, ws_bytes, stream);
}

int csa_sparse_attn_ex(const void* q, const void* kv, const void* v, const int32_t* idx, const void* kv_raw,
                       const void* v_raw, int B, int Tq, int H, int D, int Nc, int m, int topk, int Lr, long long raw0,
                       long long pos0, int W, float scale, const float* sink, const csa_cache_layout_t* layout,
                       int kv_format, const csa_rope_t* rope, void* out, float* lse_out, void* ws, size_t ws_bytes,
                       void* stream) {
    return sparse_impl("csa_sparse_attn_ex", q, kv, v, idx, kv_raw, v_raw, B, Tq, H, D, Nc, m, topk, Lr, raw0, pos0, W,
                       scale, sink, layout, kv_format, rope, out, lse_out, ws, ws_bytes, stream);
}

// As csa_sparse_attn, with the split partials in the library's static scratch instead of a workspace.
int csa_sparse_attn_noalloc(const void* q, const void* kv, const int32_t* idx, const void* kv_raw, int B, int Tq,
                            int H, int D, int Nc, int topk, int Lr, long long raw0, long long pos0, int W, float scale,
                            const float* sink, void* out, float* lse_out, void* stream) {
    const char* fn = "csa_sparse_attn_noalloc";
    csa_host::g_err[0] = 0;
    int rc = validate_sparse(fn, q, kv, idx, kv_raw, B, Tq, H, D, Nc, topk, Lr, raw0, pos0, W, scale, out, lse_out);
    if (rc) return rc;
    const size_t need = csa_host::attn_ws_bytes(B, Tq, H, D, 1, topk, W);
    REQ(need <= (size_t)CSA_NOALLOC_SCRATCH_BYTES, CSA_ERR_UNSUPPORTED,
        "%s: this call needs %zu bytes of scratch, beyond the static %llu (use csa_sparse_attn with a workspace)", fn,
        need, (unsigned long long)CSA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need) {
        rc = csa_host::scratch_ptr(fn, &ws);
        if (rc) return rc;
    }
    csa_host::AttnRows r{1, kv, Nc, 0, 1, idx, topk, kv_raw, Lr, raw0, W, sink};
    return csa_host::attn_launch(q, r, B, Tq, H, D, pos0, scale, out, lse_out, ws, need, (hipStream_t)stream,
                                 "k_attn_sparse");
}

size_t hca_dense_attn_ws_bytes(int B, int Tq, int H, int D, int Nh) {
    if (B < 1 || Tq < 1 || H < 1 || Nh < 0) return 0;
    return csa_host::attn_ws_bytes(B, Tq, H, D, 0, Nh, 0);
}

static int dense_impl(const char* fn, const void* q, const void* kv_h, const void* v_h, int B, int Tq, int H, int D,
                      int Nh, long long L, int mh, long long pos0, float scale, const float* sink,
                      const csa_cache_layout_t* layout, int kv_format, const csa_rope_t* rope, void* out,
                      float* lse_out, void* ws, size_t ws_bytes, void* stream) {
    csa_host::g_err[0] = 0;
    int rc = validate_dense(fn, q, kv_h, B, Tq, H, D, Nh, L, mh, pos0, scale, out, lse_out);
    if (rc) return rc;
    OPT_PTR(v_h);
    csa_host::CacheLayout lay;
    rc = read_layout(fn, layout, mh, Nh, 0, 0, &lay);
    if (rc) return rc;
    rc = check_ws(fn, ws, ws_bytes, csa_host::attn_ws_bytes(B, Tq, H, D, 0, Nh, 0));
    if (rc) return rc;
    csa_host::AttnRows r{0, kv_h, Nh, L, mh, nullptr, 0, nullptr, 0, 0, 0, sink};
    r.seq_lens = lay.seq_lens;
    r.v = v_h;
    r.pm = csa_host::page_map(lay, mh);
    REQ(kv_format == CSA_KV_BF16 || kv_format == CSA_KV_FP8, CSA_ERR_DTYPE, "%s: kv_format %d unknown", fn, kv_format);
    r.kv_fp8 = kv_format == CSA_KV_FP8;
    rc = read_rope(fn, rope, D, r);
    if (rc) return rc;
    return csa_host::attn_launch(q, r, B, Tq, H, D, pos0, scale, out, lse_out, ws, ws_bytes, (hipStream_t)stream,
                                 "k_attn_dense");
}

int hca_dense_attn(const void* q, const void* kv_h, int B, int Tq, int H, int D, int Nh, long long L, int mh,
                   long long pos0, float scale, const float* sink, void* out, float* lse_out, void* ws,
                   size_t ws_bytes, void* stream) {
    return dense_impl("hca_dense_attn", q, kv_h, nullptr, B, Tq, H, D, Nh, L, mh, pos0, scale, sink, nullptr,
                      CSA_KV_BF16, nullptr, out, lse_out, ws, ws_bytes, stream);
}

int hca_dense_attn_ex(const void* q, const void* kv_h, const void* v_h, int B, int Tq, int H, int D, int Nh,
                      long long L, int mh, long long pos0, float scale, const float* sink,
                      const csa_cache_layout_t* layout, int kv_format, const csa_rope_t* rope, void* out,
                      float* lse_out, void* ws, size_t ws_bytes, void* stream) {
    return dense_impl("hca_dense_attn_ex", q, kv_h, v_h, B, Tq, H, D, Nh, L, mh, pos0, scale, sink, layout, kv_format,
                      rope, out, lse_out, ws, ws_bytes, stream);
}

// Fused decode: workspace = [idx (if not caller-owned)] [index_topk ws] [attention ws (max of both layers)]
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t csa_hca_decode_ws_bytes(const csa_hca_decode_args_t* a) {
    if (!a || a->B < 1 || a->L < 1 || a->m < 1 || a->mh < 1 || a->topk < 1) return 0;
    const int Nc = (int)((a->L + a->m - 1) / a->m), Nh = (int)((a->L + a->mh - 1) / a->mh);
    size_t s = a->idx_out ? 0 : align256((size_t)a->B * a->topk * 4);
    s += align256(csa_host::index_topk_ws_bytes(a->idx_dtype, a->HI, a->dI, a->B, 1, Nc, a->topk,
                                                plain_layout(a->layout) && a->idx_dtype != CSA_MXFP4));
    s += align256(csa_host::attn_ws_bytes(a->B, 1, a->H, a->D, 1, a->topk, a->W));
    s += csa_host::attn_ws_bytes(a->B, 1, a->H, a->D, 0, Nh, 0);
    return s;
}

int csa_hca_decode(const csa_hca_decode_args_t* a, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa_hca_decode";
    csa_host::g_err[0] = 0;
    if (!a) return fail(CSA_ERR_NULL, "%s: args is NULL", fn);
    REQ(a->B >= 1 && a->L >= 1 && a->m >= 1 && a->mh >= 1, CSA_ERR_SHAPE, "%s: need B, L, m, mh >= 1", fn);
    const int Nc = (int)((a->L + a->m - 1) / a->m), Nh = (int)((a->L + a->mh - 1) / a->mh);
    const long long p = a->L - 1;
    int rc = validate_index(fn, a->q_idx, a->w_idx, a->k_idx, a->idx_dtype, a->B, 1, a->HI, a->dI, Nc, a->L, a->m, p,
                            a->topk, a->idx_out ? a->idx_out : (const int32_t*)16, nullptr);
    if (rc) return rc;
    if (a->idx_dtype == CSA_MXFP4) {
        REQ(a->q_idx_scale && a->k_idx_scale, CSA_ERR_NULL, "%s: MXFP4 indexer operands need their scales", fn);
        REQ(a->dI == 128, CSA_ERR_UNSUPPORTED, "%s: MXFP4 indexer rows of dI = 128 supported", fn);
    }
    rc = validate_sparse(fn, a->csa_q, a->kv, (const int32_t*)16, a->kv_raw, a->B, 1, a->H, a->D, Nc, a->topk, a->W,
                         a->L - a->W, p, a->W, a->scale, a->csa_out, a->csa_lse);
    if (rc) return rc;
    csa_host::CacheLayout lay;
    rc = read_layout(fn, a->layout, a->m, Nc, a->mh, Nh, &lay);
    if (rc) return rc;
    rc = validate_dense(fn, a->hca_q, a->kv_h, a->B, 1, a->H, a->D, Nh, a->L, a->mh, p, a->scale, a->hca_out,
                        a->hca_lse);
    if (rc) return rc;
    // every argument is checked before the first launch: an error leaves the outputs untouched
    csa_host::AttnRows rs{1, a->kv, Nc, 0, 1, nullptr, a->topk, a->kv_raw, a->W, a->L - a->W, a->W, a->csa_sink};
    csa_host::AttnRows rd{0, a->kv_h, Nh, a->L, a->mh, nullptr, 0, nullptr, 0, 0, 0, a->hca_sink};
    rs.seq_lens = rd.seq_lens = lay.seq_lens;
    rs.pm = csa_host::page_map(lay, a->m);
    rd.pm = csa_host::page_map(lay, a->mh);
    rc = read_rope(fn, a->csa_rope, a->D, rs);
    if (rc) return rc;
    rc = read_rope(fn, a->hca_rope, a->D, rd);
    if (rc) return rc;
    REQ(a->kv_format == CSA_KV_BF16 || a->kv_format == CSA_KV_FP8, CSA_ERR_DTYPE, "%s: kv_format %d unknown", fn,
        a->kv_format);
    REQ(a->ws_persistent == 0 || a->ws_persistent == 1, CSA_ERR_SHAPE, "%s: ws_persistent must be 0 or 1 (got %d)",
        fn, a->ws_persistent);
    rs.kv_fp8 = rd.kv_fp8 = a->kv_format == CSA_KV_FP8;
    rc = check_ws(fn, ws, ws_bytes, csa_hca_decode_ws_bytes(a));
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    char* w = (char*)ws;
    int32_t* idx = a->idx_out;
    if (!idx) {
        idx = (int32_t*)w;
        w += align256((size_t)a->B * a->topk * 4);
    }
    rs.idx = idx;
    const size_t iws = align256(csa_host::index_topk_ws_bytes(a->idx_dtype, a->HI, a->dI, a->B, 1, Nc, a->topk,
                                                              plain_layout(a->layout) && a->idx_dtype != CSA_MXFP4));
    rc = csa_host::index_topk_launch(a->q_idx, a->w_idx, a->k_idx, a->idx_dtype, a->B, 1, a->HI, a->dI, Nc, a->L, a->m,
                                     p, a->topk, idx, nullptr, nullptr, lay, (const uint8_t*)a->q_idx_scale,
                                     (const uint8_t*)a->k_idx_scale, w, st, a->ws_persistent != 0);
    if (rc) return rc;
    w += iws;
    const size_t aws = ws_bytes - (size_t)(w - (char*)ws);
    // the CSA layer's attention, then the HCA layer's (layer order: a real next layer's query depends on the
    // previous layer's output, so the two are never overlapped)
    const size_t sws = align256(csa_host::attn_ws_bytes(a->B, 1, a->H, a->D, 1, a->topk, a->W));
    rc = csa_host::attn_launch(a->csa_q, rs, a->B, 1, a->H, a->D, p, a->scale, a->csa_out, a->csa_lse, w, sws, st,
                               "k_attn_sparse");
    if (rc) return rc;
    return csa_host::attn_launch(a->hca_q, rd, a->B, 1, a->H, a->D, p, a->scale, a->hca_out, a->hca_lse, w + sws,
                                 aws - sws, st, "k_attn_dense");
}

// Partial rotary position embedding of bf16 rows (see include/csa.h).
int csa_rope(const void* x, void* y, const long long* pos, long long n, int D, int rd, int group, double theta,
             int inverse, void* stream) {
    const char* fn = "csa_rope";
    csa_host::g_err[0] = 0;
    REQ(n >= 0 && D >= 8 && D % 8 == 0, CSA_ERR_SHAPE, "%s: need n >= 0 and D a positive multiple of 8", fn);
    REQ(rd > 0 && rd % 8 == 0 && rd <= D, CSA_ERR_SHAPE, "%s: rd must be a multiple of 8 in (0, D]", fn);
    REQ(group >= 1 && n % group == 0, CSA_ERR_SHAPE, "%s: group must be >= 1 and divide n", fn);
    REQ(std::isfinite(theta) && theta > 1.0, CSA_ERR_SHAPE, "%s: theta must be finite and > 1", fn);
    REQ(inverse == 0 || inverse == 1, CSA_ERR_SHAPE, "%s: inverse must be 0 or 1", fn);
    if (n == 0) return CSA_OK;
    REQ_PTR(x);
    REQ_PTR(y);
    REQ(pos != nullptr, CSA_ERR_NULL, "%s: pos is NULL", fn);
    REQ(((uintptr_t)pos & 7u) == 0, CSA_ERR_ALIGN, "%s: pos is not 8-byte aligned", fn);
    return csa_host::rope_launch(x, y, pos, n, D, rd, group, theta, inverse, (hipStream_t)stream);
}

// FP8 KV rows and MXFP4 indexer operands (see include/csa.h).
int csa_kv_fp8_encode(const void* x, long long n, int D, void* y, void* stream) {
    const char* fn = "csa_kv_fp8_encode";
    csa_host::g_err[0] = 0;
    REQ(n >= 0, CSA_ERR_SHAPE, "%s: n must be >= 0", fn);
    REQ(D == 128 || D == 512, CSA_ERR_UNSUPPORTED, "%s: D=%d (supported 128, 512)", fn, D);
    if (n == 0) return CSA_OK;
    REQ_PTR(x);
    REQ_PTR(y);
    return csa_host::kv_fp8_launch(x, n, D, y, (hipStream_t)stream);
}

int csa_mxfp4_encode(const void* x, long long n, int len, void* codes, void* scales, void* stream) {
    const char* fn = "csa_mxfp4_encode";
    csa_host::g_err[0] = 0;
    REQ(n >= 0 && len >= 32 && len % 32 == 0 && len <= 4096, CSA_ERR_SHAPE,
        "%s: need n >= 0 and len a multiple of 32 in [32, 4096]", fn);
    if (n == 0) return CSA_OK;
    REQ_PTR(x);
    REQ_PTR(codes);
    REQ(scales != nullptr, CSA_ERR_NULL, "%s: scales is NULL", fn);
    return csa_host::mxfp4_launch(x, n, len, codes, scales, (hipStream_t)stream);
}

// Diagnostic: fp8 (OCP e4m3) -> bf16 conversion exactly as the indexer kernel does it.
int csa_debug_fp8_to_bf16(const void* in, void* out, int n, void* stream) {
    const char* fn = "csa_debug_fp8_to_bf16";
    csa_host::g_err[0] = 0;
    REQ_PTR(in);
    REQ_PTR(out);
    REQ(n >= 0 && n % 4 == 0, CSA_ERR_SHAPE, "%s: n must be a non-negative multiple of 4", fn);
    if (n == 0) return CSA_OK;
    return csa_host::fp8_to_bf16_launch(in, out, n, (hipStream_t)stream);
}

int csa_prof_enable(int on) {
    std::lock_guard<std::mutex> lk(csa_host::g_prof_mu);
    csa_host::g_prof_on = on != 0;
    return CSA_OK;
}

int csa_prof_only(const char* kernel) {
    std::lock_guard<std::mutex> lk(csa_host::g_prof_mu);
    csa_host::g_prof_only = kernel ? kernel : "";
    return CSA_OK;
}

int csa_prof_reset(void) {
    std::lock_guard<std::mutex> lk(csa_host::g_prof_mu);
    for (auto& r : csa_host::g_prof) {
        (void)hipEventSynchronize(r.b);
        csa_host::g_ev_pool.push_back(r.a);
        csa_host::g_ev_pool.push_back(r.b);
    }
    csa_host::g_prof.clear();
    return CSA_OK;
}

int csa_prof_read(const char* kernel, double* total_ms, int* launches) {
    const char* fn = "csa_prof_read";
    if (!kernel || !total_ms || !launches) return fail(CSA_ERR_NULL, "%s: NULL argument", fn);
    std::lock_guard<std::mutex> lk(csa_host::g_prof_mu);
    double t = 0;
    int n = 0;
    for (auto& r : csa_host::g_prof) {
        if (r.name != kernel) continue;
        if (hipEventSynchronize(r.b) != hipSuccess) return fail(CSA_ERR_HIP, "%s: event sync failed", fn);
        float ms = 0;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(CSA_ERR_HIP, "%s: elapsed time failed", fn);
        t += ms;
        ++n;
    }
    *total_ms = t;
    *launches = n;
    return CSA_OK;
}

}  // extern "C"

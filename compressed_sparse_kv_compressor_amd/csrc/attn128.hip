// attn128.hip -- MQA attention for D = 512 and H a multiple of 128 (the decode shape of CSA and HCA).
//
// Method: "DeepSeek-V4 技术解析：架构革新与 Coding Agent 后训练优化", section 1.1: CSA's core attention
// is Multi-Query Attention over the top-k compressed entries plus a sliding window of raw local tokens
// in one softmax; HCA attends densely to every compressed entry ("DeepSeek V4 详解", section "第一刀").
// One stored vector per entry is both key and value.
//
// Kernel layout (one workgroup = 4 waves = 128 heads of one query and one split of its rows):
//   * a wave owns 32 heads x all 512 dims: its Q^T slice (B operand of S^T = K Q^T,
//     v_mfma_f32_32x32x16_bf16) stays in 128 VGPRs and its O^T (16 d-tiles of 32 x 32 fp32) in the
//     256 AGPRs, so a wave's scores are complete after its own QK and nothing moves between waves
//     except the rows themselves;
//   * rows stream through four 32-row LDS tiles (32 KiB each, rows XOR-swizzled per 16-byte chunk)
//     filled by buffer loads to LDS; a tile is issued two steps before its QK, so every load has two
//     tiles of MFMA work to land;
//   * per tile one software-pipelined step: the online softmax of tile t is spread over the 32 QK
//     k-steps of tile t+1, then the PV MFMAs of tile t (V^T read from the same row-major tile with
//     ds_read_b64_tr_b16), then one barrier that recycles tile t's buffer;
//   * every workgroup of a launch runs the same number of steps (rows past the split are masked and
//     the loads past the last tile reread a valid row), so the loop has no data-dependent branch and
//     the load counters stay exact (a split whose tile count is not a multiple of four leaves the
//     unrolled group early, uniformly, and the final wait drains the loads in flight);
//   * FP8 entry rows (592 bytes: e4m3 codes of the 448 non-RoPE dims, the 64 RoPE dims in bf16, one
//     power-of-two scale per 64-dim group) land unswizzled in the top 592 bytes of their row slot, and
//     the wave that loaded a row widens it in place to the bf16 layout above (every decoded value is a
//     bf16 value, so the MFMA loops are those of bf16 rows) before the barrier that publishes the tile.
#include "common.h"
#include "kernels.h"
#include "attn_common.h"

namespace {

using namespace csa;
using namespace csa_attn;

constexpr int A_TPB = 256;
constexpr int NBUF = 4;                  // tile buffers (a split's tile count is a multiple of this)
constexpr int ROWB = 1024;               // bytes of one 512-wide bf16 row
constexpr int FROWB = 512 + 80;          // bytes of one FP8 row (448 codes, 64 bf16 RoPE dims, 16 scale bytes)
constexpr int FOFF = ROWB - FROWB;       // where an FP8 row lands in its slot (chunk 27)

constexpr int A128_QK_AHEAD = 4;         // K-operand LDS reads in flight ahead of the QK MFMAs
constexpr int A128_PV_AHEAD = 2;         // d-tiles of V reads in flight ahead of the PV MFMAs

typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

// R.mode 0: dense prefix (row r = entry r); 1: selected entries, masked padding up to a whole tile,
// then the raw window rows.  The mode is a uniform run-time value (one body serves both jobs of a
// fused launch).
template <bool PAGED, bool ROPE, bool FP8, bool PART>
__device__ __forceinline__ void attn128_body(
    int bid, uint16_t* buf0, uint16_t* buf1, uint16_t* buf2, uint16_t* buf3, int* rcode,
    const uint16_t* __restrict__ q, const Rows& R, int Tq, int H, long long pos0, float scale_log2, int nunits,
    int nsplit, int rps, float* __restrict__ part_o, float2* __restrict__ part_ml, uint16_t* __restrict__ out,
    float* __restrict__ lse)
{
    const int MODE = R.mode;
    constexpr int D = 512;
    constexpr int KS = D / 16;                 // 32x32x16 k-steps of QK
    constexpr int DT = D / 32;                 // 32-wide d-tiles of PV

    const int HQ = H >> 7;
    const int hq = bid % HQ, unit = bid / HQ;
    if (unit >= nunits) return;                // padding workgroups (uniform exit)
    const int bt = unit / nsplit, split = unit % nsplit;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 31, g = lane >> 5;
    const int h = hq * 128 + w * 32 + hl;

    const int b = bt / Tq;
    long long raw0;
    int ndense;
    const long long p = row_geo(R, b, bt % Tq, Tq, pos0, raw0, ndense);
    // MODE 1 row space: [0, topk) selected entries, [topk, topk32) masked padding, [topk32, +window) raw rows
    const int topk32 = MODE == 1 ? (R.topk + TILE - 1) / TILE * TILE : 0;
    int nrows;
    long long w0 = 0;
    if (MODE == 0) {
        nrows = ndense;
    } else {
        w0 = p - R.W + 1 < 0 ? 0 : p - R.W + 1;
        nrows = topk32 + (R.W > 0 ? (int)(p - w0 + 1) : 0);
    }
    const int s_begin = split * rps;
    const int s_end = min(nrows, s_begin + rps);
    const int ntiles = s_begin < nrows ? rps / TILE : 0;   // same for every non-empty split

    const int raw_first = MODE == 1 ? (int)(w0 - raw0) : 0;        // raw row of the first window row
    // The query: the wave's 32 head rows (32 KiB, contiguous) land in tile buffer w by loads to LDS, one
    // 1 KiB row per instruction with the row slots' chunk swizzle, and are read back below in the MFMA
    // layout.  (Loaded straight into registers, each instruction would touch 32 rows x 32 bytes, so every
    // 128-byte line would be fetched by four instructions.)  Issued first, so they overlap the row staging.
    // (the buffer as a 32-bit LDS address, selected in scalar registers.  The FP8-row and rotation
    // variants, whose widening or rotation leaves no registers to spare, load the query straight into
    // registers: staged, they spill.)
    constexpr bool QLDS = !FP8 && !ROPE;
    const uint32_t qbuf = __builtin_amdgcn_readfirstlane(
        (uint32_t)(size_t)(CSA_LDS char*)(w == 0 ? buf0 : (w == 1 ? buf1 : (w == 2 ? buf2 : buf3))));
    if constexpr (QLDS) {
        const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + ((size_t)bt * H + hq * 128 + w * 32) * D, 32u * ROWB);
        const uint32_t l16q = 16u * (uint32_t)lane;
#pragma unroll
        for (int r = 0; r < 32; ++r)           // lane l fetches logical chunk l ^ f(r) into slot position l
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_q, (CSA_LDS void*)(size_t)(qbuf + r * ROWB), 16,
                                                     (int)(l16q ^ (16u * (uint32_t)swz_chunk(r))), r * ROWB, 0, 0);
    }
    // The row of every slot the split will load, staged once in LDS: the entry (dense rows, selected
    // entries) or the raw row (window); -1 for masked slots (unselected padding, rows past the visible
    // ones, and the tiles loaded past the end), which load row 0 and get no weight.
    const int nstage = ntiles * TILE + NBUF * TILE;
    for (int i = threadIdx.x; i < nstage; i += A_TPB) {
        const int r = s_begin + i;
        int v = -1;
        if (r < s_end) {
            if (MODE == 0) v = r;
            else if (r < R.topk) v = R.idx[(size_t)bt * R.topk + r];
            else if (r >= topk32) v = raw_first + (r - topk32);
            if (PAGED && v >= 0 && (MODE == 0 || r < R.topk)) v = (int)entry_row(R.pm, b, R.N, v);
        }
        rcode[i] = v;
    }
    __syncthreads();

    // paged entries address the whole pool (the staged rows are pool rows); batch-major ones this sequence's
    constexpr int EROWB = FP8 ? FROWB : ROWB;  // bytes of an entry row (raw window rows are always bf16)
    const char* kvb = R.kv ? (PAGED ? (const char*)R.kv : (const char*)R.kv + (size_t)b * R.N * EROWB) : nullptr;
    const size_t kv_rows = PAGED ? (size_t)R.pm.nblocks << R.pm.eshift : (size_t)R.N;
    const uint16_t* rawb = MODE == 1 && R.kv_raw ? R.kv_raw + (size_t)b * R.Lr * D : nullptr;
    const __amdgpu_buffer_rsrc_t rs_kv = make_rsrc(kvb, kvb ? (uint32_t)(kv_rows * EROWB) : 0u);
    const __amdgpu_buffer_rsrc_t rs_raw = make_rsrc(rawb, rawb ? (uint32_t)((size_t)R.Lr * ROWB) : 0u);

    bf16x8_t qreg[KS];
    {
        if constexpr (QLDS) {
            // k-step s of head hl is logical chunk 2s + g of buffer row hl, stored at (2s + g) ^ f(hl)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");          // this wave's query rows landed
            // (qbuf is a multiple of 1 KiB, so the XOR of 32 s acts on the row offset alone)
            const uint32_t qa = qbuf + hl * ROWB + 16 * (g ^ swz_chunk(hl));
#pragma unroll
            for (int s = 0; s < KS; ++s) qreg[s] = as_bf16x8(*(const CSA_LDS u32x4_t*)(size_t)(qa ^ (32u * s)));
        } else {
            const uint16_t* qp = q + ((size_t)bt * H + h) * D + 8 * g;
#pragma unroll
            for (int s = 0; s < KS; ++s) qreg[s] = as_bf16x8(*(const u32x4_t*)(qp + 16 * s));
        }
        if constexpr (ROPE) {                   // fused rotary embedding of the last 64 dims, at +p
#pragma unroll
            for (int s = KS - ROPE_FUSED_RD / 16; s < KS; ++s)
                qreg[s] = as_bf16x8(rope8(__builtin_bit_cast(u32x4_t, qreg[s]), 16 * s + 8 * g, D, R, (double)p));
        }
        // every wave has its query in registers before any tile load reuses the buffers
        if constexpr (QLDS) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    const bf16x8_t qmask = as_bf16x8(u32x4_t{g == 0 ? BF16_NEG_2P100 : 0u, 0u, 0u, 0u});
    f32x16_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // ---- tile loads ----
    // Wave w moves row slots 8w .. 8w+7 of a tile, one 1 KiB row per instruction (16 B per lane, landing
    // at slot * 1 KiB + 16 lane); the XOR swizzle goes on the source: lane l fetches logical chunk
    // l ^ f(slot).  The rows come from the staged list (wave-uniform scalar offsets); a tile of window
    // rows reads the raw array.  One group of 8 loads serves every kind of tile, so the compiler's
    // tracking of loads into LDS stays exact (a read waits only for the loads of its own buffer).
    const uint32_t lane16 = 16u * (uint32_t)lane;
    // (FP8 tiles: lane l >= 27 fetches chunk l - 27 of the 592-byte row into chunk l of the slot; the lanes
    // below repeat chunks of the same row into slot bytes that the widening overwrites)
    auto issue = [&](uint16_t* bufp, int t) {
        CSA_LDS char* lb = (CSA_LDS char*)bufp + w * 8 * ROWB;
        const bool from_raw = MODE == 1 && s_begin + t * TILE >= topk32 && R.W > 0;
        const __amdgpu_buffer_rsrc_t rs = from_raw ? rs_raw : rs_kv;
        const CSA_LDS int* cp = (const CSA_LDS int*)rcode + t * TILE + 8 * w;
        const u32x4_t c0 = *(const CSA_LDS u32x4_t*)cp, c1 = *(const CSA_LDS u32x4_t*)(cp + 4);
        uint32_t l16 = lane16;
        asm volatile("" : "+v"(l16));             // per-issue lane offsets (nothing held across the loop)
        if constexpr (FP8) {
            // both kinds of rows land unswizzled (the widening puts every chunk in its place)
            const uint32_t voff = from_raw ? l16 : (lane >= FOFF / 16 ? l16 - FOFF : l16);
            const uint32_t rowb = from_raw ? ROWB : FROWB;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = (int)__builtin_amdgcn_readfirstlane(k < 4 ? c0[k] : c1[k - 4]);
                const uint32_t row = (uint32_t)(c >= 0 ? c : 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (CSA_LDS void*)(lb + ROWB * k), 16, (int)voff,
                                                         (int)(row * rowb), 0, 0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = (int)__builtin_amdgcn_readfirstlane(k < 4 ? c0[k] : c1[k - 4]);
                const uint32_t row = (uint32_t)(c >= 0 ? c : 0);
                const uint32_t voff = l16 ^ (16u * (uint32_t)swz_chunk(8 * w + k));   // w, k uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (CSA_LDS void*)(lb + ROWB * k), 16, (int)voff,
                                                         (int)(row * ROWB), 0, 0);
            }
        }
    };
    // FP8 tiles: each wave widens the 8 rows it loaded, once its own loads of the tile have landed.  Lane l
    // writes logical chunk l (dims 8l .. 8l+7) of the bf16 row at its swizzled place: from 8 codes times
    // the group's scale (l < 56) or from the stored bf16 RoPE dims.  A row's write takes its data from every
    // read of that row, so it is issued after them, and LDS executes one wave's instructions in order: the
    // in-place widening never overwrites bytes still to be read.  (Raw tiles land unswizzled too, and the
    // same pass moves each chunk to its place.)
    auto widen = [&](uint16_t* bufp, int t) {
        if constexpr (FP8) {
            CSA_LDS char* lb = (CSA_LDS char*)bufp + w * 8 * ROWB;
            if (MODE == 1 && s_begin + t * TILE >= topk32 && R.W > 0) {       // raw rows: swizzle in place
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    CSA_LDS char* rb = lb + ROWB * k;
                    const u32x4_t o = *(const CSA_LDS u32x4_t*)(rb + 16 * lane);
                    *(CSA_LDS u32x4_t*)(rb + 16 * (lane ^ swz_chunk(8 * w + k))) = o;
                }
                return;
            }
            const bool nope = lane < 56;
            const uint32_t a0 = nope ? FOFF + 8 * lane : FOFF + 448 + 16 * (lane - 56);
            const uint32_t sa = FOFF + 576 + (nope ? lane >> 3 : 0);
            const uint32_t keep = nope ? 0u : ~0u;    // RoPE lanes keep the stored bf16 (a select, no branch)
            typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
#pragma unroll
            for (int h = 0; h < 2; ++h) {             // two groups of 4 rows: all reads, then the writes
                u32x2_t x0[4], x1[4];
                uint32_t sb[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const CSA_LDS char* rb = lb + ROWB * (4 * h + k);
                    x0[k] = *(const CSA_LDS u32x2_t*)(rb + a0);
                    x1[k] = *(const CSA_LDS u32x2_t*)(rb + a0 + 8);
                    sb[k] = *(const CSA_LDS uint8_t*)(rb + sa);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float scale = __uint_as_float((sb[k] < 1u ? 1u : sb[k]) << 23);      // 2^(s - 127)
#define CSA_W8(X, HI) __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(X, scale, HI))
                    const u32x4_t o = {(CSA_W8(x0[k][0], false) & ~keep) | (x0[k][0] & keep),
                                       (CSA_W8(x0[k][0], true) & ~keep) | (x0[k][1] & keep),
                                       (CSA_W8(x0[k][1], false) & ~keep) | (x1[k][0] & keep),
                                       (CSA_W8(x0[k][1], true) & ~keep) | (x1[k][1] & keep)};
#undef CSA_W8
                    *(CSA_LDS u32x4_t*)(lb + ROWB * (4 * h + k) + 16 * (lane ^ swz_chunk(8 * w + 4 * h + k))) = o;
                }
            }
        }
    };
    // the lane's row (slot hl) of tile t is a valid row
    auto row_ok = [&](int t) -> bool { return rcode[t * TILE + hl] >= 0; };

    // ---- LDS reads ----
    // QK: k-step s of row hl is logical chunk 2s + g, stored at (2s + g) ^ f(hl): offset qk_off ^ 32 s.
    // PV: the transposed read of rows 8k.. and d-tile d is at ((tr_off ^ (64 d + 32 (k & 1))) + 8 KiB k).
    const uint32_t qk_off = hl * ROWB + 16 * (g ^ swz_chunk(hl));
    const int b16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 4 * (b16 >> 1) + (j16 >> 2);
    const uint32_t tr_off = tr_row * ROWB + 16 * ((2 * (b16 & 1) + ((j16 >> 1) & 1)) ^ swz_chunk(tr_row)) +
                            8 * (j16 & 1);
    auto xhalf_max = [](float v) -> float {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    auto xhalf_sum = [](float v) -> float {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    };

    float x[16];                               // scaled scores of the tile being finished
    // One step: softmax of tile t (x) spread over the QK of tile t+1 (Qbuf; okn = the lane's row of
    // tile t+1 is valid), then PV of tile t (Pbuf); returns the raw scores of tile t+1.
    auto step = [&](const uint16_t* Pbuf, const uint16_t* Qbuf, bool okn) -> f32x16_t {
        const CSA_LDS char* Pb = (const CSA_LDS char*)Pbuf;
        const CSA_LDS char* Qb = (const CSA_LDS char*)Qbuf;
        uint32_t qb = qk_off, trb = tr_off;
        asm volatile("" : "+v"(qb), "+v"(trb));   // keep the per-read XORs in the loop
        constexpr int QK_AHEAD = A128_QK_AHEAD;
        bf16x8_t ka[KS];
        f32x16_t sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
        for (int s = 0; s < QK_AHEAD; ++s) ka[s] = as_bf16x8(*(const CSA_LDS u32x4_t*)(Qb + (qb ^ (32u * s))));
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(x[8], x[9]), fmaxf(x[10], x[11])), fmaxf(fmaxf(x[12], x[13]), fmaxf(x[14], x[15]))));
        __builtin_amdgcn_sched_barrier(0);
        float alpha = 1.f, m_use = 0.f, ps = 0.f;
        u32x4_t pw0, pw1;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            sacc = mfma32_bf16(ka[s], qreg[s], sacc);
            if (s + QK_AHEAD < KS)
                ka[s + QK_AHEAD] = as_bf16x8(*(const CSA_LDS u32x4_t*)(Qb + (qb ^ (32u * (s + QK_AHEAD)))));
            if (s == 0) {
                // rescale only when the running max grows by more than 2^8 (the reference point of the
                // exponentials is free; p stays <= 256)
                mx = xhalf_max(mx);
                const bool grow = mx > m_run + 8.0f;
                alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;     // 0 on the first valid tile
                m_run = grow ? mx : m_run;
                m_use = m_run == -INFINITY ? 0.f : m_run;
            } else if (s <= 8) {
                const int j = 2 * (s - 1);
                x[j] = __builtin_amdgcn_exp2f(x[j] - m_use);                   // masked rows -> 0
                x[j + 1] = __builtin_amdgcn_exp2f(x[j + 1] - m_use);
                ps += x[j] + x[j + 1];
            } else if (s <= 12) {
                const int j = s - 9;
                pw0[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
                pw1[j] = pack_bf16x2(x[8 + 2 * j], x[8 + 2 * j + 1]);
            } else if (s == 13) {
                l_run = l_run * alpha + xhalf_sum(ps);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        {   // masked rows of tile t+1: one more k-step adds -2^100 (adds -0 to valid rows)
            const uint32_t masked = g == 0 && !okn ? BF16_ONE : 0u;
            sacc = mfma32_bf16(as_bf16x8(u32x4_t{masked, 0u, 0u, 0u}), qmask, sacc);
        }
        // (rare) the running max grew: rescale the accumulators before this tile's PV
        if (__builtin_expect(__builtin_amdgcn_readfirstlane((uint32_t)__ballot(alpha != 1.0f) |
                                                            (uint32_t)(__ballot(alpha != 1.0f) >> 32)) != 0u, 0)) {
#pragma unroll
            for (int d = 0; d < DT; ++d) acc[d] *= alpha;
        }
        const bf16x8_t pb0 = as_bf16x8(pw0), pb1 = as_bf16x8(pw1);
        // ---- O^T[d][h] += V^T P^T (rows in two k-steps of 16); V reads run PV_AHEAD d-tiles ahead ----
        auto trd = [&](uint32_t off) -> u32x2_t {
            return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (CSA_LDS i16x4_t*)const_cast<CSA_LDS char*>(Pb + off)));
        };
        constexpr int PV_AHEAD = A128_PV_AHEAD;
        u32x2_t vr[DT][4];
        auto load_d = [&](int d) {
            const uint32_t e = trb ^ (64u * d), o = trb ^ (64u * d + 32u);
            vr[d][0] = trd(e);
            vr[d][1] = trd(o + 8u * ROWB);
            vr[d][2] = trd(e + 16u * ROWB);
            vr[d][3] = trd(o + 24u * ROWB);
        };
#pragma unroll
        for (int d = 0; d < PV_AHEAD; ++d) load_d(d);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < DT; ++d) {
            const u32x2_t* v = vr[d];
            acc[d] = mfma32_bf16(as_bf16x8(u32x4_t{v[0][0], v[0][1], v[1][0], v[1][1]}), pb0, acc[d]);
            acc[d] = mfma32_bf16(as_bf16x8(u32x4_t{v[2][0], v[2][1], v[3][0], v[3][1]}), pb1, acc[d]);
            if (d + PV_AHEAD < DT) load_d(d + PV_AHEAD);
            __builtin_amdgcn_sched_barrier(0);
        }
        return sacc;
    };

    // ---- the tile pipeline ----
    // Tile t lives in buffer t % 4.  At the start of step t tiles t and t+1 are in LDS for every wave and
    // tiles t+2, t+3 are in flight.  Step t: softmax(t) + QK(t+1), PV(t); then each wave waits for its
    // own loads of tile t+2 (tile t+3's stay in flight), one barrier makes tile t+2 complete everywhere
    // and frees buffer t % 4 (PV(t) done by all), which takes the loads of tile t+4.  The last step's QK
    // runs on a buffer of dummy rows and is dropped.
    if (ntiles > 0) {
        issue(buf0, 0);
        issue(buf1, 1);
        issue(buf2, 2);
        issue(buf3, 3);
        if constexpr (FP8) {
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");               // this wave's rows of tiles 0, 1
            widen(buf0, 0);
            widen(buf1, 1);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");     // tiles 0 and 1 landed
        }
        const CSA_LDS char* Qb = (const CSA_LDS char*)buf0;
        f32x16_t s0;
#pragma unroll
        for (int j = 0; j < 16; ++j) s0[j] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            s0 = mfma32_bf16(as_bf16x8(*(const CSA_LDS u32x4_t*)(Qb + (qk_off ^ (32u * s)))), qreg[s], s0);
        const uint32_t masked = g == 0 && !row_ok(0) ? BF16_ONE : 0u;
        s0 = mfma32_bf16(as_bf16x8(u32x4_t{masked, 0u, 0u, 0u}), qmask, s0);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = s0[i] * scale_log2;
    }
    for (int t = 0; t < ntiles; t += NBUF) {
#define CSA_A128_STEP(PB, QB, NB, K)                                                                 \
        {                                                                                            \
            const f32x16_t sn = step(PB, QB, row_ok(t + K + 1));                                     \
            if constexpr (FP8) {                                                                     \
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");     /* this wave's rows of t+K+2 */   \
                widen(NB, t + K + 2);                                                                \
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                      \
            } else {                                                                                 \
                asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");  /* tile t+K+2 landed */ \
            }                                                                                        \
            issue(PB, t + K + 4);                                                                    \
            _Pragma("unroll") for (int i = 0; i < 16; ++i) x[i] = sn[i] * scale_log2;              \
        }
        // (PART: a split of ntiles % 4 != 0 tiles, whose last group ends early, uniformly; a compile-time
        //  switch, since the guards cost the other launches their register allocation)
        CSA_A128_STEP(buf0, buf1, buf2, 0)
        if (!PART || t + 1 < ntiles) CSA_A128_STEP(buf1, buf2, buf3, 1)
        if (!PART || t + 2 < ntiles) CSA_A128_STEP(buf2, buf3, buf0, 2)
        if (!PART || t + 3 < ntiles) CSA_A128_STEP(buf3, buf0, buf1, 3)
#undef CSA_A128_STEP
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // the dummy loads past the last tile

    // ---- output ----
    const bool empty = !(m_run > EMPTY_M);     // no valid row: garbage-weighted sums under a tiny max
    if (empty) {
        m_run = -INFINITY;
        l_run = 0.f;
    }
    // lane holds O^T[d*32 + 8 (j/4) + 4 g + j%4][h]
    if (nsplit == 1) {
        // (a launch with an attention sink or the fused rotary embedding and a single split runs k_attn64
        // instead; the sink and the output's rotation of a split launch are applied by the merge)
        const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
        uint16_t* op = out + ((size_t)bt * H + h) * D + 4 * g;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint2 v;
                v.x = pack_bf16x2(acc[d][4 * q4] * inv, acc[d][4 * q4 + 1] * inv);
                v.y = pack_bf16x2(acc[d][4 * q4 + 2] * inv, acc[d][4 * q4 + 3] * inv);
                *(uint2*)(op + d * 32 + 8 * q4) = v;
            }
        if (lse && g == 0) lse[(size_t)bt * H + h] = l_run > 0.f ? (m_run + log2f(l_run)) * LN2 : -INFINITY;
    } else {
        // Split partial, scaled by an exact power of two so that it fits fp16: with 2^e >= max |O| over the
        // head's 512 values, store O 2^-e (fp16, round to nearest even) with m + e and l 2^-e, which leaves
        // every term of the merge 2^(m_s - M) O_s / sum 2^(m_s - M) l_s unchanged.  Layout per (query,
        // split, head quad): [wave][chunk c][lane][8], chunk c = acc[c / 2][8 (c % 2) .. + 8], so each store
        // instruction writes 1 KiB of contiguous memory.
        float amax = 0.f;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
            for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(acc[d][j]));
        amax = xhalf_max(amax);
        const int e = empty || !(amax > 0.f) ? 0 : __builtin_amdgcn_frexp_expf(amax);   // amax < 2^e
        const float sc = empty ? 0.f : __builtin_amdgcn_ldexpf(1.0f, -e);
        const size_t slot = ((size_t)bt * nsplit + split) * HQ + hq;
        uint16_t* op = (uint16_t*)part_o + ((slot * 4 + w) * 32) * 64 * 8 + lane * 8;
        typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
        auto ph = [&](float a, float b2) -> uint32_t {
            const f16x2_t v = {(_Float16)(a * sc), (_Float16)(b2 * sc)};
            return __builtin_bit_cast(uint32_t, v);
        };
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const f32x16_t& a = acc[c / 2];
            const int j0 = 8 * (c % 2);
            *(u32x4_t*)(op + c * 64 * 8) = u32x4_t{ph(a[j0], a[j0 + 1]), ph(a[j0 + 2], a[j0 + 3]),
                                                   ph(a[j0 + 4], a[j0 + 5]), ph(a[j0 + 6], a[j0 + 7])};
        }
        if (g == 0) part_ml[(slot * 4 + w) * 32 + hl] = make_float2(m_run + (float)e, l_run * sc);
    }
}

// (by value: a bit cast applied directly to an element of a vector value is miscompiled)
__device__ __forceinline__ __attribute__((ext_vector_type(2))) _Float16 as_f16x2(uint32_t x) {
    return __builtin_bit_cast(__attribute__((ext_vector_type(2))) _Float16, x);
}

// Merge of the fp16 split partials written above, in split order: out = sum_s 2^(m_s-M) o_s /
// sum_s 2^(m_s-M) l_s.  Thread tid (0 .. 8191 per query and head quad) owns one 16-byte chunk position
// (wave w, chunk c, lane) of every split.
__device__ __forceinline__ void combine128_body(const uint16_t* __restrict__ part, const float2* __restrict__ part_ml,
                                                int H, int nsplit, uint16_t* __restrict__ out,
                                                float* __restrict__ lse, const float* __restrict__ sink, int bt,
                                                int hq, int tid, const Rows& R, int Tq, long long pos0)
{
    const int HQ = H >> 7;
    const int w = tid >> 11, c = (tid >> 6) & 31, lane = tid & 63;
    const int hl = lane & 31, g = lane >> 5;
    const int h = hq * 128 + w * 32 + hl;
    const size_t slot0 = (size_t)bt * nsplit * HQ + hq;          // split s at slot0 + s HQ
    const float2* mlp = part_ml + (slot0 * 4 + w) * 32 + hl;       // split s at mlp[s HQ 128]
    const uint16_t* pp = part + (((slot0 * 4 + w) * 32 + c) * 64 + lane) * 8;   // split s at pp[s HQ 2^19]
    const size_t ml_step = (size_t)HQ * 128, p_step = (size_t)HQ * 4 * 32 * 64 * 8;
    constexpr int UM = 32, U = 16;                                 // splits in flight (maxima, partials)
    float M = -INFINITY;
    for (int s0 = 0; s0 < nsplit; s0 += UM) {
        float mv[UM];
#pragma unroll
        for (int u = 0; u < UM; ++u) mv[u] = s0 + u < nsplit ? mlp[(size_t)(s0 + u) * ml_step].x : -INFINITY;
#pragma unroll
        for (int u = 0; u < UM; ++u) M = fmaxf(M, mv[u]);
    }
    float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < nsplit; s0 += U) {
            float2 ml[U];
            u32x4_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = s0 + u < nsplit;
                ml[u] = ok ? mlp[(size_t)(s0 + u) * ml_step] : make_float2(-INFINITY, 0.f);
                v[u] = ok ? *(const u32x4_t*)(pp + (size_t)(s0 + u) * p_step) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {          // in split order
                const float f = exp2f(ml[u].x - M);        // 0 for empty or absent splits (m = -inf)
                l += f * ml[u].y;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const auto hv = as_f16x2(v[u][k]);
                    o[2 * k] += f * (float)hv[0];
                    o[2 * k + 1] += f * (float)hv[1];
                }
            }
        }
    }
    float lse_v;
    const float inv = sink_norm(M, l, sink_log2(sink, h), lse_v);
    // o[jj] is O^T[d][h] at d = 32 (c / 2) + 8 ((8 (c % 2) + jj) / 4) + 4 g + jj % 4: two runs of 4
    const int d0 = 32 * (c >> 1) + 16 * (c & 1) + 4 * g;
    if (R.rope_rd && d0 + 12 > 512 - ROPE_FUSED_RD) {     // the output's last 64 dims turn back by -p
        long long raw0;
        int nd;
        const double sp = -(double)row_geo(R, bt / Tq, bt % Tq, Tq, pos0, raw0, nd);
#pragma unroll
        for (int k = 0; k < 4; ++k) CSA_ROPE_PAIR(o, 2 * (k & 1) + 4 * (k >> 1), 2 * (k & 1) + 4 * (k >> 1) + 1, d0 + 2 * (k & 1) + 8 * (k >> 1), 512, R, sp)
    }
    uint16_t* op = out + ((size_t)bt * H + h) * 512 + d0;
    *(uint2*)op = make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
    *(uint2*)(op + 8) = make_uint2(pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv));
    if (lse && c == 0 && g == 0) lse[(size_t)bt * H + h] = lse_v;
}

// Tile buffers [32 rows][512] bf16 (distinct objects: the compiler tells a read of one from the loads in
// flight into another) and the split's staged entry indices.
#define CSA_A128_LDS                                                        \
    __shared__ __attribute__((aligned(1024))) uint16_t buf0[TILE * 512];    \
    __shared__ __attribute__((aligned(1024))) uint16_t buf1[TILE * 512];    \
    __shared__ __attribute__((aligned(1024))) uint16_t buf2[TILE * 512];    \
    __shared__ __attribute__((aligned(1024))) uint16_t buf3[TILE * 512];    \
    __shared__ __attribute__((aligned(16))) int rcode[csa_host::ATT128_MAX_RPS + NBUF * TILE];

// Two job slots: workgroups [0, nblk_s) run job s, the rest job d; one job is launched with every workgroup
// below nblk_s.  (With the parameters selected per workgroup like this the compiler allocates the body's
// registers without spills; with the job's fields passed straight in it spilled ~100 VGPRs.)
template <bool PAGED, bool ROPE, bool FP8, bool PART>
__global__ __launch_bounds__(A_TPB, 1) void k_attn128(AttnJob js, AttnJob jd, int nblk_s)
{
    CSA_A128_LDS
    const bool first = (int)blockIdx.x < nblk_s;
    const AttnJob& j = first ? js : jd;
    attn128_body<PAGED, ROPE, FP8, PART>(first ? blockIdx.x : blockIdx.x - nblk_s, buf0, buf1, buf2, buf3, rcode, j.q, j.R, j.Tq, j.H,
                 j.pos0, j.scale_log2, j.nunits, j.nsplit, j.rps, j.part_o, j.part_ml, j.out, j.lse);
}
#undef CSA_A128_LDS

// grid (32, HQ, BT): 256 threads x 32 cover the 8192 chunk positions of one query and head quad
__global__ __launch_bounds__(256) void k_combine128(AttnJob j)
{
    combine128_body((const uint16_t*)j.part_o, j.part_ml, j.H, j.nsplit, j.out, j.lse, j.R.sink, blockIdx.z,
                    blockIdx.y, blockIdx.x * 256 + threadIdx.x, j.R, j.Tq, j.pos0);
}

}  // namespace

namespace csa_host {

int attn128_launch(const csa_attn::AttnJob& j, hipStream_t st, const char* tag) {
    const int HQ = j.H / 128, BT = j.nunits / j.nsplit;
    const int nblk = j.nunits * HQ;
    // (paged entries, the fused rotary embedding and FP8 entry rows: compile-time switches, so that the plain
    // kernel carries none of their code, whose registers it cannot spare)
    const bool paged = j.R.pm.table != nullptr, rope = j.R.rope_rd != 0, fp8 = j.R.kv_fp8 != 0;
    const bool part = (j.rps / TILE) % NBUF != 0;
#define CSA_A128(P_, R_, F_)                                                                                 \
    do {                                                                                                     \
        if (part) CSA_LAUNCH(tag, (k_attn128<P_, R_, F_, true>), dim3(nblk), dim3(A_TPB), 0, st, j, j, nblk);  \
        else CSA_LAUNCH(tag, (k_attn128<P_, R_, F_, false>), dim3(nblk), dim3(A_TPB), 0, st, j, j, nblk);      \
    } while (0)
    if (fp8) {
        if (paged && rope) CSA_A128(true, true, true);
        else if (paged) CSA_A128(true, false, true);
        else if (rope) CSA_A128(false, true, true);
        else CSA_A128(false, false, true);
    } else {
        if (paged && rope) CSA_A128(true, true, false);
        else if (paged) CSA_A128(true, false, false);
        else if (rope) CSA_A128(false, true, false);
        else CSA_A128(false, false, false);
    }
#undef CSA_A128
    if (j.nsplit > 1) CSA_LAUNCH("k_combine", k_combine128, dim3(32, HQ, BT), dim3(256), 0, st, j);
    return 0;
}

}  // namespace csa_host

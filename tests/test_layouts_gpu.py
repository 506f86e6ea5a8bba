"""GPU parity of the batch and cache layouts: variable-length batches (per-sequence token counts), paged
caches (entries reached through a block table), and values kept apart from keys.

Every case is checked per sequence against the oracle run on that sequence alone with its own length and a
contiguous copy of its cache (top-k sets bit-exact, outputs within 2e-2 of each row's largest magnitude),
and where the same kernel runs on both layouts, bitwise against the plain-layout call.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_kv_compressor_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_sparse_kv_compressor_amd import binding
    return binding


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(DEV)


def bf16_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rows_close(got_bits, want, what=""):
    g = bf16_f64(got_bits).reshape(-1, want.shape[-1])
    o = want.reshape(-1, want.shape[-1])
    err = np.abs(g - o).max(1) / np.maximum(np.abs(o).max(1), 1e-30)
    assert err.max() <= TOL, f"{what}: worst row error {err.max():.3g}"


def paged(arr, epb, seed, spare=3):
    """Scatter a batch-major cache [B][N][...] into a pool of pages of epb entries in shuffled order;
    returns (pool, table [B][max_blocks] int32, num_blocks)."""
    B, N = arr.shape[:2]
    mb = -(-N // epb)
    nblk = B * mb + spare
    perm = np.random.default_rng(seed).permutation(nblk)[:B * mb].astype(np.int32).reshape(B, mb)
    pool = np.zeros((nblk * epb,) + arr.shape[2:], arr.dtype)
    for bb in range(B):
        for k in range(mb):
            n = min(epb, N - k * epb)
            pool[perm[bb, k] * epb:perm[bb, k] * epb + n] = arr[bb, k * epb:k * epb + n]
    return pool, perm, nblk


# ---------------------------------------------------------------------------
# indexer + top-k
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("Tq", [1, 3])
@pytest.mark.parametrize("block_tokens", [0, 128, 4])     # batch-major; pages of 32 entries; of one entry
def test_index_topk_varlen(b, dtype, Tq, block_tokens):
    B, HI, dI, m, topk = 4, 8, 128, 4, 256
    L = 4 * 3000
    lens = np.array([L, 7001, 900, 5555], np.int64)
    Nc = L // m
    q, w, k, _ = synth.indexer_inputs(50 + dtype + Tq, B, Tq, HI, dI, Nc, dtype)
    layout_args = dict(seq_lens=dev(lens))
    kin = k
    if block_tokens:
        kin, table, nblk = paged(k, block_tokens // m, 7)
        layout_args.update(block_table=dev(table), num_blocks=nblk, block_tokens=block_tokens)
    lay = b.make_layout(**layout_args)
    idx = torch.empty((B, Tq, topk), dtype=torch.int32, device=DEV)
    cnt = torch.empty((B, Tq), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, Tq, topk), dtype=torch.float32, device=DEV)
    b.csa_index_topk(dev(q), dev(w), dev(kin), dtype, L, m, L - Tq, topk, idx, cnt, score_out=sc, layout=lay, Nc=Nc)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    for bb in range(B):
        Lb = int(lens[bb])
        Ncb = -(-Lb // m)
        want, wc, _, _ = oracle.index_topk(q[bb:bb + 1], w[bb:bb + 1], k[bb:bb + 1, :Ncb], Lb, m, Lb - Tq, topk, dtype)
        assert np.array_equal(gi[bb], want[0]), f"sequence {bb} (L={Lb})"
        assert np.array_equal(gc[bb], wc[0])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

SPARSE = [  # (B, Tq, H, D, W)
    (3, 1, 128, 512, 128),     # k_attn128
    (3, 2, 64, 512, 64),       # k_attn64
    (3, 2, 16, 128, 32),       # generic kernel
]


def sparse_case(seed, B, Tq, H, D, W, lens, Nc, topk):
    q, kv = synth.attn_inputs(seed, B, Tq, H, D, Nc, "vl_")
    Lr = Tq + W - 1
    _, raw = synth.attn_inputs(seed, B, 1, H, D, Lr, "vlraw_")
    g = np.random.default_rng(seed)
    idx = np.full((B, Tq, topk), -1, np.int32)
    for bb in range(B):
        ncb = -(-int(lens[bb]) // 4)
        for t in range(Tq):
            n = min(topk, ncb)
            idx[bb, t, :n] = np.sort(g.choice(ncb, n, replace=False))
    return q, kv, raw, idx, Lr


@pytest.mark.parametrize("case", SPARSE)
@pytest.mark.parametrize("paged_kv", [False, True])
def test_sparse_attn_varlen(b, case, paged_kv):
    B, Tq, H, D, W = case
    topk, Nc = 200, 3000
    lens = np.array([Nc * 4, Nc * 4 - 777, 100], np.int64)
    q, kv, raw, idx, Lr = sparse_case(60 + H, B, Tq, H, D, W, lens, Nc, topk)
    lay_args = dict(seq_lens=dev(lens))
    kvin = kv
    if paged_kv:
        kvin, table, nblk = paged(kv, 32, 8)
        lay_args.update(block_table=dev(table), num_blocks=nblk, block_tokens=128)
    out = torch.empty((B, Tq, H, D), dtype=torch.int16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    b.csa_sparse_attn(dev(q), dev(kvin), dev(idx), dev(raw), 0, 0, W, D ** -0.5, out, lse,
                      layout=b.make_layout(**lay_args), m=4, Nc=Nc)
    torch.cuda.synchronize()
    go, gl = out.cpu().numpy().view(np.uint16), lse.cpu().numpy()
    for bb in range(B):
        Lb = int(lens[bb])
        o, l = oracle.sparse_attn(q[bb:bb + 1], kv[bb:bb + 1], idx[bb:bb + 1], raw[bb:bb + 1], Lb - Lr, Lb - Tq, W,
                                  D ** -0.5)
        rows_close(go[bb], o[0], f"sequence {bb}")
        assert np.abs(gl[bb] - l[0]).max() <= TOL


@pytest.mark.parametrize("H,D", [(128, 512), (64, 512), (16, 128)])
@pytest.mark.parametrize("paged_kv", [False, True])
def test_dense_attn_varlen(b, H, D, paged_kv):
    B, Tq, mh = 3, 2, 128
    L = 128 * 700
    Nh = L // mh
    lens = np.array([L, L - 5000 - 37, 130], np.int64)
    q, kvh = synth.attn_inputs(70 + H, B, Tq, H, D, Nh, "vd_")
    lay_args = dict(seq_lens=dev(lens))
    kin = kvh
    if paged_kv:
        kin, table, nblk = paged(kvh, 1, 9)
        lay_args.update(block_table=dev(table), num_blocks=nblk, block_tokens=128)
    out = torch.empty((B, Tq, H, D), dtype=torch.int16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    b.hca_dense_attn(dev(q), dev(kin), L, mh, L - Tq, D ** -0.5, out, lse, layout=b.make_layout(**lay_args))
    torch.cuda.synchronize()
    go, gl = out.cpu().numpy().view(np.uint16), lse.cpu().numpy()
    for bb in range(B):
        Lb = int(lens[bb])
        Nhb = -(-Lb // mh)
        o, l = oracle.dense_attn(q[bb:bb + 1], kvh[bb:bb + 1, :Nhb], Lb, mh, Lb - Tq, D ** -0.5)
        rows_close(go[bb], o[0], f"sequence {bb}")
        assert np.abs(gl[bb] - l[0]).max() <= TOL


def test_paged_equals_plain_bitwise(b):
    # the same kernel on the same rows: paged and batch-major calls agree bit for bit
    B, Tq, H, D, W, topk, Nc, m = 2, 1, 128, 512, 128, 512, 4000, 4
    L = Nc * m
    q, kv = synth.attn_inputs(81, B, Tq, H, D, Nc, "pb_")
    _, raw = synth.attn_inputs(82, B, 1, H, D, W, "pbr_")
    g = np.random.default_rng(3)
    idx = np.stack([np.sort(g.choice(Nc, topk, replace=False)) for _ in range(B)]).astype(np.int32).reshape(B, 1, topk)
    pool, table, nblk = paged(kv, 32, 10)
    outs = []
    for lay, kvin in ((None, kv), (b.make_layout(block_table=dev(table), num_blocks=nblk, block_tokens=128), pool)):
        out = torch.empty((B, Tq, H, D), dtype=torch.int16, device=DEV)
        b.csa_sparse_attn(dev(q), dev(kvin), dev(idx), dev(raw), L - W, L - 1, W, D ** -0.5, out, layout=lay, m=m,
                          Nc=Nc)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    mh = 128
    Nh = L // mh
    qh, kvh = synth.attn_inputs(83, B, Tq, H, D, Nh, "pbh_")
    hpool, htable, hn = paged(kvh, 1, 11)
    res = []
    for lay, kin in ((None, kvh), (b.make_layout(block_table=dev(htable), num_blocks=hn, block_tokens=128), hpool)):
        out = torch.empty((B, Tq, H, D), dtype=torch.int16, device=DEV)
        b.hca_dense_attn(dev(qh), dev(kin), L, mh, L - 1, D ** -0.5, out, layout=lay)
        res.append(out)
    torch.cuda.synchronize()
    assert torch.equal(res[0], res[1])


# ---------------------------------------------------------------------------
# fused decode over a variable-length, paged batch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("paged_kv", [False, True])
def test_fused_decode_varlen(b, paged_kv):
    B, H, D, HI, dI, m, mh, topk, W, dt = 3, 128, 512, 8, 128, 4, 128, 256, 128, 1
    L = 128 * 120
    Nc, Nh = L // m, L // mh
    lens = np.array([L, L - 2000 - 3, 700], np.int64)
    q_idx, w_idx, k_idx, _ = synth.indexer_inputs(90, B, 1, HI, dI, Nc, dt)
    csa_q, kv = synth.attn_inputs(91, B, 1, H, D, Nc, "fd_")
    _, raw = synth.attn_inputs(92, B, 1, H, D, W, "fdr_")
    hca_q, kvh = synth.attn_inputs(93, B, 1, H, D, Nh, "fdh_")
    lay_args = dict(seq_lens=dev(lens))
    kin, kvin, kvhin = k_idx, kv, kvh
    if paged_kv:
        kin, table, nblk = paged(k_idx, 32, 12)
        # one table for the three pools: the same page ids
        kvin = np.zeros((nblk * 32, D), np.uint16)
        kvhin = np.zeros((nblk, D), np.uint16)
        for bb in range(B):
            for k in range(table.shape[1]):
                kvin[table[bb, k] * 32:(table[bb, k] + 1) * 32] = kv[bb, k * 32:(k + 1) * 32]
                kvhin[table[bb, k]] = kvh[bb, k]
        lay_args.update(block_table=dev(table), num_blocks=nblk, block_tokens=128)
    lay = b.make_layout(**lay_args)
    csa_out = torch.empty((B, H, D), dtype=torch.int16, device=DEV)
    hca_out = torch.empty_like(csa_out)
    idx = torch.empty((B, topk), dtype=torch.int32, device=DEV)
    args = b.make_decode_args(L=L, scale=D ** -0.5, csa_q=dev(csa_q).view(B, H, D), q_idx=dev(q_idx), w_idx=dev(w_idx),
                              k_idx=dev(kin), kv=dev(kvin), kv_raw=dev(raw), idx_dtype=dt, m=m, topk=topk, W=W,
                              csa_out=csa_out, hca_q=dev(hca_q).view(B, H, D), kv_h=dev(kvhin), mh=mh, hca_out=hca_out,
                              idx_out=idx, layout=lay)
    b.csa_hca_decode(args, device=torch.device(DEV))
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    gc, gh = csa_out.cpu().numpy().view(np.uint16), hca_out.cpu().numpy().view(np.uint16)
    for bb in range(B):
        Lb = int(lens[bb])
        Ncb, Nhb = -(-Lb // m), -(-Lb // mh)
        want, _, _, _ = oracle.index_topk(q_idx[bb:bb + 1], w_idx[bb:bb + 1], k_idx[bb:bb + 1, :Ncb], Lb, m, Lb - 1, topk,
                                          dt)
        assert np.array_equal(gi[bb], want[0, 0]), f"sequence {bb}"
        o, _ = oracle.sparse_attn(csa_q[bb:bb + 1], kv[bb:bb + 1], want, raw[bb:bb + 1], Lb - W, Lb - 1, W, D ** -0.5)
        rows_close(gc[bb], o[0, 0], f"csa sequence {bb}")
        o, _ = oracle.dense_attn(hca_q[bb:bb + 1], kvh[bb:bb + 1, :Nhb], Lb, mh, Lb - 1, D ** -0.5)
        rows_close(gh[bb], o[0, 0], f"hca sequence {bb}")


# ---------------------------------------------------------------------------
# separate keys and values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,D", [(128, 512), (64, 512), (16, 128)])
def test_separate_values(b, H, D):
    B, Tq, W, topk, Nc = 2, 2, 48, 300, 2000
    q, kv = synth.attn_inputs(100 + H, B, Tq, H, D, Nc, "sv_k_")
    _, v = synth.attn_inputs(101 + H, B, Tq, H, D, Nc, "sv_v_")
    Lr = Tq + W - 1
    _, raw = synth.attn_inputs(102 + H, B, 1, H, D, Lr, "sv_rk_")
    _, vraw = synth.attn_inputs(103 + H, B, 1, H, D, Lr, "sv_rv_")
    g = np.random.default_rng(H)
    idx = np.stack([np.stack([np.sort(g.choice(Nc, topk, replace=False)) for _ in range(Tq)]) for _ in range(B)])
    idx = idx.astype(np.int32)
    pos0 = Nc * 4 - Tq
    raw0 = pos0 - W + 1
    out = torch.empty((B, Tq, H, D), dtype=torch.int16, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    sink = torch.from_numpy(synth.sink_logits(5, H, "svs_")).to(DEV)
    b.csa_sparse_attn(dev(q), dev(kv), dev(idx), dev(raw), raw0, pos0, W, D ** -0.5, out, lse, v=dev(v),
                      v_raw=dev(vraw), sink=sink)
    torch.cuda.synchronize()
    o, l = oracle.sparse_attn(q, kv, idx, raw, raw0, pos0, W, D ** -0.5, sink=sink.cpu().numpy(), v=v, v_raw=vraw)
    rows_close(out.cpu().numpy().view(np.uint16), o, "sparse")
    assert np.abs(lse.cpu().numpy() - l).max() <= TOL
    # dense with separate values
    mh = 4
    L = Nc * mh
    outd = torch.empty((B, Tq, H, D), dtype=torch.int16, device=DEV)
    b.hca_dense_attn(dev(q), dev(kv), L, mh, L - Tq, D ** -0.5, outd, v_h=dev(v))
    torch.cuda.synchronize()
    o, _ = oracle.dense_attn(q, kv, L, mh, L - Tq, D ** -0.5, v_h=v)
    rows_close(outd.cpu().numpy().view(np.uint16), o, "dense")

"""Incremental compression during decode (csa_decode_append) against the oracle's compression of the whole
prefix, on a variable-length batch, with batch-major and paged caches.

A batch whose sequences were compressed in bulk (csa_hca_compress of their first 256 / 384 tokens) takes
single-token and multi-token appends that cross CSA and HCA block boundaries.  After every append the CSA
entries (KV rows and indexer keys), the HCA entries and the window rows must match the oracle's
compression of each sequence's whole prefix (2e-2 of each row's largest magnitude; e4m3 keys also get
their half-step), the open blocks' entries included, and seq_lens must have advanced on the device.  The
appended caches then serve a fused decode pair whose top-k is bit-exact and whose outputs match the oracle
run on those caches.
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


def rows_close(got, want, what):
    g = got.reshape(-1, want.shape[-1])
    o = want.reshape(-1, want.shape[-1])
    err = np.abs(g - o).max(1) / np.maximum(np.abs(o).max(1), 1e-30)
    assert err.max() <= TOL, f"{what}: worst row error {err.max():.3g} (row {int(err.argmax())})"


def e4m3_close(got_bits, want, what):
    g = oracle.e4m3_value(got_bits).reshape(-1, want.shape[-1])
    o = want.reshape(-1, want.shape[-1])
    bound = 0.0625 * np.abs(o) + TOL * np.abs(o).max(axis=1, keepdims=True) + 2.0 ** -10
    assert np.all(np.abs(g - o) <= bound), what


class Pager:
    """Shuffled page table over a pool of pages of `block_tokens` raw tokens."""

    def __init__(self, B, L, block_tokens, seed):
        self.bt = block_tokens
        self.mb = -(-L // block_tokens)
        self.nblk = B * self.mb + 2
        self.table = np.random.default_rng(seed).permutation(self.nblk)[:B * self.mb].astype(np.int32).reshape(B, self.mb)

    def scatter(self, arr, ratio):
        epb = self.bt // ratio
        B, N = arr.shape[:2]
        pool = np.zeros((self.nblk * epb,) + arr.shape[2:], arr.dtype)
        for bb in range(B):
            for k in range(self.mb):
                n = max(0, min(epb, N - k * epb))
                pool[self.table[bb, k] * epb:self.table[bb, k] * epb + n] = arr[bb, k * epb:k * epb + n]
        return pool

    def gather(self, pool, ratio, bb, n):
        epb = self.bt // ratio
        rows = [self.table[bb, j // epb] * epb + j % epb for j in range(n)]
        return pool[rows]


@pytest.mark.parametrize("ik_dtype", [0, 1])
@pytest.mark.parametrize("paged", [False, True])
def test_append_matches_prefix_compression(b, ik_dtype, paged):
    B, Dh, D, dI, m, mh, W, L = 2, 1024, 512, 128, 4, 128, 128, 1024
    Nc, Nh = L // m, L // mh
    L0 = [256, 384]
    X, wkv, wik, gate, _ = synth.compress_inputs(120 + ik_dtype, B, L, Dh, D, dI, m, heavy=True, gate_scale=2.0)
    bslot = synth.normal_f32(120, "ap_b_slot", (m,), 0.5)
    wkv_h, _, gate_h, _ = synth.compress_weights(121, Dh, D, 0, mh, gate_scale=2.0, prefix="ap_hca_")
    bslot_h = synth.normal_f32(121, "ap_b_slot_h", (mh,), 0.5)
    W_ = dict(wkv=dev(wkv), wik=dev(wik), gate=dev(gate), bslot=dev(bslot), wkv_h=dev(wkv_h), gate_h=dev(gate_h),
              bslot_h=dev(bslot_h))
    ikt = torch.int16 if ik_dtype == 0 else torch.uint8
    # bulk compression of each sequence's first L0[b] tokens into capacity-sized caches
    kv_c = np.zeros((B, Nc, D), np.uint16)
    ik_c = np.zeros((B, Nc, dI), np.uint16 if ik_dtype == 0 else np.uint8)
    kvh_c = np.zeros((B, Nh, D), np.uint16)
    win = torch.zeros((B, W, D), dtype=torch.int16, device=DEV)
    for bb in range(B):
        n, nh = L0[bb] // m, L0[bb] // mh
        kv1 = torch.empty((1, n, D), dtype=torch.int16, device=DEV)
        ik1 = torch.empty((1, n, dI), dtype=ikt, device=DEV)
        kvh1 = torch.empty((1, nh, D), dtype=torch.int16, device=DEV)
        win1 = torch.empty((1, W, D), dtype=torch.int16, device=DEV)
        b.csa_hca_compress(dev(X[bb:bb + 1, :L0[bb]]), W_["wkv"], W_["wik"], W_["gate"], W_["bslot"], m, W, kv1, ik1,
                           win1, W_["wkv_h"], W_["gate_h"], W_["bslot_h"], mh, kvh1, ik_dtype=ik_dtype)
        torch.cuda.synchronize()
        kv_c[bb, :n] = kv1[0].cpu().numpy().view(np.uint16)
        ik_c[bb, :n] = ik1[0].cpu().numpy().view(ik_c.dtype)
        kvh_c[bb, :nh] = kvh1[0].cpu().numpy().view(np.uint16)
        win[bb] = win1[0]
    layout = None
    if paged:
        pg = Pager(B, L, 128, 5)
        kv_d, ik_d, kvh_d = dev(pg.scatter(kv_c, m)), dev(pg.scatter(ik_c, m)), dev(pg.scatter(kvh_c, mh))
        layout = b.make_layout(block_table=dev(pg.table), num_blocks=pg.nblk, block_tokens=128)
    else:
        kv_d, ik_d, kvh_d = dev(kv_c), dev(ik_c), dev(kvh_c)
    seq = torch.tensor(L0, dtype=torch.int64, device=DEV)
    state = torch.zeros(B * b.lib.csa_append_state_bytes(D, dI) // 4, dtype=torch.float32, device=DEV)
    lens = list(L0)
    for T in (1, 1, 1, 3, 1, 37, 1, 90, 2):
        chunk = np.stack([X[bb, lens[bb]:lens[bb] + T] for bb in range(B)])
        b.csa_decode_append(dev(chunk), W_["wkv"], W_["wik"], W_["gate"], W_["bslot"], m, W_["wkv_h"], W_["gate_h"],
                            W_["bslot_h"], mh, L, seq, state, kv_d, ik_d, kvh_d, win, ik_dtype=ik_dtype, layout=layout)
        torch.cuda.synchronize()
        lens = [x + T for x in lens]
        assert seq.cpu().tolist() == lens
        kv_h_, ik_h_, kvh_h_ = kv_d.cpu().numpy(), ik_d.cpu().numpy(), kvh_d.cpu().numpy()
        win_h = win.cpu().numpy().view(np.uint16)
        for bb in range(B):
            Lb = lens[bb]
            nc, nh = -(-Lb // m), -(-Lb // mh)
            okv, oik, ow = oracle.compress(X[bb:bb + 1, :Lb], wkv, wik, gate, bslot, m, W=W)
            okh, _, _ = oracle.compress(X[bb:bb + 1, :Lb], wkv_h, None, gate_h, bslot_h, mh)
            if paged:
                g_kv = pg.gather(kv_h_, m, bb, nc)
                g_ik = pg.gather(ik_h_, m, bb, nc)
                g_kh = pg.gather(kvh_h_, mh, bb, nh)
            else:
                g_kv, g_ik, g_kh = kv_h_[bb, :nc], ik_h_[bb, :nc], kvh_h_[bb, :nh]
            what = f"T={T} sequence {bb} L={Lb}"
            rows_close(bf16_f64(g_kv.view(np.uint16)), okv[0], "kv " + what)
            rows_close(bf16_f64(g_kh.view(np.uint16)), okh[0], "kv_h " + what)
            if ik_dtype == 0:
                rows_close(bf16_f64(g_ik.view(np.uint16)), oik[0], "ik " + what)
            else:
                e4m3_close(g_ik.view(np.uint8), oik[0], "ik " + what)
            rows_close(bf16_f64(win_h[bb]), ow[0], "window " + what)

    # the appended caches serve a decode pair (variable lengths, same layout)
    H, HI, topk = 128, 8, 64
    q_idx = synth.encode(synth.normal_f32(7, "ap_q_idx", (B, 1, HI, dI), dI ** -0.5), ik_dtype)
    w_idx = synth.half_normal_f32(7, "ap_w_idx", (B, 1, HI), HI ** -0.5)
    csa_q, _ = synth.attn_inputs(7, B, 1, H, D, 1, "ap_csa_")
    hca_q, _ = synth.attn_inputs(7, B, 1, H, D, 1, "ap_hca_")
    dlay = b.make_layout(seq_lens=seq, block_table=dev(pg.table) if paged else None,
                         num_blocks=pg.nblk if paged else 0, block_tokens=128 if paged else 0)
    csa_out = torch.empty((B, H, D), dtype=torch.int16, device=DEV)
    hca_out = torch.empty_like(csa_out)
    idx = torch.empty((B, topk), dtype=torch.int32, device=DEV)
    args = b.make_decode_args(L=L, scale=D ** -0.5, csa_q=dev(csa_q).view(B, H, D), q_idx=dev(q_idx), w_idx=dev(w_idx),
                              k_idx=ik_d, kv=kv_d, kv_raw=win, idx_dtype=ik_dtype, m=m, topk=topk, W=W,
                              csa_out=csa_out, hca_q=dev(hca_q).view(B, H, D), kv_h=kvh_d, mh=mh, hca_out=hca_out,
                              idx_out=idx, layout=dlay)
    b.csa_hca_decode(args, device=torch.device(DEV))
    torch.cuda.synchronize()
    kv_h_, ik_h_, kvh_h_ = kv_d.cpu().numpy(), ik_d.cpu().numpy(), kvh_d.cpu().numpy()
    for bb in range(B):
        Lb = lens[bb]
        nc, nh = -(-Lb // m), -(-Lb // mh)
        if paged:
            g_kv, g_ik, g_kh = pg.gather(kv_h_, m, bb, nc), pg.gather(ik_h_, m, bb, nc), pg.gather(kvh_h_, mh, bb, nh)
        else:
            g_kv, g_ik, g_kh = kv_h_[bb, :nc], ik_h_[bb, :nc], kvh_h_[bb, :nh]
        g_kv, g_kh = g_kv.view(np.uint16)[None], g_kh.view(np.uint16)[None]
        g_ik = g_ik.view(np.uint16 if ik_dtype == 0 else np.uint8)[None]
        want, _, _, _ = oracle.index_topk(q_idx[bb:bb + 1], w_idx[bb:bb + 1], g_ik, Lb, m, Lb - 1, topk, ik_dtype)
        assert np.array_equal(idx[bb].cpu().numpy(), want[0, 0])
        o, _ = oracle.sparse_attn(csa_q[bb:bb + 1], g_kv, want, win[bb:bb + 1].cpu().numpy().view(np.uint16), Lb - W,
                                  Lb - 1, W, D ** -0.5)
        rows_close(bf16_f64(csa_out[bb].cpu().numpy().view(np.uint16)), o[0, 0], f"csa decode {bb}")
        o, _ = oracle.dense_attn(hca_q[bb:bb + 1], g_kh, Lb, mh, Lb - 1, D ** -0.5)
        rows_close(bf16_f64(hca_out[bb].cpu().numpy().view(np.uint16)), o[0, 0], f"hca decode {bb}")


def test_append_drops_tokens_beyond_capacity(b):
    B, Dh, D, dI, m, mh, W, L = 1, 256, 64, 0, 4, 8, 16, 40
    X, wkv, _, gate, bslot = synth.compress_inputs(130, B, 64, Dh, D, 0, m)
    wkv_h, _, gate_h, bslot_h = synth.compress_weights(131, Dh, D, 0, mh, prefix="cap_")
    kv = torch.zeros((B, L // m, D), dtype=torch.int16, device=DEV)
    kvh = torch.zeros((B, L // mh, D), dtype=torch.int16, device=DEV)
    win = torch.zeros((B, W, D), dtype=torch.int16, device=DEV)
    seq = torch.tensor([32], dtype=torch.int64, device=DEV)
    state = torch.zeros(B * b.lib.csa_append_state_bytes(D, dI) // 4, dtype=torch.float32, device=DEV)
    # 12 tokens offered, 8 fit
    b.csa_decode_append(dev(X[:, 32:44]), dev(wkv), None, dev(gate), dev(bslot), m, dev(wkv_h), dev(gate_h),
                        dev(bslot_h), mh, L, seq, state, kv, None, kvh, win)
    torch.cuda.synchronize()
    assert seq.item() == L
    okv, _, ow = oracle.compress(X[:, :L], wkv, None, gate, bslot, m, W=W)
    got = bf16_f64(kv.cpu().numpy().view(np.uint16))
    rows_close(got[0, 8:], okv[0, 8:], "entries of the appended tokens")
    rows_close(bf16_f64(win.cpu().numpy().view(np.uint16))[0, -8:], ow[0, -8:], "window rows of the appended tokens")


def test_append_odd_hidden_and_row_blocks(b):
    # from empty sequences: hidden 192 (six 32-wide steps over four K quarters: uneven quarters), 15 then 18 new
    # token rows (a partial 16-row block, then two blocks), both caches and the window vs the oracle's prefix
    B, Dh, D, dI, m, mh, W, L = 3, 192, 128, 64, 4, 8, 8, 64
    X, wkv, wik, gate, bslot = synth.compress_inputs(140, B, L, Dh, D, dI, m)
    wkv_h, _, gate_h, bslot_h = synth.compress_weights(141, Dh, D, 0, mh, prefix="oh_")
    kv = torch.zeros((B, L // m, D), dtype=torch.int16, device=DEV)
    ik = torch.zeros((B, L // m, dI), dtype=torch.int16, device=DEV)
    kvh = torch.zeros((B, L // mh, D), dtype=torch.int16, device=DEV)
    win = torch.zeros((B, W, D), dtype=torch.int16, device=DEV)
    seq = torch.zeros(B, dtype=torch.int64, device=DEV)
    state = torch.zeros(B * b.lib.csa_append_state_bytes(D, dI) // 4, dtype=torch.float32, device=DEV)
    n = 0
    for T in (5, 6):
        b.csa_decode_append(dev(X[:, n:n + T]), dev(wkv), dev(wik), dev(gate), dev(bslot), m, dev(wkv_h), dev(gate_h),
                            dev(bslot_h), mh, L, seq, state, kv, ik, kvh, win)
        torch.cuda.synchronize()
        n += T
        assert seq.cpu().tolist() == [n] * B
        nc, nh = -(-n // m), -(-n // mh)
        for bb in range(B):
            okv, oik, ow = oracle.compress(X[bb:bb + 1, :n], wkv, wik, gate, bslot, m, W=W)
            okh, _, _ = oracle.compress(X[bb:bb + 1, :n], wkv_h, None, gate_h, bslot_h, mh)
            what = f"after {n} tokens, sequence {bb}"
            rows_close(bf16_f64(kv[bb, :nc].cpu().numpy().view(np.uint16)), okv[0], "kv " + what)
            rows_close(bf16_f64(ik[bb, :nc].cpu().numpy().view(np.uint16)), oik[0], "ik " + what)
            rows_close(bf16_f64(kvh[bb, :nh].cpu().numpy().view(np.uint16)), okh[0], "kv_h " + what)
            rows_close(bf16_f64(win[bb].cpu().numpy().view(np.uint16))[W - min(n, W):], ow[0][W - min(n, W):],
                       "window " + what)

"""Decode-path (one query per sequence) band rescoring on the GPU: the exact tiers beyond the fp64 fast
path, and fp32 rounding ties decided by terms far below the rounding position.

The selection is defined on canonical fp32 scores (each per-head dot product is the exact sum rounded
once), so an entry whose exact dot lies a hair above a rounding midpoint must round up and then tie
with an entry sitting on the upper float, losing or winning by index.  These inputs force the decode
selector's band through its fixed-point window path (products spanning 60 binades), its long
accumulator (spans beyond 2^100) and, for e4m3 keys, the fast path on a rounding midpoint.  The
expected sets are stated by hand and checked on the oracle first.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_kv_compressor_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_sparse_kv_compressor_amd import binding
    return binding


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(DEV)


def run_decode_index(b, q, w, k, L, m, topk, dtype):
    B = q.shape[0]
    idx = torch.empty((B, 1, topk), dtype=torch.int32, device=DEV)
    cnt = torch.empty((B, 1), dtype=torch.int32, device=DEV)
    b.csa_index_topk(dev(q), dev(w), dev(k), dtype, L, m, L - 1, topk, idx, cnt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def tie_inputs(qv, special, seed, dtype, HI=8, dI=128, Nc=256, key_scale=2.0 ** -10):
    """One query whose head 0 carries qv (other heads and weights 0), small random keys, and the given
    key rows (dims 0..3) planted at the given entries."""
    qf = np.zeros((1, 1, HI, dI), np.float32)
    qf[0, 0, 0, :4] = qv
    w = np.zeros((1, 1, HI), np.float32)
    w[0, 0, 0] = 1.0
    g = np.random.default_rng(seed)
    kf = np.zeros((1, Nc, dI), np.float32)
    kf[0, :, :4] = (g.standard_normal((Nc, 4)) * key_scale).astype(np.float32)
    for j, row in special.items():
        kf[0, j, :4] = row
    return synth.encode(qf, dtype), w, synth.encode(kf, dtype)


def check(b, q, w, k, want, m=4, dtype=0):
    L = k.shape[1] * m
    topk = len(want)
    o_idx, _, _, _ = oracle.index_topk(q, w, k, L, m, L - 1, topk, dtype)
    assert o_idx[0, 0].tolist() == want, f"oracle {o_idx[0, 0].tolist()} != {want}"
    g_idx, g_cnt = run_decode_index(b, q, w, k, L, m, topk, dtype)
    assert g_cnt[0, 0] == topk
    assert np.array_equal(g_idx, o_idx), f"gpu {g_idx[0, 0].tolist()} != {want}"


def test_decode_rounding_tie_window_path(b):
    # head dots spanning 60 binades (beyond the exact fp64 fast path): 1 + 2^-24 + 2^-60 rounds up to
    # 1 + 2^-23 and ties with entry 100 (exactly 1 + 2^-23), 1 + 2^-24 - 2^-60 rounds down to 1
    q, w, k = tie_inputs([1.0, 2.0 ** -12, 2.0 ** -30, 1.0],
                         {100: [1.0, 0.0, 0.0, 2.0 ** -23], 50: [1.0, 2.0 ** -12, 2.0 ** -30, 0.0],
                          30: [1.0, 2.0 ** -12, -(2.0 ** -30), 0.0]}, 3, 0)
    check(b, q, w, k, [50, 100])


def test_decode_rounding_tie_wide_path(b):
    # the same structure at 2^100 with a 2^-100 sticky term: 200 binades between the products, which
    # the decode selector's band resolves with the long accumulator
    q, w, k = tie_inputs([2.0 ** 50, 2.0 ** 38, 2.0 ** -50, 2.0 ** 50],
                         {100: [2.0 ** 50, 0.0, 0.0, 2.0 ** 27], 50: [2.0 ** 50, 2.0 ** 38, 2.0 ** -50, 0.0],
                          30: [2.0 ** 50, 2.0 ** 38, -(2.0 ** -50), 0.0]}, 4, 0)
    check(b, q, w, k, [50, 100])


def test_decode_rounding_tie_e4m3(b):
    # e4m3: 128 + 2^-17 + 2^-18 rounds up to 128 + 2^-16 (entry 50) and ties entry 100 exactly;
    # 128 + 2^-17 - 2^-18 (entry 20) rounds down, and the midpoint 128 + 2^-17 (entry 30) rounds to even
    q, w, k = tie_inputs([16.0, 2.0 ** -8, 2.0 ** -9, 2.0 ** -7],
                         {100: [8.0, 0.0, 0.0, 2.0 ** -9], 50: [8.0, 2.0 ** -9, 2.0 ** -9, 0.0],
                          20: [8.0, 2.0 ** -9, -(2.0 ** -9), 0.0], 30: [8.0, 2.0 ** -9, 0.0, 0.0]}, 5, 1,
                         key_scale=2.0 ** -3)
    check(b, q, w, k, [50, 100], dtype=1)


@pytest.mark.parametrize("dtype", [0, 1])
def test_decode_rounding_tie_inside_large_row(b, dtype):
    # the same tie planted among 40000 Gaussian entries of the 1M-decode key distribution, scaled so
    # that the planted scores lead (the band then holds exactly the planted entries)
    Nc, dI, HI = 40000, 128, 8
    if dtype == 0:
        qv = [1.0, 2.0 ** -12, 2.0 ** -30, 1.0]
        special = {31000: [1.0, 0.0, 0.0, 2.0 ** -23], 17: [1.0, 2.0 ** -12, 2.0 ** -30, 0.0],
                   9: [1.0, 2.0 ** -12, -(2.0 ** -30), 0.0]}
        want = [17, 31000]
    else:
        qv = [16.0, 2.0 ** -8, 2.0 ** -9, 2.0 ** -7]
        special = {31000: [8.0, 0.0, 0.0, 2.0 ** -9], 17: [8.0, 2.0 ** -9, 2.0 ** -9, 0.0],
                   9: [8.0, 2.0 ** -9, -(2.0 ** -9), 0.0], 12: [8.0, 2.0 ** -9, 0.0, 0.0]}
        want = [17, 31000]
    q, w, k = tie_inputs(qv, special, 6, dtype, HI=HI, dI=dI, Nc=Nc,
                         key_scale=dI ** -0.5 if dtype == 0 else 0.25)
    check(b, q, w, k, want, dtype=dtype)

"""The certified error bound behind the bit-exact top-k, checked on the GPU through score_out.

The selection is exact only if every approximate MFMA score S~ lies within the bound the kernels certify
for it.  The model (per entry s, heads h, A_h = sum_i |q_hi k_si|, d_h the exact per-head dot):
    E_h = 2^-17 A_h,   Delta_s = sum_h |w_h| (2^-19 (|d_h| + 2 E_h) + E_h) (1 + 2^-10) + 2^-24 |S| + 2^-126
(2^-17 = 128 fp32 unit roundoffs: the worst-order accumulation error of a dot over at most 128 exact
products; 2^-19 covers the head reduction and the final rounding of each exact dot).  score_out returns S~ of every selected entry; on adversarial inputs
(Gaussian, all-positive, cancelling sums, elements scaled by 2^-12..2^12, tiny magnitudes) the measured
|S~ - S| must stay at least 8 times inside Delta_s, for the decode contraction (16x16x32 bf16 MFMA, with
e4m3 keys widened exactly) and for the many-query one (32x32x16 bf16 MFMA).
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_kv_compressor_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
MARGIN = 8.0


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_sparse_kv_compressor_amd import binding
    return binding


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(DEV)


def values(bits, dtype):
    return oracle.bf16_value(bits) if dtype == 0 else oracle.e4m3_value(bits)


def make_inputs(kind, B, Tq, HI, dI, Nc, dtype, seed):
    g = np.random.default_rng(seed)
    s = dI ** -0.5
    q = g.standard_normal((B, Tq, HI, dI)) * s
    k = g.standard_normal((B, Nc, dI)) * s
    if kind == "positive":
        q, k = np.abs(q), np.abs(k)
    elif kind == "cancelling":
        # k_s = c_s * (-1)^i * |q_0| + small noise: large sum |p|, small dot products
        sign = np.where(np.arange(dI) % 2 == 0, 1.0, -1.0)
        base = np.abs(q[:, :1, :1, :])                                   # [B][1][1][dI]
        c = g.uniform(0.5, 2.0, (B, Nc, 1))
        k = c * sign * base[:, 0] + 0.01 * s * g.standard_normal((B, Nc, dI))
        q = np.broadcast_to(base, q.shape) * (1 + 0.01 * g.standard_normal(q.shape))
    elif kind == "scaled":
        q = q * 2.0 ** g.integers(-12, 13, q.shape)
        k = k * 2.0 ** g.integers(-12, 13, k.shape)
    elif kind == "tiny":
        q, k = q * 2.0 ** -55, k * 2.0 ** -55
    if dtype == 1:                      # e4m3 range: keep magnitudes representable
        q = np.clip(q * 8, -440, 440)
        k = np.clip(k * 8, -440, 440)
    w = np.abs(g.standard_normal((B, Tq, HI))).astype(np.float32) * np.float32(HI ** -0.5)
    return synth.encode(q.astype(np.float32), dtype), w, synth.encode(k.astype(np.float32), dtype)


def check_margin(b, q, w, k, L, m, pos0, topk, dtype):
    B, Tq, HI, dI = q.shape
    Nc = k.shape[1]
    idx = torch.empty((B, Tq, topk), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, Tq, topk), dtype=torch.float32, device=DEV)
    b.csa_index_topk(dev(q), dev(w), dev(k), dtype, L, m, pos0, topk, idx, score_out=sc)
    torch.cuda.synchronize()
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    S, _ = oracle.index_scores(q, w, k, L, m, pos0, dtype)
    oi, _ = oracle.topk(S, _nv(L, m, pos0, Tq, B), topk)
    assert np.array_equal(gi, oi)
    qv, kv = values(q, dtype), values(k, dtype)
    worst = np.inf
    for bb in range(B):
        for t in range(Tq):
            sel = gi[bb, t]
            sel = sel[sel >= 0]
            ks = kv[bb, sel]                                                # [n][dI]
            A = np.abs(qv[bb, t])[None, :, :] * np.abs(ks)[:, None, :]       # [n][HI][dI]
            A = A.sum(-1)
            d = (qv[bb, t][None, :, :] * ks[:, None, :]).sum(-1)            # fp64 estimate of the exact dot
            E = 2.0 ** -17 * A
            wa = np.abs(w[bb, t].astype(np.float64))[None, :]
            Sx = S[bb, t, sel].astype(np.float64)
            delta = (wa * (2.0 ** -19 * (np.abs(d) + 2 * E) + E)).sum(-1) * (1 + 2.0 ** -10) \
                + 2.0 ** -24 * np.abs(Sx) + 2.0 ** -126
            err = np.abs(gs[bb, t, :sel.size].astype(np.float64) - Sx)
            assert np.isfinite(gs[bb, t, :sel.size]).all()
            with np.errstate(divide="ignore"):
                ratio = np.where(err > 0, delta / err, np.inf)
            worst = min(worst, ratio.min())
    assert worst >= MARGIN, f"measured error only {worst:.3g}x inside the certified bound"
    return worst


def _nv(L, m, pos0, Tq, B):
    Nc = -(-L // m)
    p = pos0 + np.arange(Tq)
    nv = np.where(p >= L - 1, Nc, np.minimum((p + 1) // m, Nc))
    return np.broadcast_to(nv, (B, Tq)).astype(np.int32)


KINDS = ["gaussian", "positive", "cancelling", "scaled", "tiny"]


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("kind", KINDS)
def test_decode_scores_within_certified_bound(b, kind, dtype):
    if dtype == 1 and kind == "tiny":
        pytest.skip("e4m3 has no magnitudes below 2^-9")
    B, HI, dI, m, Nc, topk = 2, 8, 128, 4, 6000, 512
    q, w, k = make_inputs(kind, B, 1, HI, dI, Nc, dtype, 1 + KINDS.index(kind))
    L = Nc * m
    worst = check_margin(b, q, w, k, L, m, L - 1, topk, dtype)
    print(f"decode {kind} dtype {dtype}: error at least {worst:.3g}x inside the bound")


@pytest.mark.parametrize("kind", KINDS)
def test_many_query_scores_within_certified_bound(b, kind):
    B, Tq, HI, dI, m, Nc, topk = 1, 64, 8, 128, 4, 2048, 128
    q, w, k = make_inputs(kind, B, Tq, HI, dI, Nc, 0, 11 + KINDS.index(kind))
    L = Nc * m
    worst = check_margin(b, q, w, k, L, m, L - Tq, topk, 0)
    print(f"many-query {kind}: error at least {worst:.3g}x inside the bound")


def test_score_out_is_nan_where_nothing_is_scored(b):
    # fewer visible entries than k: every visible entry is selected without scoring
    q, w, k = make_inputs("gaussian", 1, 1, 8, 128, 50, 0, 3)
    idx = torch.empty((1, 1, 64), dtype=torch.int32, device=DEV)
    sc = torch.zeros((1, 1, 64), dtype=torch.float32, device=DEV)
    b.csa_index_topk(dev(q), dev(w), dev(k), 0, 200, 4, 199, 64, idx, score_out=sc)
    torch.cuda.synchronize()
    assert (idx.cpu().numpy()[0, 0] == np.r_[np.arange(50), -np.ones(14)]).all()
    assert np.isnan(sc.cpu().numpy()).all()

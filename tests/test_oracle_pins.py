"""Pins of the CPU oracle against facts it does not compute itself.

Each test ties one oracle function to something other than its own formula:
closed forms, textbook routines (numpy / scipy / torch on the CPU), exact
rational brute force (fractions.Fraction), invariants, special cases, and the
entry counts printed on the pages (tests/golden/entry_counts.json).

The choice of the compressor's gate form and of the indexer's score form are
readings of pages that print no formula ("parity unpinned" for that choice);
what is pinned here is that the oracle computes those readings correctly.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from compressed_sparse_kv_compressor_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# exact rational helpers (independent of the oracle's C code)
# ---------------------------------------------------------------------------

def frac_bf16(bits):
    u = np.array([int(bits)], np.uint32) << 16
    return Fraction(float(u.view(np.float32)[0]))


def frac_e4m3(bits):
    b = int(bits)
    s, e, f = b >> 7, (b >> 3) & 15, b & 7
    v = Fraction(f, 512) if e == 0 else Fraction(8 + f, 8) * Fraction(2) ** (e - 7)
    return -v if s else v


def frac_to_f32(x: Fraction) -> float:
    """Round a rational to the nearest fp32 (ties to even), as a Python float."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 23)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


def brute_dot(a, b, dtype):
    fv = frac_bf16 if dtype == oracle.BF16 else frac_e4m3
    return frac_to_f32(sum((fv(x) * fv(y) for x, y in zip(a, b)), Fraction(0)))


def brute_score(q, w, k, dtype):
    S = Fraction(0)
    for h in range(q.shape[0]):
        d = brute_dot(q[h], k, dtype)
        r = d if d > 0 else 0.0
        S = Fraction(frac_to_f32(Fraction(float(np.float32(w[h]))) * Fraction(r) + S))
    return float(S)


def rand_bf16(g, n, scale=1.0):
    return synth.to_bf16_bits((g.standard_normal(n) * scale).astype(np.float32))


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.bf16_value(bits)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.all(np.isnan(got[np.isnan(want)]))


def test_e4m3_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m], want[m])
    # OCP e4m3fn landmarks: largest normal 448, smallest subnormal 2^-9, NaN at S.1111.111
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_bf16_round_matches_torch_on_fp32_values():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 3.0e38, 1e-40, -1e-41]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    assert oracle.bf16_round([1 + 2 ** -8])[0] == 0x3F80
    assert oracle.bf16_round([1 + 3 * 2 ** -8])[0] == 0x3F82


def test_e4m3_round_matches_torch_and_saturates():
    g = np.random.default_rng(2)
    x = (g.standard_normal(20000) * 10.0 ** g.uniform(-4, 2.3, 20000)).astype(np.float32)
    x = x[np.abs(x) < 440]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_round(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert oracle.e4m3_round([1e6])[0] == 0x7E and oracle.e4m3_round([-500.0])[0] == 0xFE
    assert oracle.e4m3_round([2.0 ** -10])[0] == 0x00  # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_round([3 * 2.0 ** -10])[0] == 0x02  # tie between 2^-9 and 2^-8 -> even


# ---------------------------------------------------------------------------
# exact dot product and canonical score (A2)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 7, 64, 128])
def test_exact_dot_bf16_random_vs_fraction(n):
    g = np.random.default_rng(n)
    for trial in range(40):
        a = rand_bf16(g, n, 10.0 ** g.uniform(-3, 3))
        b = rand_bf16(g, n, 10.0 ** g.uniform(-3, 3))
        assert oracle.exact_dot_f32(a, b) == np.float32(brute_dot(a, b, oracle.BF16))


def test_exact_dot_edge_cases_vs_fraction():
    def bf(vals):
        return synth.to_bf16_bits(np.array(vals, np.float32))
    cases = [
        (bf([1e30, 1e-30, -1e30]), bf([1e8, 1e-8, 1e8])),              # huge span, cancellation
        (bf([1.0, -1.0, 2.0 ** -120]), bf([3.0, 3.0, 2.0 ** -10])),      # result far below the cancelled terms
        (np.array([0x0001, 0x0002, 0x8003], np.uint16), np.array([0x3f80, 0x0001, 0x4000], np.uint16)),  # subnormals
        (bf([0.0, -0.0]), bf([1.0, 2.0])),                               # exact zero
        (bf([1.0, 2.0 ** -24]), bf([1.0, 1.0])),                         # exact fp32 tie 1 + 2^-24 -> 1
        (bf([1.0, 2.0 ** -24, 2.0 ** -60]), bf([1.0, 1.0, 1.0])),        # just above the tie -> round up
        (bf([1.0, 3 * 2.0 ** -24]), bf([1.0, 1.0])),                     # tie to even upward
        (bf([3.0e38, 3.0e38]), bf([2.0, 2.0])),                          # overflow -> inf
    ]
    for a, b in cases:
        got = oracle.exact_dot_f32(a, b)
        want = brute_dot(a, b, oracle.BF16)
        assert (got == want) or (math.isinf(want) and got == want), (a, b, got, want)
    assert oracle.exact_dot_f32(bf([1.0, 2.0 ** -24]), bf([1.0, 1.0])) == np.float32(1.0)
    assert oracle.exact_dot_f32(bf([1.0, 2.0 ** -24, 2.0 ** -60]), bf([1.0, 1.0, 1.0])) == np.float32(1 + 2 ** -23)


def test_exact_dot_e4m3_vs_fraction_and_exhaustive_pairs():
    g = np.random.default_rng(3)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    # every code times every code (n = 1)
    for a in codes[::5]:
        for b in codes[::3]:
            got = oracle.exact_dot_f32(np.array([a], np.uint8), np.array([b], np.uint8), oracle.E4M3)
            assert got == np.float32(brute_dot([a], [b], oracle.E4M3))
    for n in (16, 128):
        for _ in range(30):
            a = g.choice(codes, n)
            b = g.choice(codes, n)
            assert oracle.exact_dot_f32(a, b, oracle.E4M3) == np.float32(brute_dot(a, b, oracle.E4M3))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.E4M3])
def test_canonical_score_vs_fraction(dtype):
    g = np.random.default_rng(10 + dtype)
    HI, dI = 8, 32
    for _ in range(30):
        qf = (g.standard_normal((HI, dI)) / np.sqrt(dI)).astype(np.float32)
        kf = (g.standard_normal(dI) / np.sqrt(dI)).astype(np.float32)
        q = synth.encode(qf, dtype)
        k = synth.encode(kf, dtype)
        w = np.abs(g.standard_normal(HI)).astype(np.float32)
        w[0] = -w[0]  # a negative weight exercises the general fma chain
        assert oracle.index_score(q, w, k, dtype) == np.float32(brute_score(q, w, k, dtype))


def test_score_all_heads_negative_is_plus_zero():
    q = synth.to_bf16_bits(np.full((4, 8), 0.5, np.float32))
    k = synth.to_bf16_bits(np.full(8, -0.25, np.float32))
    s = oracle.index_score(q, np.ones(4, np.float32), k)
    assert s == 0.0 and not np.signbit(s)


# ---------------------------------------------------------------------------
# entry counts and visibility
# ---------------------------------------------------------------------------

def test_entry_counts_printed_on_pages():
    with open(os.path.join(GOLDEN, "entry_counts.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        L, m, n = case["L"], case["m"], case["entries"]
        assert oracle.n_visible(L - 1, L, m) == n          # all entries visible at the last token
        assert (L + m - 1) // m == n


@pytest.mark.parametrize("m", [1, 2, 4, 5, 128])
def test_visibility_closed_form(m):
    for L in range(1, 3 * m + 2):
        Nc = -(-L // m)
        for p in range(0, L + 2):
            want = Nc if p >= L - 1 else (p + 1) // m
            assert oracle.n_visible(p, L, m) == want, (L, m, p)


def test_compress_entry_count_is_ceil_L_over_m():
    g = np.random.default_rng(4)
    Dh, D = 64, 16
    for m in (1, 3, 4):
        for L in range(1, 3 * m + 2):
            X = rand_bf16(g, L * Dh).reshape(1, L, Dh)
            W = rand_bf16(g, D * Dh, 0.1).reshape(D, Dh)
            kv, _, _ = oracle.compress(X, W, None, np.zeros(Dh, np.float32), None, m)
            assert kv.shape == (1, -(-L // m), D)


# ---------------------------------------------------------------------------
# compressor (A1)
# ---------------------------------------------------------------------------

def _bf16_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup_compress(seed, B, L, Dh, D, dI, m):
    X, wkv, wik, gate, bslot = synth.compress_inputs(seed, B, L, Dh, D, dI, m)
    Y = _bf16_f64(X) @ _bf16_f64(wkv).T            # per-token projections [B][L][D]
    Yi = _bf16_f64(X) @ _bf16_f64(wik).T if wik is not None else None
    return X, wkv, wik, gate, bslot, Y, Yi


def test_zero_gate_gives_block_mean_including_tail():
    B, L, Dh, D, dI, m = 2, 23, 64, 32, 16, 4     # L % m = 3: a partial tail block
    X, wkv, wik, gate, bslot, Y, Yi = _setup_compress(5, B, L, Dh, D, dI, m)
    kv, ik, _ = oracle.compress(X, wkv, wik, np.zeros(Dh, np.float32), None, m)
    for j in range(-(-L // m)):
        t0, t1 = j * m, min((j + 1) * m, L)
        np.testing.assert_allclose(kv[:, j], Y[:, t0:t1].mean(1), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ik[:, j], Yi[:, t0:t1].mean(1), rtol=1e-12, atol=1e-14)


def test_ratio_one_is_identity():
    B, L, Dh, D = 1, 9, 64, 32
    X, wkv, _, gate, _, Y, _ = _setup_compress(6, B, L, Dh, D, 0, 1)
    kv, _, _ = oracle.compress(X, wkv, None, gate, np.zeros(1, np.float32), 1)
    np.testing.assert_allclose(kv, Y, rtol=1e-12, atol=1e-14)


def test_two_token_gate_is_logistic():
    B, L, Dh, D, m = 1, 10, 64, 16, 2
    X, wkv, _, gate, _, Y, _ = _setup_compress(7, B, L, Dh, D, 0, m)
    bslot = np.array([0.3, -0.2], np.float32)
    kv, _, _ = oracle.compress(X, wkv, None, gate, bslot, m)
    z = _bf16_f64(X)[0] @ gate.astype(np.float64) + np.tile(bslot.astype(np.float64), L // 2)
    for j in range(L // 2):
        a0 = scipy.special.expit(z[2 * j] - z[2 * j + 1])
        np.testing.assert_allclose(kv[0, j], a0 * Y[0, 2 * j] + (1 - a0) * Y[0, 2 * j + 1], rtol=1e-10, atol=1e-13)


def test_dominant_slot_bias_selects_one_token():
    B, L, Dh, D, m = 1, 14, 64, 16, 4
    X, wkv, _, _, _, Y, _ = _setup_compress(8, B, L, Dh, D, 0, m)
    bslot = np.array([0, 0, 800.0, 0], np.float32)
    kv, _, _ = oracle.compress(X, wkv, None, np.zeros(Dh, np.float32), bslot, m)
    for j in range(L // m):
        np.testing.assert_allclose(kv[0, j], Y[0, j * m + 2], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(kv[0, L // m], Y[0, 12:14].mean(0), rtol=1e-12, atol=1e-14)  # tail has no slot 2


def test_compress_convex_and_permutation_invariant():
    B, L, Dh, D, m = 2, 32, 64, 16, 4
    X, wkv, _, gate, _, Y, _ = _setup_compress(9, B, L, Dh, D, 0, m)
    g = np.random.default_rng(9)
    bslot = g.standard_normal(m).astype(np.float32)
    kv, _, _ = oracle.compress(X, wkv, None, gate * 8, bslot, m)
    Yb = Y.reshape(B, L // m, m, D)
    assert np.all(kv <= Yb.max(2) + 1e-12) and np.all(kv >= Yb.min(2) - 1e-12)
    perm = g.permutation(m)
    Xp = X.reshape(B, L // m, m, Dh)[:, :, perm].reshape(B, L, Dh)
    kv2, _, _ = oracle.compress(Xp, wkv, None, gate * 8, bslot[perm], m)
    np.testing.assert_allclose(kv2, kv, rtol=1e-12, atol=1e-14)


def test_window_rows_are_raw_projections():
    B, L, Dh, D, m, W = 2, 10, 64, 16, 4, 6
    X, wkv, _, gate, _, Y, _ = _setup_compress(11, B, L, Dh, D, 0, m)
    _, _, win = oracle.compress(X, wkv, None, gate, None, m, W=W)
    np.testing.assert_allclose(win, Y[:, L - W:], rtol=1e-12, atol=1e-14)
    _, _, win2 = oracle.compress(X[:, :3], wkv, None, gate, None, m, W=5)   # L < W: zero rows first
    np.testing.assert_allclose(win2[:, 2:], Y[:, :3], rtol=1e-12, atol=1e-14)
    assert np.all(win2[:, :2] == 0)


def test_entry_range_matches_full_run():
    B, L, Dh, D, dI, m = 1, 40, 64, 16, 8, 4
    X, wkv, wik, gate, _, _, _ = _setup_compress(12, B, L, Dh, D, dI, m)
    kv, ik, _ = oracle.compress(X, wkv, wik, gate, None, m)
    kv2, ik2, _ = oracle.compress(X, wkv, wik, gate, None, m, j0=3, j1=7)
    assert np.array_equal(kv[:, 3:7], kv2) and np.array_equal(ik[:, 3:7], ik2)


# ---------------------------------------------------------------------------
# top-k (A3)
# ---------------------------------------------------------------------------

def test_topk_vs_sorted_brute_force_with_ties():
    g = np.random.default_rng(20)
    rows, Nc = 30, 200
    S = g.integers(0, 12, (rows, Nc)).astype(np.float32) / 4   # many exact ties
    S[0, :5] = -0.0
    S[0, 5:10] = 0.0
    nv = g.integers(0, Nc + 1, rows).astype(np.int32)
    for k in (1, 7, 50, 200, 300):
        idx, cnt = oracle.topk(S, nv, k)
        for r in range(rows):
            order = sorted(range(nv[r]), key=lambda j: (-float(S[r, j]), j))
            want = sorted(order[:k])
            c = min(k, nv[r])
            assert cnt[r] == c
            assert list(idx[r, :c]) == want and np.all(idx[r, c:] == -1)


def test_topk_covers_all_visible_and_nests():
    g = np.random.default_rng(21)
    S = g.standard_normal((5, 64)).astype(np.float32)
    nv = np.array([64, 10, 0, 1, 63], np.int32)
    idx, cnt = oracle.topk(S, nv, 64)
    for r in range(5):
        assert list(idx[r, :nv[r]]) == list(range(nv[r]))
    prev = None
    for k in range(1, 40):
        idx, _ = oracle.topk(S, nv, k)
        cur = [set(row[row >= 0]) for row in idx]
        if prev is not None:
            assert all(a <= b for a, b in zip(prev, cur))
        prev = cur


def test_duplicated_keys_lower_index_wins():
    g = np.random.default_rng(22)
    B, Tq, HI, dI, Nc = 1, 1, 4, 64, 50
    q, w, k, _ = synth.indexer_inputs(22, B, Tq, HI, dI, Nc)
    S, nv = oracle.index_scores(q, w, k, L=4 * Nc, m=4, pos0=4 * Nc - 1)
    order = np.argsort(-S[0, 0], kind="stable")
    # copy the best key to a higher index and an even lower index than the 3rd best
    best = order[0]
    lo, hi = min(order[1], order[2]) - 1, Nc - 1
    k2 = k.copy()
    k2[0, hi] = k[0, best]
    if lo >= 0 and lo != best:
        k2[0, lo] = k[0, best]
    S2, _ = oracle.index_scores(q, w, k2, L=4 * Nc, m=4, pos0=4 * Nc - 1)
    dups = [j for j in range(Nc) if np.array_equal(k2[0, j], k[0, best])]
    assert len(set(S2[0, 0, dups].tolist())) == 1          # bit-identical scores
    idx, _ = oracle.topk(S2, np.array([[Nc]]), 1)
    assert idx[0, 0, 0] == min(dups)


def test_planted_keys_are_selected():
    B, Tq, HI, dI, Nc, k = 2, 1, 8, 128, 2048, 32
    q, w, kk, planted = synth.indexer_inputs(23, B, Tq, HI, dI, Nc, planted=16)
    idx, cnt, S, _ = oracle.index_topk(q, w, kk, L=4 * Nc, m=4, pos0=4 * Nc - 1, k=k)
    for b in range(B):
        assert set(planted[b]) <= set(idx[b, 0].tolist())
        others = np.setdiff1d(np.arange(Nc), planted[b])
        assert S[b, 0, planted[b]].min() > S[b, 0, others].max()


def test_index_scores_prefix_visibility():
    B, Tq, HI, dI, L, m = 1, 6, 4, 64, 37, 4
    Nc = -(-L // m)
    q, w, k, _ = synth.indexer_inputs(24, B, Tq, HI, dI, Nc)
    pos0 = L - Tq
    S, nv = oracle.index_scores(q, w, k, L, m, pos0)
    for t in range(Tq):
        p = pos0 + t
        assert nv[0, t] == (Nc if p >= L - 1 else (p + 1) // m)
        assert np.all(np.isnan(S[0, t, nv[0, t]:])) and not np.any(np.isnan(S[0, t, :nv[0, t]]))
        for j in range(nv[0, t]):
            assert S[0, t, j] == oracle.index_score(q[0, t], w[0, t], k[0, j])


# ---------------------------------------------------------------------------
# attention (A4, A5)
# ---------------------------------------------------------------------------

def _textbook_mqa(qf, Kf, scale):
    """softmax(scale * q K^T) K in fp64, per head; and logsumexp."""
    logits = scale * qf @ Kf.T
    p = scipy.special.softmax(logits, axis=-1)
    return p @ Kf, scipy.special.logsumexp(logits, axis=-1)


def test_hca_ratio_one_is_textbook_mqa_numpy_and_torch():
    B, Tq, H, D, L = 2, 3, 16, 64, 40
    q, rows = synth.attn_inputs(30, B, Tq, H, D, L, "hca_")
    scale = 16 / np.sqrt(D)                                   # sharp softmax
    out, lse = oracle.dense_attn(q, rows, L=L, mh=1, pos0=L - Tq, scale=scale)
    qf, Kf = _bf16_f64(q), _bf16_f64(rows)
    for b in range(B):
        for t in range(Tq):
            n = L - Tq + t + 1                                 # causal: tokens 0..p
            o, l = _textbook_mqa(qf[b, t], Kf[b, :n], scale)
            np.testing.assert_allclose(out[b, t], o, rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(lse[b, t], l, rtol=1e-12)
            Kt = torch.from_numpy(Kf[b, :n])[None, None].expand(1, H, n, D)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qf[b, t])[None, :, None, :], Kt, Kt, scale=scale)
            np.testing.assert_allclose(out[b, t], ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-13)


def test_single_key_and_zero_query():
    B, Tq, H, D = 1, 1, 16, 32
    q, rows = synth.attn_inputs(31, B, Tq, H, D, 5, "s_")
    out, lse = oracle.dense_attn(q, rows[:, :1], L=4, mh=4, pos0=3, scale=0.3)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(_bf16_f64(rows[0, 0]), (H, D)), rtol=1e-15)
    qz = np.zeros_like(q)
    out, lse = oracle.dense_attn(qz, rows, L=5, mh=1, pos0=4, scale=0.3)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(_bf16_f64(rows[0]).mean(0), (H, D)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.log(5.0), rtol=1e-14)


def test_full_selection_without_window_equals_dense():
    B, Tq, H, D, Nc, m = 2, 1, 16, 64, 33, 4
    L = Nc * m - 2
    q, rows = synth.attn_inputs(32, B, Tq, H, D, Nc, "p7_")
    idx = np.tile(np.arange(Nc, dtype=np.int32), (B, Tq, 1))
    out_s, lse_s = oracle.sparse_attn(q, rows, idx, None, raw0=0, pos0=L - 1, W=0, scale=0.2)
    out_d, lse_d = oracle.dense_attn(q, rows, L=L, mh=m, pos0=L - 1, scale=0.2)
    np.testing.assert_allclose(out_s, out_d, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse_s, lse_d, rtol=1e-13)


def test_window_only_is_sliding_window_attention():
    B, Tq, H, D, Lr, W = 1, 5, 16, 32, 20, 6
    q, raw = synth.attn_inputs(33, B, Tq, H, D, Lr, "w_")
    idx = -np.ones((B, Tq, 3), np.int32)
    kv = np.zeros((B, 2, D), np.uint16)
    out, lse = oracle.sparse_attn(q, kv, idx, raw, raw0=0, pos0=Lr - Tq, W=W, scale=0.5)
    qf, Rf = _bf16_f64(q), _bf16_f64(raw)
    Q = torch.from_numpy(qf[0]).permute(1, 0, 2)               # [H][Tq][D]
    K = torch.from_numpy(Rf[0])[None].expand(H, Lr, D)
    pos = torch.arange(Lr - Tq, Lr)[:, None]
    cols = torch.arange(Lr)[None]
    mask = (cols <= pos) & (cols > pos - W)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, K, attn_mask=mask, scale=0.5)
    np.testing.assert_allclose(out[0], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-13)
    # window clipped at position 0
    out2, _ = oracle.sparse_attn(q[:, :1], kv, idx[:, :1], raw, raw0=0, pos0=2, W=W, scale=0.5)
    o, _ = _textbook_mqa(qf[0, 0], Rf[0, :3], 0.5)
    np.testing.assert_allclose(out2[0, 0], o, rtol=1e-10, atol=1e-13)


def test_sparse_union_is_one_softmax_and_convex():
    B, Tq, H, D, Nc, W = 1, 1, 16, 32, 40, 4
    q, rows = synth.attn_inputs(34, B, Tq, H, D, Nc, "u_")
    _, raw = synth.attn_inputs(35, B, Tq, H, D, 8, "r_")
    idx = np.array([[[3, 9, 17, 30, -1, -1]]], np.int32)
    out, lse = oracle.sparse_attn(q, rows, idx, raw, raw0=0, pos0=7, W=W, scale=2.0)
    Kf = np.concatenate([_bf16_f64(rows[0, [3, 9, 17, 30]]), _bf16_f64(raw[0, 4:8])])
    o, l = _textbook_mqa(_bf16_f64(q[0, 0]), Kf, 2.0)
    np.testing.assert_allclose(out[0, 0], o, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], l, rtol=1e-12)
    assert np.all(out[0, 0] <= Kf.max(0) + 1e-12) and np.all(out[0, 0] >= Kf.min(0) - 1e-12)


def test_empty_key_set():
    q, rows = synth.attn_inputs(36, 1, 1, 16, 32, 4, "e_")
    out, lse = oracle.dense_attn(q, rows, L=8, mh=4, pos0=2, scale=1.0)   # no entry complete yet
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# attention sink: a per-head logit in the softmax denominator with no value row (P1 section 1.1)

def test_sink_zero_equals_an_extra_all_zero_row():
    # a row of zeros has logit scale * (q . 0) = 0 and contributes no value: exactly a sink of 0
    B, Tq, H, D, Nc = 1, 2, 16, 64, 30
    q, rows = synth.attn_inputs(37, B, Tq, H, D, Nc, "sk_")
    _, raw = synth.attn_inputs(38, B, Tq, H, D, 6, "skr_")
    kvz = np.concatenate([rows, np.zeros((B, 1, D), np.uint16)], axis=1)
    idx = np.array([[[2, 7, 11, 25, -1], [0, 5, 6, 29, 13]]], np.int32)
    idx_z = np.concatenate([idx, np.full((B, Tq, 1), Nc, np.int32)], axis=-1)
    out_s, lse_s = oracle.sparse_attn(q, rows, idx, raw, raw0=0, pos0=4, W=3, scale=0.7, sink=np.zeros(H))
    out_z, lse_z = oracle.sparse_attn(q, kvz, idx_z, raw, raw0=0, pos0=4, W=3, scale=0.7)
    np.testing.assert_allclose(out_s, out_z, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse_s, lse_z, rtol=1e-13)


def test_sink_limits_and_textbook_softmax():
    B, Tq, H, D, L = 1, 1, 16, 32, 12
    q, rows = synth.attn_inputs(39, B, Tq, H, D, L, "sl_")
    out0, lse0 = oracle.dense_attn(q, rows, L=L, mh=1, pos0=L - 1, scale=0.4)
    out_m, lse_m = oracle.dense_attn(q, rows, L=L, mh=1, pos0=L - 1, scale=0.4, sink=np.full(H, -np.inf))
    assert np.array_equal(out_m, out0) and np.array_equal(lse_m, lse0)          # -inf: no sink
    big = np.full(H, 1.0e4)
    out_b, lse_b = oracle.dense_attn(q, rows, L=L, mh=1, pos0=L - 1, scale=0.4, sink=big)
    assert np.all(out_b == 0) and np.array_equal(lse_b[0, 0], big)               # all attention on the sink
    out_e, lse_e = oracle.dense_attn(q, rows, L=L, mh=4, pos0=2, scale=0.4, sink=np.arange(H) * 0.5)
    assert np.all(out_e == 0) and np.array_equal(lse_e[0, 0], np.arange(H) * 0.5)   # no row: lse = sink
    # per-head sinks against a library softmax over the logits and the sink
    sk = np.linspace(-3.0, 3.0, H)
    out_s, lse_s = oracle.dense_attn(q, rows, L=L, mh=1, pos0=L - 1, scale=0.4, sink=sk)
    qf, Kf = _bf16_f64(q[0, 0]), _bf16_f64(rows[0])
    logits = np.concatenate([0.4 * qf @ Kf.T, sk[:, None]], axis=1)
    p = scipy.special.softmax(logits, axis=1)
    np.testing.assert_allclose(out_s[0, 0], p[:, :-1] @ Kf, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lse_s[0, 0], scipy.special.logsumexp(logits, axis=1), rtol=1e-13)


# ---------------------------------------------------------------------------
# C11: partial rotary position embedding
# ---------------------------------------------------------------------------

def _rope_rows(seed, n, D):
    return synth.to_bf16_bits(synth.normal_f32(seed, "rope_x", (n, D)))


def test_rope_matches_library_interleaved_rotation():
    """The rotated part equals transformers' DeepSeek-V3 interleaved rotary routine (which returns the pair
    halves de-interleaved) with cos/sin from its Llama rotary-embedding module, theta = 10000, rd = 64."""
    from transformers import LlamaConfig
    from transformers.models.deepseek_v3.modeling_deepseek_v3 import apply_rotary_pos_emb_interleave
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
    D, rd, n = 128, 64, 40
    x = _rope_rows(1, n, D)
    pos = np.arange(n, dtype=np.int64) * 7 + 3                      # positions 3 .. 276
    got = oracle.rope(x, pos, rd=rd, theta=10000.0)
    cfg = LlamaConfig(hidden_size=rd, num_attention_heads=1, head_dim=rd, rope_theta=10000.0)
    emb = LlamaRotaryEmbedding(config=cfg)
    xt = torch.from_numpy(oracle.bf16_value(x)[:, D - rd:]).view(1, 1, n, rd)   # (batch, heads, seq, dim)
    cos, sin = emb(xt.float(), torch.from_numpy(pos).view(1, n))
    ref, _ = apply_rotary_pos_emb_interleave(xt, xt, cos.double(), sin.double())
    ref = ref.view(n, rd).numpy()
    mine = np.concatenate([got[:, D - rd::2], got[:, D - rd + 1::2]], axis=1)
    assert np.abs(mine - ref).max() < 1e-4                          # the library's cos/sin are fp32
    assert np.array_equal(got[:, :D - rd], oracle.bf16_value(x)[:, :D - rd])


def test_rope_rotation_invariants():
    D, rd = 512, 64
    x = _rope_rows(2, 6, D)
    xv = oracle.bf16_value(x)
    assert np.array_equal(oracle.rope(x, np.zeros(6, np.int64)), xv)              # position 0: identity
    p = np.array([0, 1, 1000, 65_537, 262_143, 1_048_575], np.int64)
    y = oracle.rope(x, p, rd=rd)
    yi = oracle.rope(x, p, rd=rd, inverse=True)
    assert np.array_equal(y[:, :D - rd], xv[:, :D - rd])
    # each pair keeps its length
    pr = lambda a: a[:, D - rd:].reshape(6, rd // 2, 2)
    assert np.allclose(np.hypot(*np.moveaxis(pr(y), -1, 0)), np.hypot(*np.moveaxis(pr(xv), -1, 0)), atol=1e-12)
    # the inverse is the rotation by the opposite angle: rope(x, p)_j . rope_inv(x, p)_j = |x_j|^2 cos(2 a_j) and
    # the forward rotation of a vector by p then by -p is the vector (checked as a relative-position identity)
    q, k = xv[0], xv[1]
    qb, kb = x[0:1], x[1:2]
    for i, j in [(5, 2), (1000, 999), (262_143, 100)]:
        lhs = oracle.rope(qb, [i])[0, D - rd:] @ oracle.rope(kb, [j])[0, D - rd:]
        rhs = oracle.rope(qb, [i - j])[0, D - rd:] @ k[D - rd:]
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
        inv = oracle.rope(qb, [i], inverse=True)[0, D - rd:] @ oracle.rope(kb, [j], inverse=True)[0, D - rd:]
        assert abs(inv - oracle.rope(qb, [j - i])[0, D - rd:] @ k[D - rd:]) < 1e-9 * (1 + abs(rhs))
    assert np.allclose(yi[1:2], oracle.rope(x[1:2], [-1]), atol=0)                 # inverse at p == forward at -p


def test_rope_group_maps_rows_to_positions():
    x = _rope_rows(3, 12, 128)
    pos = np.array([4, 9000, 77], np.int64)
    a = oracle.rope(x, pos, group=4)
    b = oracle.rope(x, np.repeat(pos, 4))
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.rope(x, pos, group=5)


# ---------------------------------------------------------------------------
# separate keys and values (the variant that keeps them apart)
# ---------------------------------------------------------------------------

def test_separate_values_match_library_attention():
    # sparse: selected entries + window, values from their own arrays; the library's SDPA (fp64, CPU) over
    # the gathered key and value rows gives the same result
    B, Tq, H, D, Nc, W, Lr = 2, 2, 16, 32, 30, 5, 9
    q, kv = synth.attn_inputs(40, B, Tq, H, D, Nc, "sk_")
    _, v = synth.attn_inputs(41, B, Tq, H, D, Nc, "sv_")
    _, raw = synth.attn_inputs(42, B, Tq, H, D, Lr, "rk_")
    _, vraw = synth.attn_inputs(43, B, Tq, H, D, Lr, "rv_")
    idx = np.array([[[1, 4, 9, 22, -1], [0, 7, 8, 29, 3]]] * B, np.int32)
    raw0, pos0 = 100, 106
    out, lse = oracle.sparse_attn(q, kv, idx, raw, raw0=raw0, pos0=pos0, W=W, scale=0.7, v=v, v_raw=vraw)
    for b in range(B):
        for t in range(Tq):
            p = pos0 + t
            sel = [j for j in idx[b, t] if j >= 0]
            win = list(range(max(0, p - W + 1) - raw0, p - raw0 + 1))
            K = np.concatenate([_bf16_f64(kv[b, sel]), _bf16_f64(raw[b, win])])
            V = np.concatenate([_bf16_f64(v[b, sel]), _bf16_f64(vraw[b, win])])
            Q = torch.from_numpy(_bf16_f64(q[b, t]))[:, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q, torch.from_numpy(K)[None].expand(H, -1, -1), torch.from_numpy(V)[None].expand(H, -1, -1), scale=0.7)
            np.testing.assert_allclose(out[b, t], ref[:, 0].numpy(), rtol=1e-10, atol=1e-13)
            lg = 0.7 * _bf16_f64(q[b, t]) @ K.T
            np.testing.assert_allclose(lse[b, t], np.log(np.exp(lg).sum(1)), rtol=1e-12)
    # dense: every visible entry with its own value
    out_d, _ = oracle.dense_attn(q, kv, L=Nc * 4, mh=4, pos0=Nc * 4 - Tq, scale=0.7, v_h=v)
    for b in range(B):
        K, V = _bf16_f64(kv[b]), _bf16_f64(v[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(_bf16_f64(q[b, -1]))[:, None, :], torch.from_numpy(K)[None].expand(H, -1, -1),
            torch.from_numpy(V)[None].expand(H, -1, -1), scale=0.7)
        np.testing.assert_allclose(out_d[b, -1], ref[:, 0].numpy(), rtol=1e-10, atol=1e-13)


def test_separate_values_single_row_and_linearity():
    B, Tq, H, D = 1, 1, 16, 32
    q, kv = synth.attn_inputs(44, B, Tq, H, D, 6, "lk_")
    _, v1 = synth.attn_inputs(45, B, Tq, H, D, 6, "lv1_")
    _, v2 = synth.attn_inputs(46, B, Tq, H, D, 6, "lv2_")
    # one visible entry: the output is that entry's value, not its key
    out, _ = oracle.dense_attn(q, kv[:, :1], L=4, mh=4, pos0=3, scale=0.3, v_h=v1[:, :1])
    np.testing.assert_array_equal(out[0, 0], np.broadcast_to(_bf16_f64(v1[0, 0]), (H, D)))
    # the output is linear in the values: out(v1) + out(v2) = out over value rows v1 + v2
    a, _ = oracle.dense_attn(q, kv, L=24, mh=4, pos0=23, scale=0.3, v_h=v1)
    c, _ = oracle.dense_attn(q, kv, L=24, mh=4, pos0=23, scale=0.3, v_h=v2)
    s = _bf16_f64(v1) + _bf16_f64(v2)
    w = np.exp(0.3 * _bf16_f64(q[0, 0]) @ _bf16_f64(kv[0]).T)
    w /= w.sum(1, keepdims=True)
    np.testing.assert_allclose(a[0, 0] + c[0, 0], w @ s[0], rtol=1e-12, atol=1e-15)
    # values equal to the keys reproduce the shared-row result exactly
    same, _ = oracle.dense_attn(q, kv, L=24, mh=4, pos0=23, scale=0.3, v_h=kv)
    base, _ = oracle.dense_attn(q, kv, L=24, mh=4, pos0=23, scale=0.3)
    np.testing.assert_array_equal(same, base)


# ---------------------------------------------------------------------------
# FP8 storage of the non-RoPE KV dimensions (C12) and MXFP4 indexer operands (C13)
# ---------------------------------------------------------------------------

def _fp8_case(seed, n, D, scale):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((n, D)) * scale * 2.0 ** g.integers(-6, 7, (n, 1))).astype(np.float32)
    x[0, :64] = 0.0                                           # an all-zero group
    x[1, 5] = 448.0 * 2.0 ** -10                              # a group whose maximum sits exactly on 448 * 2^e
    return synth.to_bf16_bits(x)


@pytest.mark.parametrize("D", [128, 512])
def test_kv_fp8_encode_matches_library_e4m3(D):
    x = _fp8_case(3, 20, D, 0.05)
    y = oracle.kv_fp8_encode(x)
    assert y.shape == (20, D + 80) and oracle.kv_fp8_row_bytes(D) == D + 80
    xv = _bf16_f64(x)
    for r in range(x.shape[0]):
        for g in range((D - 64) // 64):
            amax = np.abs(xv[r, 64 * g:64 * g + 64]).max()
            if amax == 0:
                e = 0
            else:                                             # smallest e with amax <= 448 * 2^e, in exact rationals
                e = math.ceil(math.log2(amax / 448.0)) + 1
                while Fraction(amax) <= Fraction(448) * Fraction(2) ** (e - 1):
                    e -= 1
            assert y[r, D + 64 + g] == e + 127
            ref = torch.from_numpy(np.ldexp(xv[r, 64 * g:64 * g + 64], -e).astype(np.float32))
            ref = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(y[r, 64 * g:64 * g + 64], ref)
        assert np.array_equal(y[r, D - 64:D + 64].view(np.uint16), x[r, D - 64:])        # RoPE dims untouched
        assert (y[r, D + 64 + (D - 64) // 64:] == 0).all()
    assert (y[0, D + 64] == 127) and (y[0, :64] == 0).all()


@pytest.mark.parametrize("D", [128, 512])
def test_kv_fp8_decode_and_round_trip(D):
    x = _fp8_case(4, 16, D, 0.05)
    y = oracle.kv_fp8_encode(x)
    got = oracle.kv_fp8_decode(y, D)
    # independent decode through the library's e4m3 type
    codes = torch.from_numpy(np.ascontiguousarray(y[:, :D - 64])).view(torch.float8_e4m3fn).double().numpy()
    scale = np.repeat(np.ldexp(1.0, y[:, D + 64:D + 64 + (D - 64) // 64].astype(np.int64) - 127), 64, axis=1)
    np.testing.assert_array_equal(got[:, :D - 64], codes * scale)
    xv = _bf16_f64(x)
    np.testing.assert_array_equal(got[:, D - 64:], xv[:, D - 64:])
    err = np.abs(got[:, :D - 64] - xv[:, :D - 64])
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(xv[:, :D - 64]), 2.0 ** -10 * scale))
    # values already on the grid come back exactly
    np.testing.assert_array_equal(oracle.kv_fp8_decode(oracle.kv_fp8_encode(synth.to_bf16_bits(got.astype(np.float32))),
                                                       D), got)


def _mx_reference(xv):
    """The MX FP4 encoding from its specification, in plain numpy (independent of the oracle's C)."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    n = xv.shape[-1]
    codes = np.zeros(xv.shape[:-1] + (n // 2,), np.uint8)
    scales = np.zeros(xv.shape[:-1] + (n // 32,), np.uint8)
    for idx in np.ndindex(xv.shape[:-1]):
        for blk in range(n // 32):
            v = xv[idx][32 * blk:32 * blk + 32]
            amax = np.abs(v).max()
            X = -127 if amax == 0 else int(np.clip(np.frexp(amax)[1] - 1 - 2, -127, 127))
            scales[idx][blk] = X + 127
            for i, t in enumerate(np.ldexp(v, -X)):
                a = min(abs(t), 6.0)
                d = np.abs(mags - a)
                cand = np.flatnonzero(d == d.min())
                k = int(cand[0]) if len(cand) == 1 else int(cand[cand % 2 == 0][0])
                c = k | (8 if (t < 0 and k) else 0)
                j = 32 * blk + i
                codes[idx][j // 2] |= c << (4 * (j & 1))
    return codes, scales


def test_mxfp4_encode_matches_specification():
    g = np.random.default_rng(5)
    x = (g.standard_normal((6, 128)) * 2.0 ** g.integers(-20, 20, (6, 1))).astype(np.float32)
    x[0, :32] = 0.0
    # ties of E2M1 at scale 2^0 (amax 6): 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 2.5 -> 2, 5 -> 4, 3.5 -> 4
    x[1, 32:64] = 0.0
    x[1, 32:39] = [6.0, 0.25, 0.75, 1.25, 2.5, 5.0, -3.5]
    xb = synth.to_bf16_bits(x)
    codes, scales = oracle.mxfp4_encode(xb)
    rc, rs = _mx_reference(_bf16_f64(xb))
    assert np.array_equal(scales, rs) and np.array_equal(codes, rc)
    vals = oracle.mxfp4_values(codes, scales)
    np.testing.assert_array_equal(vals[1, 32:39], [6.0, 0.0, 1.0, 1.0, 2.0, 4.0, -4.0])
    assert scales[0, 0] == 0 and (vals[0, :32] == 0).all()


def test_mxfp4_exact_dot_vs_fraction_and_bf16_path():
    g = np.random.default_rng(6)
    for _ in range(20):
        a = synth.to_bf16_bits((g.standard_normal(128) * 2.0 ** g.integers(-30, 30, 128)).astype(np.float32))
        b_ = synth.to_bf16_bits((g.standard_normal(128) * 0.1).astype(np.float32))
        ac, as_ = oracle.mxfp4_encode(a)
        bc, bs = oracle.mxfp4_encode(b_)
        av, bv = oracle.mxfp4_values(ac, as_), oracle.mxfp4_values(bc, bs)
        want = frac_to_f32(sum((Fraction(float(p)) * Fraction(float(q)) for p, q in zip(av, bv)), Fraction(0)))
        assert oracle.exact_dot_mxfp4(ac, as_, bc, bs) == np.float32(want)


def test_mxfp4_scores_equal_bf16_scores_of_the_decoded_values():
    # every MXFP4 value of a quantized bf16 vector is a bf16 value, so the canonical MXFP4 scores and selection
    # must equal the bf16 path's on the decoded values
    B, Tq, HI, dI, Nc, m, k = 1, 2, 8, 128, 300, 4, 40
    q, w, kk, _ = synth.indexer_inputs(7, B, Tq, HI, dI, Nc, 0)
    qc, qs = oracle.mxfp4_encode(q)
    kc, ks = oracle.mxfp4_encode(kk)
    L = Nc * m
    idx, cnt, S, nv = oracle.index_topk_mxfp4(qc, qs, w, kc, ks, L, m, L - Tq, k)
    qb = synth.to_bf16_bits(oracle.mxfp4_values(qc, qs).astype(np.float32))
    kb = synth.to_bf16_bits(oracle.mxfp4_values(kc, ks).astype(np.float32))
    assert np.array_equal(_bf16_f64(qb), oracle.mxfp4_values(qc, qs))
    idx2, cnt2, S2, _ = oracle.index_topk(qb, w, kb, L, m, L - Tq, k)
    assert np.array_equal(S, S2, equal_nan=True) and np.array_equal(idx, idx2) and np.array_equal(cnt, cnt2)

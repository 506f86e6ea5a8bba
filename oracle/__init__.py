"""CPU oracle for the hybrid compressed attention (CSA + HCA) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and this
package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent
rows only); this module is argument marshalling with numpy.  Each function
states the step of the method it follows; the page citations are in
``oracle.c`` next to the code.

Dtypes on the boundary: bf16 values are ``np.uint16`` bit patterns, OCP e4m3
values are ``np.uint8`` bit patterns, fp32 parameters are ``np.float32``.

Parity pins: every function here is pinned by tests in
``tests/test_oracle_pins.py`` against closed forms, library routines, exact
rational brute force and invariants.  The *choice* of the compressor's gate
form and of the indexer's score form are readings of silent pages; those two
choices are "parity unpinned" (no page prints a formula or a worked value).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
E4M3 = 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        LL = ctypes.c_longlong
        D = ctypes.c_double
        lib.ora_bf16_value.argtypes = [ctypes.c_uint16]
        lib.ora_bf16_value.restype = D
        lib.ora_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.ora_e4m3_value.restype = D
        lib.ora_bf16_round.argtypes = [D]
        lib.ora_bf16_round.restype = ctypes.c_uint16
        lib.ora_e4m3_round.argtypes = [D]
        lib.ora_e4m3_round.restype = ctypes.c_uint8
        lib.ora_exact_dot_f32.argtypes = [P, P, I, I]
        lib.ora_exact_dot_f32.restype = ctypes.c_float
        lib.ora_n_visible.argtypes = [LL, LL, I]
        lib.ora_n_visible.restype = I
        lib.ora_compress.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, I, I, P, P, P]
        lib.ora_compress.restype = None
        lib.ora_index_score.argtypes = [P, P, P, I, I, I]
        lib.ora_index_score.restype = ctypes.c_float
        lib.ora_index_scores.argtypes = [I, I, I, I, I, LL, I, LL, I, P, P, P, P, P]
        lib.ora_index_scores.restype = None
        lib.ora_topk.argtypes = [I, I, I, P, P, P, P]
        lib.ora_topk.restype = None
        lib.ora_sparse_attn.argtypes = [I, I, I, I, I, I, I, LL, LL, I, D, P, P, P, P, P, P, P, P, P]
        lib.ora_sparse_attn.restype = I
        lib.ora_dense_attn.argtypes = [I, I, I, I, I, LL, I, LL, D, P, P, P, P, P, P]
        lib.ora_dense_attn.restype = None
        lib.ora_rope.argtypes = [I, I, I, I, D, I, P, P, P]
        lib.ora_rope.restype = None
        lib.ora_kv_fp8_row_bytes.argtypes = [I]
        lib.ora_kv_fp8_row_bytes.restype = I
        lib.ora_kv_fp8_encode.argtypes = [I, I, P, P]
        lib.ora_kv_fp8_encode.restype = None
        lib.ora_kv_fp8_decode.argtypes = [I, I, P, P]
        lib.ora_kv_fp8_decode.restype = None
        lib.ora_mxfp4_encode.argtypes = [I, I, P, P, P]
        lib.ora_mxfp4_encode.restype = None
        lib.ora_mxfp4_value.argtypes = [P, P, I]
        lib.ora_mxfp4_value.restype = D
        lib.ora_exact_dot_mxfp4.argtypes = [P, P, P, P, I]
        lib.ora_exact_dot_mxfp4.restype = ctypes.c_float
        lib.ora_index_scores_mxfp4.argtypes = [I, I, I, I, I, LL, I, LL, P, P, P, P, P, P, P]
        lib.ora_index_scores_mxfp4.restype = None
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _key_dtype(dtype):
    return np.uint16 if dtype == BF16 else np.uint8


# --- number formats --------------------------------------------------------

def bf16_value(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (as float64)."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.vectorize(lambda x: lib.ora_bf16_value(int(x)), otypes=[np.float64])(b)


def e4m3_value(bits) -> np.ndarray:
    """Exact value of OCP e4m3 bit patterns (as float64; NaN for 0x7f/0xff)."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint8)
    return np.vectorize(lambda x: lib.ora_e4m3_value(int(x)), otypes=[np.float64])(b)


def bf16_round(x) -> np.ndarray:
    """Round-to-nearest-even encoding of float64 values as bf16 bit patterns."""
    lib = _load()
    return np.vectorize(lambda v: lib.ora_bf16_round(float(v)), otypes=[np.uint16])(np.asarray(x, np.float64))


def e4m3_round(x) -> np.ndarray:
    """Round-to-nearest-even, saturating (+-448) encoding as OCP e4m3 bits."""
    lib = _load()
    return np.vectorize(lambda v: lib.ora_e4m3_round(float(v)), otypes=[np.uint8])(np.asarray(x, np.float64))


# --- A2 pieces --------------------------------------------------------------

def exact_dot_f32(a_bits, b_bits, dtype=BF16) -> np.float32:
    """Exact sum of a[i]*b[i] (bf16 or e4m3 bit patterns), rounded once to fp32."""
    lib = _load()
    a, pa = _c(a_bits, _key_dtype(dtype))
    b, pb = _c(b_bits, _key_dtype(dtype))
    assert a.shape == b.shape and a.ndim == 1
    return np.float32(lib.ora_exact_dot_f32(pa, pb, a.size, dtype))


def index_score(q_bits, w, k_bits, dtype=BF16) -> np.float32:
    """Canonical indexer score of one entry: fma chain of w_h * ReLU(RN32(q_h.k))."""
    lib = _load()
    q, pq = _c(q_bits, _key_dtype(dtype))
    w, pw = _c(w, np.float32)
    k, pk = _c(k_bits, _key_dtype(dtype))
    HI, dI = q.shape
    return np.float32(lib.ora_index_score(pq, pw, pk, HI, dI, dtype))


def n_visible(p: int, L: int, m: int) -> int:
    """Number of compressed entries visible to the query at absolute position p."""
    return int(_load().ora_n_visible(p, L, m))


def index_scores(q_idx, w_idx, k_idx, L: int, m: int, pos0: int, dtype=BF16):
    """Scores S[B][Tq][Nc] (NaN where invisible) and n_vis[B][Tq].

    q_idx[B][Tq][HI][dI], w_idx[B][Tq][HI] fp32, k_idx[B][Nc][dI]."""
    lib = _load()
    q, pq = _c(q_idx, _key_dtype(dtype))
    w, pw = _c(w_idx, np.float32)
    k, pk = _c(k_idx, _key_dtype(dtype))
    B, Tq, HI, dI = q.shape
    Nc = k.shape[1]
    assert k.shape == (B, Nc, dI) and w.shape == (B, Tq, HI)
    S = np.empty((B, Tq, Nc), np.float32)
    nv = np.empty((B, Tq), np.int32)
    lib.ora_index_scores(B, Tq, HI, dI, Nc, L, m, pos0, dtype, pq, pw, pk, _ptr(S), _ptr(nv))
    return S, nv


def topk(S, n_vis, k: int):
    """Top-k under (score desc, index asc): idx[..][k] ascending, -1 padded; cnt."""
    lib = _load()
    S = np.ascontiguousarray(S, np.float32)
    lead = S.shape[:-1]
    Nc = S.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    nv = np.ascontiguousarray(n_vis, np.int32).reshape(rows)
    idx = np.empty((rows, k), np.int32)
    cnt = np.empty(rows, np.int32)
    lib.ora_topk(rows, Nc, k, _ptr(S), _ptr(nv), _ptr(idx), _ptr(cnt))
    return idx.reshape(*lead, k), cnt.reshape(lead)


def index_topk(q_idx, w_idx, k_idx, L: int, m: int, pos0: int, k: int, dtype=BF16):
    S, nv = index_scores(q_idx, w_idx, k_idx, L, m, pos0, dtype)
    idx, cnt = topk(S, nv, k)
    return idx, cnt, S, nv


# --- A4 / A5 ---------------------------------------------------------------

def _sink(sink, H):
    if sink is None:
        return None
    s = np.ascontiguousarray(sink, dtype=np.float64)
    if s.shape != (H,):
        raise ValueError("sink: one logit per head")
    return s


def sparse_attn(q, kv, idx, kv_raw, raw0: int, pos0: int, W: int, scale: float, sink=None, v=None, v_raw=None):
    """CSA attention over selected entries + raw window; returns (out, lse) fp64.  sink: optional
    per-head attention-sink logits [H] (an extra denominator term with no value row).  v, v_raw: optional
    separate values of the entries and the raw rows (both or neither; default: each row is its own value)."""
    lib = _load()
    q, pq = _c(q, np.uint16)
    kv, pk = _c(kv, np.uint16)
    idx, pi = _c(idx, np.int32)
    B, Tq, H, D = q.shape
    Nc = kv.shape[1]
    topk_ = idx.shape[-1]
    if kv_raw is None:
        kv_raw = np.zeros((B, 0, D), np.uint16)
    kr, pr = _c(kv_raw, np.uint16)
    Lr = kr.shape[1]
    out = np.empty((B, Tq, H, D), np.float64)
    lse = np.empty((B, Tq, H), np.float64)
    sk = _sink(sink, H)
    if (v is None) != (v_raw is None):
        raise ValueError("sparse_attn: give both v and v_raw or neither")
    pv = pvr = None
    if v is not None:
        v, pv = _c(v, np.uint16)
        v_raw, pvr = _c(v_raw, np.uint16)
        if v.shape != kv.shape or v_raw.shape != kr.shape:
            raise ValueError("sparse_attn: values must have the keys' shapes")
    rc = lib.ora_sparse_attn(B, Tq, H, D, Nc, topk_, Lr, raw0, pos0, W, float(scale),
                             pq, pk, pi, pr, pv, pvr, _ptr(sk), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle sparse_attn: index or window outside the given rows")
    return out, lse


def dense_attn(q, kv_h, L: int, mh: int, pos0: int, scale: float, sink=None, v_h=None):
    """HCA attention over all visible compressed entries; returns (out, lse) fp64 (sink as above; v_h:
    optional separate values of the entries)."""
    lib = _load()
    q, pq = _c(q, np.uint16)
    kv, pk = _c(kv_h, np.uint16)
    B, Tq, H, D = q.shape
    Nh = kv.shape[1]
    out = np.empty((B, Tq, H, D), np.float64)
    lse = np.empty((B, Tq, H), np.float64)
    sk = _sink(sink, H)
    pv = None
    if v_h is not None:
        v_h, pv = _c(v_h, np.uint16)
        if v_h.shape != kv.shape:
            raise ValueError("dense_attn: values must have the keys' shape")
    lib.ora_dense_attn(B, Tq, H, D, Nh, L, mh, pos0, float(scale), pq, pk, pv, _ptr(sk), _ptr(out), _ptr(lse))
    return out, lse


def rope(x, pos, rd: int = 64, theta: float = 10000.0, inverse: bool = False, group: int = 1):
    """Partial rotary position embedding of bf16 rows x[..., D] (C11): the last rd dimensions are rotated in
    adjacent pairs, pair j by pos * theta^(-2j/rd) (negated when inverse); row r takes pos[r // group].
    Returns fp64 rows of x's shape."""
    lib = _load()
    x, px = _c(x, np.uint16)
    D = x.shape[-1]
    n = x.size // D
    pos = np.ascontiguousarray(pos, dtype=np.int64).reshape(-1)
    if rd % 2 or not 0 < rd <= D or n % group or pos.size != n // group:
        raise ValueError("rope: rd even in (0, D], one position per group of rows")
    y = np.empty(x.shape, np.float64)
    lib.ora_rope(n, D, rd, group, float(theta), 1 if inverse else 0, px, _ptr(pos), _ptr(y))
    return y


# --- A1 ---------------------------------------------------------------------

def compress(hidden, w_kv, w_ik, w_gate, b_slot, m: int, W: int = 0, j0: int = 0, j1=None):
    """Softmax-gated pooling of projected KV (and indexer keys) over blocks of m.

    hidden[B][L][Dh] bf16, w_kv[D][Dh] bf16, w_ik[dI][Dh] bf16 or None,
    w_gate[Dh] fp32, b_slot[m] fp32 or None.  Returns fp64 (kv[B][j1-j0][D],
    ik or None, win[B][W][D] or None)."""
    lib = _load()
    X, px = _c(hidden, np.uint16)
    Wk, pw = _c(w_kv, np.uint16)
    B, L, Dh = X.shape
    D = Wk.shape[0]
    if w_ik is not None:
        Wi, pwi = _c(w_ik, np.uint16)
        dI = Wi.shape[0]
    else:
        Wi, pwi, dI = None, None, 0
    g, pg = _c(w_gate, np.float32)
    if b_slot is not None:
        bs, pb = _c(b_slot, np.float32)
    else:
        bs, pb = None, None
    Nc = (L + m - 1) // m
    if j1 is None:
        j1 = Nc
    nj = j1 - j0
    kv = np.empty((B, nj, D), np.float64)
    ik = np.empty((B, nj, dI), np.float64) if dI else None
    win = np.empty((B, W, D), np.float64) if W else None
    lib.ora_compress(B, L, Dh, D, dI, m, W, px, pw, pwi, pg, pb, j0, j1,
                     _ptr(kv), _ptr(ik), _ptr(win))
    return kv, ik, win


# --- C12: FP8 storage of the non-RoPE KV dimensions ----------------------------------------------------------

def kv_fp8_row_bytes(D: int) -> int:
    return int(_load().ora_kv_fp8_row_bytes(D))


def kv_fp8_encode(x):
    """bf16 KV rows x[..., D] -> uint8 rows [..., D + 80]: e4m3 codes of the first D - 64 dimensions in groups of
    64 with a power-of-two scale each, the last 64 (RoPE) dimensions kept as bf16, the scale exponents."""
    lib = _load()
    x, px = _c(x, np.uint16)
    D = x.shape[-1]
    n = x.size // D
    y = np.empty(x.shape[:-1] + (D + 80,), np.uint8)
    lib.ora_kv_fp8_encode(n, D, px, _ptr(y))
    return y


def kv_fp8_decode(y, D: int):
    """uint8 rows [..., D + 80] -> fp64 values [..., D]."""
    lib = _load()
    y, py = _c(y, np.uint8)
    n = y.size // (D + 80)
    x = np.empty(y.shape[:-1] + (D,), np.float64)
    lib.ora_kv_fp8_decode(n, D, py, _ptr(x))
    return x


# --- C13: MXFP4 indexer operands --------------------------------------------------------------------------

def mxfp4_encode(x):
    """bf16 vectors x[..., n] (n % 32 == 0) -> (codes uint8 [..., n/2], scales uint8 [..., n/32]) in the OCP MX
    FP4 format (E2M1 elements, one E8M0 scale per 32)."""
    lib = _load()
    x, px = _c(x, np.uint16)
    n = x.shape[-1]
    rows = x.size // n
    codes = np.empty(x.shape[:-1] + (n // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (n // 32,), np.uint8)
    lib.ora_mxfp4_encode(rows, n, px, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp4_values(codes, scales):
    """Exact values (fp64) of MXFP4 vectors."""
    lib = _load()
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    n = codes.shape[-1] * 2
    rows = codes.size // (n // 2)
    out = np.empty(codes.shape[:-1] + (n,), np.float64)
    flat = out.reshape(rows, n)
    for r in range(rows):
        cr = codes.reshape(rows, n // 2)[r]
        sr = scales.reshape(rows, n // 32)[r]
        pcr, psr = _c(cr, np.uint8)[1], _c(sr, np.uint8)[1]
        for i in range(n):
            flat[r, i] = lib.ora_mxfp4_value(pcr, psr, i)
    return out


def exact_dot_mxfp4(ac, as_, bc, bs) -> np.float32:
    lib = _load()
    ac, pac = _c(ac, np.uint8)
    as_, pas = _c(as_, np.uint8)
    bc, pbc = _c(bc, np.uint8)
    bs, pbs = _c(bs, np.uint8)
    return np.float32(lib.ora_exact_dot_mxfp4(pac, pas, pbc, pbs, ac.size * 2))


def index_topk_mxfp4(qc, qs, w_idx, kc, ks, L: int, m: int, pos0: int, k: int):
    """Canonical scores over MXFP4 operands (q codes [B][Tq][HI][dI/2], scales [B][Tq][HI][dI/32]; k codes
    [B][Nc][dI/2], scales [B][Nc][dI/32]) and their top-k: (idx, cnt, S, n_vis)."""
    lib = _load()
    qc, pqc = _c(qc, np.uint8)
    qs, pqs = _c(qs, np.uint8)
    w, pw = _c(w_idx, np.float32)
    kc, pkc = _c(kc, np.uint8)
    ks, pks = _c(ks, np.uint8)
    B, Tq, HI, half = qc.shape
    dI = half * 2
    Nc = kc.shape[1]
    S = np.empty((B, Tq, Nc), np.float32)
    nv = np.empty((B, Tq), np.int32)
    lib.ora_index_scores_mxfp4(B, Tq, HI, dI, Nc, L, m, pos0, pqc, pqs, pw, pkc, pks, _ptr(S), _ptr(nv))
    idx, cnt = topk(S, nv, k)
    return idx, cnt, S, nv

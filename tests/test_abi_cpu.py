"""C-ABI contract tests that need no GPU: the library loads, exports every
function include/csa.h declares, sizes workspaces on the host, and rejects bad
arguments with the documented status codes before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")
LIB = os.path.join(ROOT, "compressed_sparse_kv_compressor_amd", "libcsa.so")

CSA_OK, CSA_ERR_NULL, CSA_ERR_SHAPE, CSA_ERR_DTYPE, CSA_ERR_ALIGN, CSA_ERR_WORKSPACE, CSA_ERR_UNSUPPORTED = range(7)


@pytest.fixture(scope="module")
def b():
    if not os.path.exists(LIB):
        from compressed_sparse_kv_compressor_amd import build
        build.build()
    from compressed_sparse_kv_compressor_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_][a-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("csa_", "hca_"))))


def test_every_declared_symbol_is_exported(b):
    names = declared_functions()
    assert len(names) >= 15, names
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in csa.h but not exported"
    assert set(names) == set(b.EXPORTED)


def test_version_and_status_strings(b):
    assert b.lib.csa_abi_version() == 6
    assert b.lib.csa_status_str(CSA_ERR_WORKSPACE) == b"CSA_ERR_WORKSPACE"
    assert b.lib.csa_status_str(99) == b"CSA_ERR_UNKNOWN"


def test_workspace_sizes_are_host_arithmetic(b):
    lib = b.lib
    assert lib.csa_index_topk_ws_bytes(8, 1, 8, 128, 262144, 1024, 1) > 8 * 262144 * 4
    assert lib.csa_index_topk_ws_bytes(0, 1, 8, 128, 10, 4, 0) == 0
    # chunked prefill, 8192 queries x 65536 entries: the many-query path keeps no score matrix
    assert lib.csa_index_topk_ws_bytes(1, 8192, 8, 128, 65536, 1024, 0) < 8192 * 65536 * 4 // 2
    # the same queries in e4m3, or with 4 heads of 64, are widened to bf16 8 x 128 on that path (two
    # widened operand copies, still no score matrix); 16 heads take the per-query path, which holds the scores
    bf16_ws = lib.csa_index_topk_ws_bytes(1, 8192, 8, 128, 65536, 1024, 0)
    widened = 65536 * 256 + 8192 * 8 * 256 + 8192 * 8 * 4
    assert bf16_ws < lib.csa_index_topk_ws_bytes(1, 8192, 8, 128, 65536, 1024, 1) <= bf16_ws + widened + 3 * 256
    assert lib.csa_index_topk_ws_bytes(1, 8192, 4, 64, 65536, 1024, 0) < 8192 * 65536 * 4 // 2
    assert lib.csa_index_topk_ws_bytes(1, 8192, 16, 128, 65536, 1024, 1) > 8192 * 65536 * 4
    assert lib.csa_sparse_attn_ws_bytes(8, 1, 128, 512, 1024, 128) > 0
    assert lib.hca_dense_attn_ws_bytes(1, 1, 16, 128, 32) == 0          # one split: no partials
    # compression of 4 x 65536 tokens of hidden 4096: the pooled rows, plus split-K partials only for
    # the projections with few output tiles (the window rows, the HCA entries)
    pooled = 4 * 16384 * 4096 * 2
    assert lib.csa_compress_ws_bytes(4, 65536, 4096, 512, 128, 4, 0) == pooled
    assert pooled < lib.csa_compress_ws_bytes(4, 65536, 4096, 512, 128, 4, 128) <= pooled + (64 << 20)
    assert lib.csa_compress_ws_bytes(4, 65536, 4096, 512, 0, 128, 0) > 4 * 512 * 4096 * 2
    assert lib.csa_compress_ws_bytes(4, 65536, 4096, 512, 0, 0, 0) == 0


A16 = ctypes.c_void_p(16 * 1000)       # aligned, never dereferenced (validation fails first)
BAD = ctypes.c_void_p(16 * 1000 + 2)   # misaligned


def test_index_topk_validation_codes(b):
    lib = b.lib
    f = lib.csa_index_topk
    good = dict(q=A16, w=A16, k=A16, dt=0, B=1, Tq=1, HI=8, dI=128, Nc=1024, L=4096, m=4, pos0=4095, topk=64,
                idx=A16, cnt=None, score=None, ws=A16, wsb=10 ** 9)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return f(a["q"], a["w"], a["k"], a["dt"], a["B"], a["Tq"], a["HI"], a["dI"], a["Nc"], a["L"], a["m"],
                 a["pos0"], a["topk"], a["idx"], a["cnt"], a["score"], a["ws"], a["wsb"], None)

    assert call(q=None) == CSA_ERR_NULL
    assert call(k=BAD) == CSA_ERR_ALIGN
    assert call(dt=7) == CSA_ERR_DTYPE
    assert call(Nc=1000) == CSA_ERR_SHAPE                 # not ceil(L/m)
    assert call(pos0=4096) == CSA_ERR_SHAPE               # query beyond the context
    assert call(topk=0) == CSA_ERR_SHAPE
    assert call(HI=3) == CSA_ERR_UNSUPPORTED
    assert call(dI=96) == CSA_ERR_UNSUPPORTED
    assert call(topk=5000) == CSA_ERR_UNSUPPORTED
    assert call(wsb=10) == CSA_ERR_WORKSPACE
    assert b"workspace" in lib.csa_last_error()
    assert call(ws=None) == CSA_ERR_NULL
    assert call(score=BAD) == CSA_ERR_ALIGN


def test_attention_validation_codes(b):
    lib = b.lib
    sp = lib.csa_sparse_attn
    # q, kv, idx, kv_raw, B, Tq, H, D, Nc, topk, Lr, raw0, pos0, W, scale, sink, out, lse, ws, wsb, stream
    assert sp(A16, A16, A16, A16, 1, 1, 16, 96, 10, 4, 8, 0, 7, 4, 0.1, None, A16, None, A16, 10 ** 9, None) == CSA_ERR_UNSUPPORTED
    assert sp(A16, A16, A16, A16, 1, 1, 24, 128, 10, 4, 8, 0, 7, 4, 0.1, None, A16, None, A16, 10 ** 9, None) == CSA_ERR_UNSUPPORTED
    assert sp(A16, A16, A16, None, 1, 1, 16, 128, 10, 4, 8, 0, 7, 4, 0.1, None, A16, None, A16, 10 ** 9, None) == CSA_ERR_NULL
    # window needs raw rows starting at 4 but they start at 5
    assert sp(A16, A16, A16, A16, 1, 1, 16, 128, 10, 4, 8, 5, 7, 4, 0.1, None, A16, None, A16, 10 ** 9, None) == CSA_ERR_SHAPE
    # window needs position 7 but rows end at 6
    assert sp(A16, A16, A16, A16, 1, 1, 16, 128, 10, 4, 7, 0, 7, 4, 0.1, None, A16, None, A16, 10 ** 9, None) == CSA_ERR_SHAPE
    assert sp(A16, A16, A16, A16, 1, 1, 16, 128, 10, 4, 8, 0, 7, 4, float("nan"), None, A16, None, A16, 10 ** 9, None) == CSA_ERR_SHAPE
    de = lib.hca_dense_attn
    # q, kv_h, B, Tq, H, D, Nh, L, mh, pos0, scale, sink, out, lse, ws, wsb, stream
    assert de(A16, A16, 1, 1, 16, 128, 31, 4096, 128, 4095, 0.1, None, A16, None, A16, 10 ** 9, None) == CSA_ERR_SHAPE
    assert de(A16, None, 1, 1, 16, 128, 32, 4096, 128, 4095, 0.1, None, A16, None, A16, 10 ** 9, None) == CSA_ERR_NULL
    assert de(A16, A16, 1, 1, 16, 128, 32, 4096, 128, 4095, 0.1, None, BAD, None, A16, 10 ** 9, None) == CSA_ERR_ALIGN


def test_compress_and_decode_validation_codes(b):
    lib = b.lib
    c = lib.csa_compress
    # hidden, w_kv, w_ik, w_gate, b_slot, B, L, Dh, D, dI, m, W, ik_dtype, kv, ik, win, ws, wsb, stream
    assert c(A16, A16, None, A16, None, 1, 100, 100, 128, 0, 4, 0, 0, A16, None, None, A16, 10 ** 9, None) == CSA_ERR_UNSUPPORTED
    assert c(A16, A16, A16, A16, None, 1, 100, 128, 128, 64, 4, 0, 0, A16, None, None, A16, 10 ** 9, None) == CSA_ERR_NULL
    assert c(A16, A16, None, A16, None, 1, 100, 128, 128, 0, 4, 8, 0, A16, None, None, A16, 10 ** 9, None) == CSA_ERR_NULL
    assert c(A16, A16, None, A16, None, 1, 100, 128, 128, 0, 4, 0, 5, A16, None, None, A16, 10 ** 9, None) == CSA_ERR_DTYPE
    assert c(A16, A16, None, A16, None, 1, 100, 128, 128, 0, 4, 0, 0, A16, None, None, A16, 10, None) == CSA_ERR_WORKSPACE
    args = b.DecodeArgs(B=1, L=4096, H=16, D=128, scale=0.1, csa_q=A16, q_idx=A16, w_idx=A16, k_idx=A16, kv=A16,
                        kv_raw=A16, idx_dtype=0, HI=4, dI=64, m=4, topk=64, W=128, csa_out=A16, csa_lse=None,
                        idx_out=None, hca_q=A16, kv_h=None, mh=128, hca_out=A16, hca_lse=None)
    assert lib.csa_hca_decode(ctypes.byref(args), A16, 10 ** 9, None) == CSA_ERR_NULL
    assert lib.csa_hca_decode(None, A16, 10 ** 9, None) == CSA_ERR_NULL
    args.kv_h = A16
    args.kv_format = 7                     # checked before any launch
    assert lib.csa_hca_decode(ctypes.byref(args), A16, 10 ** 9, None) == CSA_ERR_DTYPE
    args.kv_format = 0
    args.ws_persistent = 2                 # 0 or 1 only, checked before any launch
    assert lib.csa_hca_decode(ctypes.byref(args), A16, 10 ** 9, None) == CSA_ERR_SHAPE
    args.ws_persistent = 0
    assert lib.csa_hca_decode(ctypes.byref(args), A16, 16, None) == CSA_ERR_WORKSPACE
    assert lib.csa_hca_decode_ws_bytes(ctypes.byref(args)) > 16


def test_decode_args_keep_their_tensors_alive(b):
    """The decode args hold bare addresses; the struct must own references to what they point into."""
    import gc
    import weakref

    import torch
    t = torch.zeros(16, dtype=torch.float32)
    ref = weakref.ref(t)
    z = torch.zeros(4, dtype=torch.int16)
    args = b.make_decode_args(L=8, scale=0.1, csa_q=torch.zeros(1, 16, 128, dtype=torch.int16), q_idx=z.view(1, 1, 4),
                              w_idx=z, k_idx=z, kv=z, kv_raw=z, idx_dtype=0, m=4, topk=1, W=0, csa_out=z,
                              hca_q=torch.zeros(1, 16, 128, dtype=torch.int16), kv_h=z, mh=4, hca_out=z, csa_sink=t)
    del t
    gc.collect()
    assert ref() is not None and args.csa_sink == ref().data_ptr()


def test_rope_validation_codes(b):
    """Argument checks of csa_rope (no launch: every call fails before one, or has no rows)."""
    lib = b.lib
    r = lib.csa_rope
    # x, y, pos, n, D, rd, group, theta, inverse, stream
    assert r(None, None, None, 0, 512, 64, 1, 10000.0, 0, None) == 0                    # no rows: no-op
    assert r(A16, A16, A16, 4, 500, 64, 1, 10000.0, 0, None) == CSA_ERR_SHAPE            # D % 8
    assert r(A16, A16, A16, 4, 512, 60, 1, 10000.0, 0, None) == CSA_ERR_SHAPE            # rd % 8
    assert r(A16, A16, A16, 4, 128, 256, 1, 10000.0, 0, None) == CSA_ERR_SHAPE           # rd > D
    assert r(A16, A16, A16, 4, 512, 64, 3, 10000.0, 0, None) == CSA_ERR_SHAPE            # group does not divide n
    assert r(A16, A16, A16, 4, 512, 64, 1, 1.0, 0, None) == CSA_ERR_SHAPE                # theta <= 1
    assert r(A16, A16, A16, 4, 512, 64, 1, float("inf"), 0, None) == CSA_ERR_SHAPE
    assert r(A16, A16, A16, 4, 512, 64, 1, 10000.0, 2, None) == CSA_ERR_SHAPE            # inverse not 0/1
    assert r(A16, A16, None, 4, 512, 64, 1, 10000.0, 0, None) == CSA_ERR_NULL
    assert r(BAD, A16, A16, 4, 512, 64, 1, 10000.0, 0, None) == CSA_ERR_ALIGN


def test_layout_validation_codes(b):
    """The batch / cache layout is checked before any launch."""
    lib = b.lib
    f = lib.csa_index_topk_ex

    def idx_call(lay, **kw):
        a = dict(q=A16, w=A16, k=A16, dt=0, B=1, Tq=1, HI=8, dI=128, Nc=1024, L=4096, m=4, pos0=4095, topk=64)
        a.update(kw)
        return f(a["q"], a["w"], a["k"], a["dt"], a["B"], a["Tq"], a["HI"], a["dI"], a["Nc"], a["L"], a["m"],
                 a["pos0"], a["topk"], A16, None, None, ctypes.byref(lay), None, None, A16, 10 ** 9, None)

    ok = b.CacheLayout(seq_lens=A16, block_table=A16, max_blocks=32, num_blocks=40, block_tokens=128)
    assert idx_call(b.CacheLayout(seq_lens=ctypes.c_void_p(16 * 1000 + 4))) == CSA_ERR_ALIGN
    bad_tokens = b.CacheLayout(block_table=A16, max_blocks=32, num_blocks=40, block_tokens=100)
    assert idx_call(bad_tokens) == CSA_ERR_UNSUPPORTED                          # not a multiple of m
    npow2 = b.CacheLayout(block_table=A16, max_blocks=32, num_blocks=40, block_tokens=12)
    assert idx_call(npow2) == CSA_ERR_UNSUPPORTED                               # 3 entries per page
    short = b.CacheLayout(block_table=A16, max_blocks=31, num_blocks=40, block_tokens=128)
    assert idx_call(short) == CSA_ERR_SHAPE                                     # 31 x 32 < 1024 entries
    assert idx_call(b.CacheLayout(block_table=A16, max_blocks=32, num_blocks=0, block_tokens=128)) == CSA_ERR_SHAPE
    assert lib.csa_index_topk_ex_ws_bytes(1, 8192, 8, 128, 65536, 1024, 0, None) < \
        lib.csa_index_topk_ex_ws_bytes(1, 8192, 8, 128, 65536, 1024, 0, ctypes.byref(ok))   # no many-query path
    sp = lib.csa_sparse_attn_ex
    # q, kv, v, idx, kv_raw, v_raw, B, Tq, H, D, Nc, m, topk, Lr, raw0, pos0, W, scale, sink, layout, fmt, rope, out, ...
    var = b.CacheLayout(seq_lens=A16)
    assert sp(A16, A16, None, A16, A16, None, 2, 2, 16, 128, 100, 4, 8, 9, 0, 0, 9, 0.1, None, ctypes.byref(var), 0,
              None, A16, None, A16, 10 ** 9, None) == CSA_ERR_SHAPE                   # Lr < Tq + W - 1
    assert sp(A16, A16, BAD, A16, A16, None, 2, 2, 16, 128, 100, 4, 8, 10, 0, 0, 9, 0.1, None, ctypes.byref(var), 0,
              None, A16, None, A16, 10 ** 9, None) == CSA_ERR_ALIGN
    assert sp(A16, A16, None, A16, A16, None, 2, 2, 16, 128, 100, 0, 8, 10, 0, 0, 9, 0.1, None, ctypes.byref(var), 0,
              None, A16, None, A16, 10 ** 9, None) == CSA_ERR_SHAPE                   # m = 0
    # the fused rotary embedding: rd must be 64, theta finite and > 1
    for rope, code in (((32, 1e4), CSA_ERR_UNSUPPORTED), ((64, 1.0), CSA_ERR_SHAPE), ((64, float("inf")), CSA_ERR_SHAPE)):
        rp = b.RopeSpec(rd=rope[0], theta=rope[1])
        assert sp(A16, A16, None, A16, A16, None, 2, 2, 16, 128, 100, 4, 8, 10, 0, 0, 9, 0.1, None, None, 0,
                  ctypes.byref(rp), A16, None, A16, 10 ** 9, None) == code

"""Thin Python binding of libcsa.so (include/csa.h).

Argument marshalling only: torch tensors supply device memory and the current
stream; every step of the method runs in the library's HIP kernels.  Each
function has the C entry point's name and raises CsaError on a non-zero status.
If libcsa.so is missing the import fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

BF16 = 0
E4M3 = 1
MXFP4 = 2
KV_BF16 = 0
KV_FP8 = 1


class CsaError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, LL, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_size_t
    sig = {
        "csa_abi_version": ([], I),
        "csa_status_str": ([I], ctypes.c_char_p),
        "csa_last_error": ([], ctypes.c_char_p),
        "csa_compress_ws_bytes": ([I, LL, I, I, I, I, I], Z),
        "csa_compress": ([P, P, P, P, P, I, LL, I, I, I, I, I, I, P, P, P, P, Z, P], I),
        "csa_hca_compress_ws_bytes": ([I, LL, I, I, I, I, I, I], Z),
        "csa_hca_compress": ([P, I, LL, I, P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, I, P, P, Z, P], I),
        "csa_append_state_bytes": ([I, I], Z),
        "csa_decode_append_ws_bytes": ([I, I, I, I], Z),
        "csa_decode_append": ([P, I, I, I, P, P, P, P, I, I, I, I, P, P, P, I, LL, P, P, P, P, P, P, I, P, P, Z, P], I),
        "csa_index_topk_ws_bytes": ([I, I, I, I, I, I, I], Z),
        "csa_index_topk": ([P, P, P, I, I, I, I, I, I, LL, I, LL, I, P, P, P, P, Z, P], I),
        "csa_index_topk_ex_ws_bytes": ([I, I, I, I, I, I, I, P], Z),
        "csa_index_topk_ex": ([P, P, P, I, I, I, I, I, I, LL, I, LL, I, P, P, P, P, P, P, P, Z, P], I),
        "csa_sparse_attn_ex": ([P, P, P, P, P, P, I, I, I, I, I, I, I, I, LL, LL, I, F, P, P, I, P, P, P, P, Z, P], I),
        "hca_dense_attn_ex": ([P, P, P, I, I, I, I, I, LL, I, LL, F, P, P, I, P, P, P, P, Z, P], I),
        "csa_kv_fp8_encode": ([P, LL, I, P, P], I),
        "csa_mxfp4_encode": ([P, LL, I, P, P, P], I),
        "csa_sparse_attn_ws_bytes": ([I, I, I, I, I, I], Z),
        "csa_sparse_attn": ([P, P, P, P, I, I, I, I, I, I, I, LL, LL, I, F, P, P, P, P, Z, P], I),
        "csa_sparse_attn_noalloc": ([P, P, P, P, I, I, I, I, I, I, I, LL, LL, I, F, P, P, P, P], I),
        "hca_dense_attn_ws_bytes": ([I, I, I, I, I], Z),
        "hca_dense_attn": ([P, P, I, I, I, I, I, LL, I, LL, F, P, P, P, P, Z, P], I),
        "csa_hca_decode_ws_bytes": ([P], Z),
        "csa_hca_decode": ([P, P, Z, P], I),
        "csa_rope": ([P, P, P, LL, I, I, I, ctypes.c_double, I, P], I),
        "csa_debug_fp8_to_bf16": ([P, P, I, P], I),
        "csa_prof_enable": ([I], I),
        "csa_prof_reset": ([], I),
        "csa_prof_only": ([ctypes.c_char_p], I),
        "csa_prof_read": ([ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I)], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()

EXPORTED = ("csa_abi_version", "csa_status_str", "csa_last_error", "csa_compress_ws_bytes", "csa_compress",
            "csa_hca_compress_ws_bytes", "csa_hca_compress",
            "csa_index_topk_ws_bytes", "csa_index_topk", "csa_sparse_attn_ws_bytes", "csa_sparse_attn",
            "csa_sparse_attn_noalloc", "csa_append_state_bytes", "csa_decode_append_ws_bytes", "csa_decode_append",
            "csa_index_topk_ex_ws_bytes", "csa_index_topk_ex", "csa_sparse_attn_ex",
            "hca_dense_attn_ex", "csa_kv_fp8_encode", "csa_mxfp4_encode",
            "hca_dense_attn_ws_bytes", "hca_dense_attn", "csa_hca_decode_ws_bytes", "csa_hca_decode",
            "csa_rope", "csa_debug_fp8_to_bf16", "csa_prof_enable", "csa_prof_reset", "csa_prof_read",
            "csa_prof_only")


class CacheLayout(ctypes.Structure):
    """Mirror of csa_cache_layout_t (variable-length batch and/or paged caches)."""
    _fields_ = [("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int),
                ("num_blocks", ctypes.c_int), ("block_tokens", ctypes.c_int)]


def make_layout(seq_lens=None, block_table=None, num_blocks: int = 0, block_tokens: int = 0) -> CacheLayout:
    """seq_lens: int64 device tensor [B] or None; block_table: int32 device tensor [B][max_blocks] or None."""
    if seq_lens is not None and (seq_lens.dtype != torch.int64 or not seq_lens.is_contiguous()):
        raise ValueError("seq_lens must be a contiguous int64 tensor")
    if block_table is not None and (block_table.dtype != torch.int32 or block_table.dim() != 2
                                    or not block_table.is_contiguous()):
        raise ValueError("block_table must be a contiguous int32 [B][max_blocks] tensor")
    lay = CacheLayout(seq_lens=_p(seq_lens), block_table=_p(block_table),
                      max_blocks=0 if block_table is None else block_table.shape[1], num_blocks=num_blocks,
                      block_tokens=block_tokens)
    lay._keep = (seq_lens, block_table)
    return lay


def _lay(layout):
    return None if layout is None else ctypes.byref(layout)


class RopeSpec(ctypes.Structure):
    """Mirror of csa_rope_t: the fused rotary embedding of an attention call (rd = 64)."""
    _fields_ = [("rd", ctypes.c_int), ("theta", ctypes.c_double)]


def _rope(rope):
    """None, or (rd, theta) -> a csa_rope_t the call can point at."""
    return None if rope is None else RopeSpec(rd=int(rope[0]), theta=float(rope[1]))


class DecodeArgs(ctypes.Structure):
    """Mirror of csa_hca_decode_args_t."""
    _fields_ = [
        ("B", ctypes.c_int), ("L", ctypes.c_longlong), ("H", ctypes.c_int), ("D", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("csa_q", ctypes.c_void_p), ("q_idx", ctypes.c_void_p), ("w_idx", ctypes.c_void_p),
        ("k_idx", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_raw", ctypes.c_void_p),
        ("idx_dtype", ctypes.c_int), ("HI", ctypes.c_int), ("dI", ctypes.c_int), ("m", ctypes.c_int),
        ("topk", ctypes.c_int), ("W", ctypes.c_int),
        ("csa_out", ctypes.c_void_p), ("csa_lse", ctypes.c_void_p), ("idx_out", ctypes.c_void_p),
        ("csa_sink", ctypes.c_void_p),
        ("hca_q", ctypes.c_void_p), ("kv_h", ctypes.c_void_p), ("mh", ctypes.c_int),
        ("hca_out", ctypes.c_void_p), ("hca_lse", ctypes.c_void_p), ("hca_sink", ctypes.c_void_p),
        ("layout", ctypes.POINTER(CacheLayout)),
        ("q_idx_scale", ctypes.c_void_p), ("k_idx_scale", ctypes.c_void_p),
        ("csa_rope", ctypes.POINTER(RopeSpec)), ("hca_rope", ctypes.POINTER(RopeSpec)),
        ("kv_format", ctypes.c_int), ("ws_persistent", ctypes.c_int),
    ]


def _check(rc: int):
    if rc != 0:
        raise CsaError(f"{lib.csa_status_str(rc).decode()}: {lib.csa_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace(nbytes: int, device) -> torch.Tensor | None:
    """Device workspace of at least nbytes (256-byte aligned by the caching allocator)."""
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def csa_compress(hidden, w_kv, w_ik, w_gate, b_slot, m: int, W: int, kv_out, ik_out=None, win_out=None,
                 ik_dtype: int = BF16, ws=None, stream=None):
    B, L, Dh = hidden.shape
    D = w_kv.shape[0]
    dI = w_ik.shape[0] if w_ik is not None else 0
    need = lib.csa_compress_ws_bytes(B, L, Dh, D, dI if ik_out is not None else 0, m, W if win_out is not None else 0)
    if ws is None:
        ws = workspace(need, hidden.device)
    _check(lib.csa_compress(_p(hidden), _p(w_kv), _p(w_ik), _p(w_gate), _p(b_slot), B, L, Dh, D, dI, m, W, ik_dtype,
                            _p(kv_out), _p(ik_out), _p(win_out), _p(ws), 0 if ws is None else ws.numel(),
                            _stream(stream)))


def csa_hca_compress(hidden, w_kv, w_ik, w_gate, b_slot, m: int, W: int, kv_out, ik_out, win_out, w_kv_h, w_gate_h,
                     b_slot_h, mh: int, kv_h_out, ik_dtype: int = BF16, ws=None, stream=None):
    B, L, Dh = hidden.shape
    D = w_kv.shape[0]
    dI = w_ik.shape[0] if w_ik is not None else 0
    need = lib.csa_hca_compress_ws_bytes(B, L, Dh, D, dI if ik_out is not None else 0, m,
                                         W if win_out is not None else 0, mh)
    if ws is None:
        ws = workspace(need, hidden.device)
    _check(lib.csa_hca_compress(_p(hidden), B, L, Dh, _p(w_kv), _p(w_ik), _p(w_gate), _p(b_slot), D, dI, m, W,
                                ik_dtype, _p(kv_out), _p(ik_out), _p(win_out), _p(w_kv_h), _p(w_gate_h), _p(b_slot_h),
                                mh, _p(kv_h_out), _p(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def csa_decode_append(hidden, w_kv, w_ik, w_gate, b_slot, m: int, w_kv_h, w_gate_h, b_slot_h, mh: int, L: int,
                      seq_lens, state, kv_out, ik_out, kv_h_out, win, ik_dtype: int = BF16, layout=None, ws=None,
                      stream=None):
    """Append hidden[B][T][Dh] to every sequence (see csa.h): projections, running block pools in `state`
    (bytes: lib.csa_append_state_bytes(D, dI) per sequence), rewritten entries, shifted window, seq_lens += T."""
    B, T, Dh = hidden.shape
    D = w_kv.shape[0]
    dI = w_ik.shape[0] if w_ik is not None else 0
    W = win.shape[1] if win is not None else 0
    if seq_lens.dtype != torch.int64 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be B int64 values")
    if ws is None:
        ws = workspace(lib.csa_decode_append_ws_bytes(B, T, D, dI), hidden.device)
    _check(lib.csa_decode_append(_p(hidden), B, T, Dh, _p(w_kv), _p(w_ik), _p(w_gate), _p(b_slot), D, dI, m, ik_dtype,
                                 _p(w_kv_h), _p(w_gate_h), _p(b_slot_h), mh, L, _p(seq_lens), _p(state), _p(kv_out),
                                 _p(ik_out), _p(kv_h_out), _p(win), W, _lay(layout), _p(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)))


def csa_index_topk(q_idx, w_idx, k_idx, dtype: int, L: int, m: int, pos0: int, topk: int, idx_out, cnt_out=None,
                   ws=None, stream=None, score_out=None, layout=None, Nc=None, q_scale=None, k_scale=None):
    """layout (make_layout): variable-length batch and/or paged keys (k_idx is then the pool and Nc = ceil(L/m)
    unless given).  dtype MXFP4: q_idx / k_idx are the E2M1 codes (last dim dI/2) and q_scale / k_scale their
    E8M0 scales (last dim dI/32)."""
    B, Tq, HI, dI = q_idx.shape
    if dtype == MXFP4:
        dI *= 2
    if Nc is None:
        Nc = k_idx.shape[1] if (layout is None or not layout.block_table) else -(-L // m)
    ex = layout is not None or dtype == MXFP4
    if not ex:
        need = lib.csa_index_topk_ws_bytes(B, Tq, HI, dI, Nc, topk, dtype)
    else:
        need = lib.csa_index_topk_ex_ws_bytes(B, Tq, HI, dI, Nc, topk, dtype, _lay(layout))
    if ws is None:
        ws = workspace(need, q_idx.device)
    if not ex:
        _check(lib.csa_index_topk(_p(q_idx), _p(w_idx), _p(k_idx), dtype, B, Tq, HI, dI, Nc, L, m, pos0, topk,
                                  _p(idx_out), _p(cnt_out), _p(score_out), _p(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream)))
    else:
        _check(lib.csa_index_topk_ex(_p(q_idx), _p(w_idx), _p(k_idx), dtype, B, Tq, HI, dI, Nc, L, m, pos0, topk,
                                     _p(idx_out), _p(cnt_out), _p(score_out), _lay(layout), _p(q_scale), _p(k_scale),
                                     _p(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def _sink(sink, H: int):
    """The per-head attention-sink logits: None, or H float32 values on the device."""
    if sink is not None and (sink.dtype != torch.float32 or sink.numel() != H or not sink.is_contiguous()):
        raise ValueError(f"sink must be {H} contiguous float32 values, got {sink.dtype} x {sink.numel()}")
    return _p(sink)


def csa_sparse_attn(q, kv, idx, kv_raw, raw0: int, pos0: int, W: int, scale: float, out, lse_out=None, ws=None,
                    stream=None, sink=None, v=None, v_raw=None, layout=None, m: int = 1, Nc=None, kv_format=KV_BF16,
                    rope=None):
    """v, v_raw: separate values (or None); layout (make_layout): variable-length batch and/or paged entries
    (kv and v are then pools of ratio m; Nc = the entries per sequence the idx refer to); kv_format KV_FP8: kv
    (and v) rows in the FP8 format (csa_kv_fp8_encode); rope = (rd, theta): the fused rotary embedding."""
    B, Tq, H, D = q.shape
    if Nc is None:
        Nc = kv.shape[1] if kv is not None else 0
    topk = idx.shape[-1] if idx is not None else 0
    Lr = kv_raw.shape[1] if kv_raw is not None else 0
    need = lib.csa_sparse_attn_ws_bytes(B, Tq, H, D, topk, W)
    if ws is None:
        ws = workspace(need, q.device)
    if layout is None and v is None and v_raw is None and kv_format == KV_BF16 and rope is None:
        _check(lib.csa_sparse_attn(_p(q), _p(kv), _p(idx), _p(kv_raw), B, Tq, H, D, Nc, topk, Lr, raw0, pos0, W,
                                   float(scale), _sink(sink, H), _p(out), _p(lse_out), _p(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)))
    else:
        _check(lib.csa_sparse_attn_ex(_p(q), _p(kv), _p(v), _p(idx), _p(kv_raw), _p(v_raw), B, Tq, H, D, Nc, m, topk,
                                      Lr, raw0, pos0, W, float(scale), _sink(sink, H), _lay(layout), kv_format,
                                      _lay(_rope(rope)), _p(out), _p(lse_out), _p(ws), 0 if ws is None else ws.numel(),
                                      _stream(stream)))


def csa_sparse_attn_noalloc(q, kv, idx, kv_raw, raw0: int, pos0: int, W: int, scale: float, out, lse_out=None,
                            stream=None, sink=None):
    """csa_sparse_attn with the split partials in the library's static scratch (no workspace, no allocation)."""
    B, Tq, H, D = q.shape
    Nc = kv.shape[1] if kv is not None else 0
    topk = idx.shape[-1] if idx is not None else 0
    Lr = kv_raw.shape[1] if kv_raw is not None else 0
    _check(lib.csa_sparse_attn_noalloc(_p(q), _p(kv), _p(idx), _p(kv_raw), B, Tq, H, D, Nc, topk, Lr, raw0, pos0, W,
                                       float(scale), _sink(sink, H), _p(out), _p(lse_out), _stream(stream)))


def hca_dense_attn(q, kv_h, L: int, mh: int, pos0: int, scale: float, out, lse_out=None, ws=None, stream=None,
                   sink=None, v_h=None, layout=None, kv_format=KV_BF16, rope=None):
    """v_h: separate values (or None); layout (make_layout): variable-length batch (L = capacity) and/or a
    paged pool kv_h of ratio mh; kv_format KV_FP8: FP8 entry rows; rope = (rd, theta): the fused rotary
    embedding."""
    B, Tq, H, D = q.shape
    Nh = -(-L // mh) if (layout is not None and layout.block_table) else kv_h.shape[1]
    need = lib.hca_dense_attn_ws_bytes(B, Tq, H, D, Nh)
    if ws is None:
        ws = workspace(need, q.device)
    if layout is None and v_h is None and kv_format == KV_BF16 and rope is None:
        _check(lib.hca_dense_attn(_p(q), _p(kv_h), B, Tq, H, D, Nh, L, mh, pos0, float(scale), _sink(sink, H),
                                  _p(out), _p(lse_out), _p(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    else:
        _check(lib.hca_dense_attn_ex(_p(q), _p(kv_h), _p(v_h), B, Tq, H, D, Nh, L, mh, pos0, float(scale),
                                     _sink(sink, H), _lay(layout), kv_format, _lay(_rope(rope)), _p(out),
                                     _p(lse_out), _p(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def make_decode_args(*, L, scale, csa_q, q_idx, w_idx, k_idx, kv, kv_raw, idx_dtype, m, topk, W, csa_out,
                     hca_q, kv_h, mh, hca_out, csa_lse=None, hca_lse=None, idx_out=None, csa_sink=None,
                     hca_sink=None, layout=None, q_idx_scale=None, k_idx_scale=None, csa_rope=None,
                     hca_rope=None, kv_format=KV_BF16, ws_persistent=False) -> DecodeArgs:
    """The csa_hca_decode_args_t of one decode step.  ws_persistent: the workspace passed to csa_hca_decode is
    kept across calls with these sizes, zero-filled once before the first (torch.zeros) and written by nothing
    else in between; each call then leaves it ready for the next."""
    B, H, D = csa_q.shape[0], csa_q.shape[-2], csa_q.shape[-1]
    HI, dI = q_idx.shape[-2], q_idx.shape[-1] * (2 if idx_dtype == MXFP4 else 1)
    args = DecodeArgs(B=B, L=L, H=H, D=D, scale=float(scale), csa_q=_p(csa_q), q_idx=_p(q_idx), w_idx=_p(w_idx),
                      k_idx=_p(k_idx), kv=_p(kv), kv_raw=_p(kv_raw), idx_dtype=idx_dtype, HI=HI, dI=dI, m=m,
                      topk=topk, W=W, csa_out=_p(csa_out), csa_lse=_p(csa_lse), idx_out=_p(idx_out),
                      csa_sink=_sink(csa_sink, H), hca_q=_p(hca_q), kv_h=_p(kv_h), mh=mh, hca_out=_p(hca_out),
                      hca_lse=_p(hca_lse), hca_sink=_sink(hca_sink, hca_q.shape[-2]),
                      layout=None if layout is None else ctypes.pointer(layout), q_idx_scale=_p(q_idx_scale),
                      k_idx_scale=_p(k_idx_scale), kv_format=kv_format, ws_persistent=int(bool(ws_persistent)))
    crope, hrope = _rope(csa_rope), _rope(hca_rope)
    if crope is not None:
        args.csa_rope = ctypes.pointer(crope)
    if hrope is not None:
        args.hca_rope = ctypes.pointer(hrope)
    # the struct holds bare device addresses: keep every tensor they point into alive as long as the struct
    args._keep = (csa_q, q_idx, w_idx, k_idx, kv, kv_raw, csa_out, csa_lse, idx_out, csa_sink, hca_q, kv_h, hca_out,
                  hca_lse, hca_sink, layout, q_idx_scale, k_idx_scale, crope, hrope)
    return args


def csa_hca_decode_ws_bytes(args: DecodeArgs) -> int:
    return int(lib.csa_hca_decode_ws_bytes(ctypes.byref(args)))


def csa_hca_decode(args: DecodeArgs, ws=None, stream=None, device=None):
    need = csa_hca_decode_ws_bytes(args)
    if ws is None:
        if args.ws_persistent:
            raise ValueError("ws_persistent needs a caller-kept workspace (zero-filled before the first call)")
        ws = workspace(need, device or torch.device("cuda"))
    _check(lib.csa_hca_decode(ctypes.byref(args), _p(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def csa_rope(x, pos, out=None, rd: int = 64, theta: float = 10000.0, inverse: bool = False, stream=None):
    """Partial rotary embedding of bf16 rows x[..., D] (int16 bit tensor) into out (x itself when None);
    pos: int64 device tensor with one position per group of rows, group = rows / pos.numel()."""
    D = x.shape[-1]
    n = x.numel() // D
    if pos.dtype != torch.int64 or pos.numel() == 0 or n % pos.numel():
        raise ValueError("pos must be a non-empty int64 tensor whose size divides the row count")
    out = x if out is None else out
    _check(lib.csa_rope(_p(x), _p(out), _p(pos), n, D, rd, n // pos.numel(), float(theta), 1 if inverse else 0,
                        _stream(stream)))
    return out


def csa_kv_fp8_encode(x, out=None, stream=None):
    """bf16 KV rows x[..., D] (int16 bits) -> uint8 FP8 rows [..., D + 80]."""
    D = x.shape[-1]
    if out is None:
        out = torch.empty(x.shape[:-1] + (D + 80,), dtype=torch.uint8, device=x.device)
    _check(lib.csa_kv_fp8_encode(_p(x), x.numel() // D, D, _p(out), _stream(stream)))
    return out


def csa_mxfp4_encode(x, codes=None, scales=None, stream=None):
    """bf16 vectors x[..., n] (int16 bits) -> (codes uint8 [..., n/2], scales uint8 [..., n/32]) in MXFP4."""
    n = x.shape[-1]
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (n // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (n // 32,), dtype=torch.uint8, device=x.device)
    _check(lib.csa_mxfp4_encode(_p(x), x.numel() // n, n, _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def csa_debug_fp8_to_bf16(inp, out, stream=None):
    _check(lib.csa_debug_fp8_to_bf16(_p(inp), _p(out), inp.numel(), _stream(stream)))


def prof_enable(on: bool):
    _check(lib.csa_prof_enable(1 if on else 0))


def prof_only(kernel):
    """Record only launches of `kernel` (None: all)."""
    _check(lib.csa_prof_only(kernel.encode() if kernel else None))


def prof_reset():
    _check(lib.csa_prof_reset())


def prof_read(kernel: str):
    t = ctypes.c_double()
    n = ctypes.c_int()
    _check(lib.csa_prof_read(kernel.encode(), ctypes.byref(t), ctypes.byref(n)))
    return t.value, n.value

"""Seeded synthetic inputs for the compressed-attention path.

This module only draws random numbers and encodes them (bf16 / OCP e4m3 via
torch's own conversions); it holds none of the method's arithmetic.  Both the
HIP path's tests/bench and the CPU oracle consume what it returns.

Every tensor has its own PCG64 stream, seeded from (seed, crc32(name)), so a
tensor's values do not depend on which other tensors were drawn or in which
order.  The pages measure nothing on a dataset; these generators stand in for
real activations with the distributions stated per workload (Gaussian scaled
by 1/sqrt(last dim), half-normal indexer head weights, planted high-relevance
keys, and a 1% Student-t(3) heavy-tail mixture).
"""
from __future__ import annotations

import zlib

import numpy as np
import torch

_CHUNK = 1 << 24  # elements per generation chunk (bounds temporary memory)


def rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), zlib.crc32(name.encode())])))


def normal_f32(seed: int, name: str, shape, scale: float = 1.0) -> np.ndarray:
    g = rng(seed, name)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = g.standard_normal(e - s, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape(shape)


def heavy_tail_f32(seed: int, name: str, shape, scale: float = 1.0, frac: float = 0.01, nu: float = 3.0) -> np.ndarray:
    """N(0,1) with probability 1-frac, Student-t(nu) with probability frac, times scale."""
    g = rng(seed, name)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = g.standard_normal(e - s, dtype=np.float32)
        pick = g.random(e - s) < frac
        k = int(pick.sum())
        if k:
            x[pick] = g.standard_t(nu, size=k).astype(np.float32)
        out[s:e] = x
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape(shape)


def half_normal_f32(seed: int, name: str, shape, scale: float = 1.0) -> np.ndarray:
    return np.abs(normal_f32(seed, name, shape, scale))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) using torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn bit patterns (uint8) using torch's conversion (|x| < 448 expected)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encode(x: np.ndarray, dtype: int) -> np.ndarray:
    return to_bf16_bits(x) if dtype == 0 else to_e4m3_bits(x)


def normal_bits(seed, name, shape, scale, dtype=0):
    return encode(normal_f32(seed, name, shape, scale), dtype)


# ---------------------------------------------------------------------------
# Workload builders (return numpy bit arrays; no method arithmetic)
# ---------------------------------------------------------------------------

def indexer_inputs(seed, B, Tq, HI, dI, Nc, dtype=0, planted=0, planted_rho=4.0):
    """q_idx[B][Tq][HI][dI], w_idx[B][Tq][HI] (half-normal / sqrt(HI)), k_idx[B][Nc][dI].

    planted > 0: per sequence, `planted` distinct seeded entries get a key
    aligned with the head-weighted sum of that sequence's first query's heads,
    scaled to planted_rho times a typical key norm, plus small noise."""
    s = 1.0 / np.sqrt(dI)
    qf = normal_f32(seed, "q_idx", (B, Tq, HI, dI), s)
    w = half_normal_f32(seed, "w_idx", (B, Tq, HI), 1.0 / np.sqrt(HI))
    kf = normal_f32(seed, "k_idx", (B, Nc, dI), s)
    planted_idx = None
    if planted:
        g = rng(seed, "planted")
        planted_idx = np.stack([np.sort(g.choice(Nc, size=planted, replace=False)) for _ in range(B)])
        for b in range(B):
            u = (w[b, 0][:, None] * qf[b, 0]).sum(0)
            u = u / np.linalg.norm(u)
            noise = g.standard_normal((planted, dI)).astype(np.float32) * np.float32(0.05 * s)
            kf[b, planted_idx[b]] = (planted_rho * u)[None, :] + noise
    return encode(qf, dtype), w.astype(np.float32), encode(kf, dtype), planted_idx


def attn_inputs(seed, B, Tq, H, D, Nrows, prefix, heavy=False):
    """q[B][Tq][H][D] and rows[B][Nrows][D] as bf16, N(0,1)/sqrt(D) (or the heavy-tail mix)."""
    f = heavy_tail_f32 if heavy else normal_f32
    s = 1.0 / np.sqrt(D)
    q = to_bf16_bits(f(seed, prefix + "q", (B, Tq, H, D), s))
    rows = to_bf16_bits(f(seed, prefix + "rows", (B, Nrows, D), s))
    return q, rows


def sink_logits(seed, H, prefix, scale=2.0):
    """Per-head attention-sink logits (natural log units) as float32, N(0, scale^2)."""
    return normal_f32(seed, prefix + "sink", (H,), scale)


def compress_weights(seed, Dh, D, dI, m, gate_scale=1.0, prefix=""):
    """The weights of compress_inputs alone (same streams): w_kv, w_ik (or None), w_gate, b_slot."""
    wkv = to_bf16_bits(normal_f32(seed, prefix + "w_kv", (D, Dh), 1.0 / np.sqrt(Dh)))
    wik = to_bf16_bits(normal_f32(seed, prefix + "w_ik", (dI, Dh), 1.0 / np.sqrt(Dh))) if dI else None
    gate = normal_f32(seed, prefix + "w_gate", (Dh,), gate_scale / np.sqrt(Dh))
    return wkv, wik, gate, np.zeros(m, np.float32)


def compress_inputs(seed, B, L, Dh, D, dI, m, heavy=False, gate_scale=1.0, prefix=""):
    """hidden[B][L][Dh] bf16, w_kv[D][Dh] bf16, w_ik[dI][Dh] bf16 (or None),
    w_gate[Dh] fp32 ~ N(0,1)/sqrt(Dh) * gate_scale, b_slot[m] fp32 zeros."""
    f = heavy_tail_f32 if heavy else normal_f32
    X = to_bf16_bits(f(seed, prefix + "hidden", (B, L, Dh), 1.0))
    wkv = to_bf16_bits(normal_f32(seed, prefix + "w_kv", (D, Dh), 1.0 / np.sqrt(Dh)))
    wik = to_bf16_bits(normal_f32(seed, prefix + "w_ik", (dI, Dh), 1.0 / np.sqrt(Dh))) if dI else None
    gate = normal_f32(seed, prefix + "w_gate", (Dh,), gate_scale / np.sqrt(Dh))
    bslot = np.zeros(m, np.float32)
    return X, wkv, wik, gate, bslot


# ---------------------------------------------------------------------------
# Device-side generation for the large workloads (same streams, chunked)
# ---------------------------------------------------------------------------

def normal_bits_to_device(seed, name, shape, scale, dtype, device, heavy=False):
    """Generate like normal_bits / heavy-tail bits, chunked, straight into a device tensor.

    Returns a torch tensor of dtype int16 (bf16 bits) or uint8 (e4m3 bits) on `device`;
    identical values to the host generator for the same (seed, name)."""
    g = rng(seed, name)
    n = int(np.prod(shape))
    tdt = torch.int16 if dtype == 0 else torch.uint8
    out = torch.empty(n, dtype=tdt, device=device)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = g.standard_normal(e - s, dtype=np.float32)
        if heavy:
            pick = g.random(e - s) < 0.01
            k = int(pick.sum())
            if k:
                x[pick] = g.standard_t(3.0, size=k).astype(np.float32)
        x *= np.float32(scale)
        t = torch.from_numpy(x)
        t = t.to(torch.bfloat16).view(torch.int16) if dtype == 0 else t.to(torch.float8_e4m3fn).view(torch.uint8)
        out[s:e].copy_(t)
    return out.view(*shape)


def parallel_bits_to_device(seed, name, shape, scale, dtype, device, workers=8, heavy=False):
    """Like normal_bits_to_device but each 2^24-element chunk has its own
    substream (seed, crc32(name), chunk), generated by a thread pool: the large
    caches of the 1M-context workloads fill in seconds.  Values differ from the
    single-stream generators; use the same function on both sides.  heavy: the
    N(0,1) / Student-t(3) mixture of heavy_tail_f32 (1% t draws per chunk)."""
    import concurrent.futures as cf
    n = int(np.prod(shape))
    tdt = torch.int16 if dtype == 0 else torch.uint8
    out = torch.empty(n, dtype=tdt, device=device)
    starts = list(range(0, n, _CHUNK))

    def gen(ci):
        s = starts[ci]
        e = min(n, s + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), zlib.crc32(name.encode()), ci])))
        x = g.standard_normal(e - s, dtype=np.float32)
        if heavy:
            pick = g.random(e - s) < 0.01
            k = int(pick.sum())
            if k:
                x[pick] = g.standard_t(3.0, size=k).astype(np.float32)
        x *= np.float32(scale)
        t = torch.from_numpy(x)
        return t.to(torch.bfloat16).view(torch.int16) if dtype == 0 else t.to(torch.float8_e4m3fn).view(torch.uint8)

    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for ci, t in enumerate(ex.map(gen, range(len(starts)))):
            s = starts[ci]
            out[s:s + t.numel()].copy_(t)
    return out.view(*shape)


def indexer_inputs_to_device(seed, B, Tq, HI, dI, Nc, dtype, device, planted=0, planted_rho=4.0):
    """Indexer inputs of the large batched workloads: q_idx and w_idx as in indexer_inputs (host streams,
    returned as numpy bits and float32), k_idx generated on the device by parallel_bits_to_device.
    planted > 0: per sequence, `planted` distinct seeded entries get the planted key of indexer_inputs
    (aligned with the head-weighted sum of the sequence's first query, planted_rho times a typical key
    norm, plus small noise), written over the generated rows.  Returns (q_bits, w, k_device, planted_idx)."""
    s = 1.0 / np.sqrt(dI)
    qf = normal_f32(seed, "q_idx", (B, Tq, HI, dI), s)
    w = half_normal_f32(seed, "w_idx", (B, Tq, HI), 1.0 / np.sqrt(HI)).astype(np.float32)
    k = parallel_bits_to_device(seed, "k_idx", (B, Nc, dI), s, dtype, device)
    planted_idx = None
    if planted:
        g = rng(seed, "planted")
        planted_idx = np.stack([np.sort(g.choice(Nc, size=planted, replace=False)) for _ in range(B)])
        for b in range(B):
            u = (w[b, 0][:, None] * qf[b, 0]).sum(0)
            u = u / np.linalg.norm(u)
            noise = g.standard_normal((planted, dI)).astype(np.float32) * np.float32(0.05 * s)
            rows = encode((planted_rho * u)[None, :] + noise, dtype)
            rows_t = torch.from_numpy(rows.view(np.int16) if dtype == 0 else rows).to(device)
            k[b, torch.from_numpy(planted_idx[b].astype(np.int64)).to(device)] = rows_t
    return encode(qf, dtype), w, k, planted_idx

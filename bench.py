"""Benchmark: one interleaved CSA + HCA decode pair at 1M context on one MI355X.

Workload (decode_b8_1m): 8 sequences x 1,048,576 raw tokens, one query token
each.  CSA layer: m = 4 -> 262,144 compressed entries per sequence, OCP-e4m3
indexer keys (8 heads x 128), top-k = 1024, 128-token raw window, MQA with
128 query heads x 512.  HCA layer: m' = 128 -> 8,192 entries, dense MQA.
A step is one csa_hca_decode call (indexer scores -> top-k -> sparse attention
-> dense attention) over one batch; inputs are resident in HBM.  Three copies
of every input rotate across steps so that the 256 MB Infinity Cache cannot
serve a step from the previous one.

Prints one JSON line: queries/s (value), the indexer-score kernel's achieved
HBM bandwidth against the 8 TB/s peak (roofline), and the CPU oracle timed on
a bounded sample of the same workload (cpu_baseline), plus a sampled parity
check of that sample against the GPU result.

The metric's second part, indexer prefill TFLOP/s, is measured in the same run
and reported under "indexer_prefill" (workload prefill_8k_on_256k: 8192 new
query tokens at the end of a 262,144-token context, 65,536 bf16 indexer keys,
8 heads x 128, causal at block granularity, top-k = 1024).  A call there is one
csa_index_topk over all 8192 queries; FLOPs are 2 HI dI per (query, visible
entry); its roofline is the contraction kernel against the bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA+HCA decode queries/s & HBM GB/s at 1M ctx; indexer prefill TFLOP/s"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
DOMINANT = "k_score"
PREFILL_DOMINANT = "k_pscore"
PREFILL_KERNELS = ("k_pzero", "k_pnorm", "k_pscore_sample", "k_pthresh", "k_pscore", "k_pselect", "k_pfb_score",
                   "k_pfb_select", "k_pfallback")
KERNELS = ("k_fill", "k_score", "k_collect", "k_select", "k_attn_sparse", "k_attn_dense", "k_combine")


def kernel_source_sha() -> str:
    """Hash of the sources the indexer-score kernel is built from, comments and blank space removed (a
    comment edit does not invalidate counters taken on the same code)."""
    import re
    h = hashlib.sha256()
    for f in ("index_topk.hip", "index_common.h", "common.h", "exact_dot.h"):
        with open(os.path.join(ROOT, "compressed_sparse_kv_compressor_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(per_launch_alg_bytes):
    """HBM traffic of the dominant kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "k_score_decode_b8_1m_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_src_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=20, help="timed calls of the prefill indexer leg (0: skip)")
    ap.add_argument("--compress-steps", type=int, default=10,
                    help="timed calls of the compression + decode-stack leg (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed region, run two plain device copies of MIB MiB (a kernel of known "
                         "traffic to scale rocprofv3 FETCH_SIZE / WRITE_SIZE by)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from compressed_sparse_kv_compressor_amd import binding as b
    from compressed_sparse_kv_compressor_amd import synth
    from compressed_sparse_kv_compressor_amd.configs import DECODE_B8_1M as cfg

    dev = torch.device("cuda:0")
    B, H, D, L, HI, dI = cfg.B, cfg.H, cfg.D, cfg.L, cfg.HI, cfg.dI
    Nc, Nh, W, topk = cfg.Nc, cfg.Nh, cfg.W, cfg.topk
    es = 1 if cfg.idx_dtype == 1 else 2
    t0 = time.time()
    g = synth.parallel_bits_to_device
    base = dict(
        q_idx=g(0, "q_idx", (B, 1, HI, dI), dI ** -0.5, cfg.idx_dtype, dev),
        k_idx=g(0, "k_idx", (B, Nc, dI), dI ** -0.5, cfg.idx_dtype, dev),
        csa_q=g(0, "csa_q", (B, H, D), D ** -0.5, 0, dev),
        kv=g(0, "kv", (B, Nc, D), D ** -0.5, 0, dev),
        raw=g(0, "raw", (B, W, D), D ** -0.5, 0, dev),
        hca_q=g(0, "hca_q", (B, H, D), D ** -0.5, 0, dev),
        kv_h=g(0, "kv_h", (B, Nh, D), D ** -0.5, 0, dev),
    )
    base["w_idx"] = torch.from_numpy(synth.half_normal_f32(0, "w_idx", (B, 1, HI), HI ** -0.5)).to(dev)
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(args.copies - 1)]
    gen_s = time.time() - t0

    outs = []
    dargs = []
    for c in copies:
        csa_out = torch.empty((B, H, D), dtype=torch.int16, device=dev)
        hca_out = torch.empty((B, H, D), dtype=torch.int16, device=dev)
        idx = torch.empty((B, topk), dtype=torch.int32, device=dev)
        outs.append((csa_out, hca_out, idx))
        dargs.append(b.make_decode_args(L=L, scale=cfg.scale, csa_q=c["csa_q"], q_idx=c["q_idx"], w_idx=c["w_idx"],
                                        k_idx=c["k_idx"], kv=c["kv"], kv_raw=c["raw"], idx_dtype=cfg.idx_dtype,
                                        m=cfg.m, topk=topk, W=W, csa_out=csa_out, hca_q=c["hca_q"], kv_h=c["kv_h"],
                                        mh=cfg.mh, hca_out=hca_out, idx_out=idx))
    ws = b.workspace(b.csa_hca_decode_ws_bytes(dargs[0]), dev)
    stream = torch.cuda.current_stream()

    def step(i):
        b.csa_hca_decode(dargs[i % len(dargs)], ws=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: HIP events (on the launch stream) around the dominant kernel only
    b.prof_reset()
    b.prof_only(DOMINANT)
    b.prof_enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    b.prof_enable(False)
    ms, n = b.prof_read(DOMINANT)
    score_us = ms / n * 1000.0 if n else None
    ms_step = elapsed / args.steps * 1e3
    value = B * args.steps / elapsed

    # per-kernel breakdown (separate, untimed pass: events around every launch)
    b.prof_reset()
    b.prof_only(None)
    b.prof_enable(True)
    for i in range(min(args.steps, 30)):
        step(i)
    torch.cuda.synchronize()
    b.prof_enable(False)
    kern = {}
    for name in KERNELS:
        kms, kn = b.prof_read(name)
        if kn:
            kern[name] = round(kms / kn * 1000.0, 2)      # average microseconds per launch
    b.prof_reset()

    # algorithmic bytes (every input read once, outputs written once)
    score_bytes = B * Nc * dI * es + B * HI * dI * es + B * HI * 4
    step_bytes = (score_bytes + B * (topk + W) * D * 2 + 2 * B * H * D * 2 + B * Nh * D * 2 + 2 * B * H * D * 2)
    achieved = score_bytes / (score_us * 1e-6) / 1e9 if score_us else None

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "L": L, "H": H, "D": D, "m": cfg.m, "mh": cfg.mh, "topk": topk,
                   "W": W, "HI": HI, "dI": dI, "idx_dtype": "e4m3" if cfg.idx_dtype else "bf16",
                   "parallelism": "single-gpu", "input_copies": args.copies},
        "step_algorithmic_bytes": step_bytes,
        "step_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "kernel_us_breakdown": kern,
        "roofline": {"bound": "hbm", "kernel": DOMINANT,
                     "achieved": round(achieved, 1) if achieved else None,
                     "kernel_us": round(score_us, 2) if score_us else None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
                     "traffic": load_traffic(score_bytes), "algorithmic_bytes_per_launch": score_bytes},
        "input_gen_s": round(gen_s, 1),
    }

    if args.copy_calibration > 0:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = args.copy_calibration << 20

    if not args.no_cpu_baseline:
        out.update(cpu_leg(cfg, base, outs[0], dev))
    del copies, base, dargs, outs, ws
    torch.cuda.empty_cache()
    if args.prefill_steps > 0:
        out["indexer_prefill"] = prefill_leg(args, dev, cpu=not args.no_cpu_baseline)
    if args.compress_steps > 0:
        out["compress_stack"] = compress_leg(args, dev, cpu=not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


def prefill_leg(args, dev, cpu=True):
    """csa_index_topk over 8192 queries of the chunked-prefill workload."""
    import numpy as np
    import torch

    from compressed_sparse_kv_compressor_amd import binding as b
    from compressed_sparse_kv_compressor_amd import synth
    from compressed_sparse_kv_compressor_amd.configs import PREFILL_8K_256K as pc

    Tq, L, m, HI, dI, topk, Nc, pos0 = pc.Tq, pc.L, pc.m, pc.HI, pc.dI, pc.topk, pc.Nc, pc.pos0
    g = synth.parallel_bits_to_device
    q_idx = g(0, "prefill_q_idx", (1, Tq, HI, dI), dI ** -0.5, 0, dev)
    k_idx = g(0, "prefill_k_idx", (1, Nc, dI), dI ** -0.5, 0, dev)
    w_idx = torch.from_numpy(synth.half_normal_f32(0, "prefill_w_idx", (1, Tq, HI), HI ** -0.5)).to(dev)
    idx = torch.empty((1, Tq, topk), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, Tq), dtype=torch.int32, device=dev)
    ws = b.workspace(b.lib.csa_index_topk_ws_bytes(1, Tq, HI, dI, Nc, topk, 0), dev)
    stream = torch.cuda.current_stream()

    def call():
        b.csa_index_topk(q_idx, w_idx, k_idx, 0, L, m, pos0, topk, idx, cnt, ws=ws, stream=stream)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    b.prof_reset()
    b.prof_only(PREFILL_DOMINANT)
    b.prof_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.prefill_steps):
        call()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    b.prof_enable(False)
    kms, kn = b.prof_read(PREFILL_DOMINANT)
    b.prof_reset()
    b.prof_only(None)
    b.prof_enable(True)
    for _ in range(min(args.prefill_steps, 10)):
        call()
    torch.cuda.synchronize()
    b.prof_enable(False)
    kern = {}
    for name in PREFILL_KERNELS:
        t, n = b.prof_read(name)
        if n:
            kern[name] = round(t / n * 1000.0, 2)
    b.prof_reset()

    nv = np.minimum((pos0 + np.arange(Tq) + 1) // m, Nc)
    flops = 2.0 * HI * dI * float(nv.sum())            # visible (query, entry) pairs
    ms_call = el / args.prefill_steps * 1e3
    k_us = kms / kn * 1000.0 if kn else None
    res = {
        "workload": pc.name, "Tq": Tq, "L": L, "Nc": Nc, "HI": HI, "dI": dI, "topk": topk, "dtype": "bf16",
        "calls": args.prefill_steps, "ms_per_call": round(ms_call, 4),
        "value": round(flops / (ms_call * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
        "algorithmic_flops_per_call": flops,
        "frac_of_bf16_peak": round(flops / (ms_call * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        "kernel_us_breakdown": kern,
        "roofline": {"bound": "mfma", "kernel": PREFILL_DOMINANT,
                     "achieved": round(flops / (k_us * 1e-6) / 1e12, 1) if k_us else None,
                     "kernel_us": round(k_us, 2) if k_us else None, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / (k_us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
                     if k_us else None, "traffic": None},
    }
    if cpu:
        res.update(prefill_cpu_leg(pc, q_idx, w_idx, k_idx, idx))
    del q_idx, k_idx, w_idx, ws
    torch.cuda.empty_cache()
    res["sparse_attn"] = prefill_attn_leg(args, dev, pc, idx)
    return res


COMPRESS_KERNELS = ("k_pool2", "k_pool", "k_gemm2", "k_g2reduce", "k_gemm", "k_fill", "k_score", "k_collect", "k_select", "k_attn_sparse",
                    "k_attn_dense", "k_combine")


def compress_leg(args, dev, cpu=True):
    """Compression of 4 x 64K tokens of hidden 4096 into the CSA (m = 4, indexer keys, window) and HCA
    (m' = 128) caches, then a CSA, HCA, CSA, HCA stack of one-token decodes against them."""
    import numpy as np
    import torch

    from compressed_sparse_kv_compressor_amd import binding as b
    from compressed_sparse_kv_compressor_amd import synth
    from compressed_sparse_kv_compressor_amd.configs import COMPRESS_B4_64K as cc

    B, L, Dh, D, dI, HI, m, mh, W, H, topk = cc.B, cc.L, cc.Dh, cc.D, cc.dI, cc.HI, cc.m, cc.mh, cc.W, cc.H, cc.topk
    Nc, Nh = -(-L // m), -(-L // mh)
    t0 = time.time()
    X = synth.parallel_bits_to_device(0, "c5_hidden", (B, L, Dh), 1.0, 0, dev, heavy=True)
    tod = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    wkv, wik, gate, bslot = (tod(a) for a in synth.compress_weights(0, Dh, D, dI, m, prefix="c5_csa_"))
    hw = synth.compress_weights(0, Dh, D, 0, mh, prefix="c5_hca_")
    wkv_h, gate_h, bslot_h = tod(hw[0]), tod(hw[2]), tod(hw[3])
    gen_s = time.time() - t0
    kv = torch.empty((B, Nc, D), dtype=torch.int16, device=dev)
    ik = torch.empty((B, Nc, dI), dtype=torch.int16, device=dev)
    win = torch.empty((B, W, D), dtype=torch.int16, device=dev)
    kv_h = torch.empty((B, Nh, D), dtype=torch.int16, device=dev)
    ws = b.workspace(b.lib.csa_hca_compress_ws_bytes(B, L, Dh, D, dI, m, W, mh), dev)
    stream = torch.cuda.current_stream()

    def compress():
        b.csa_hca_compress(X, wkv, wik, gate, bslot, m, W, kv, ik, win, wkv_h, gate_h, bslot_h, mh, kv_h,
                           ik_dtype=0, ws=ws, stream=stream)

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def breakdown(fn, n):
        b.prof_reset()
        b.prof_only(None)
        b.prof_enable(True)
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        b.prof_enable(False)
        kern = {}
        for name in COMPRESS_KERNELS:
            t, k = b.prof_read(name)
            if k:
                kern[name] = {"us_per_call": round(t / n * 1000.0, 2), "launches_per_call": k // n}
        b.prof_reset()
        return kern

    ms_c = timed(compress, args.compress_steps)
    kern_c = breakdown(compress, min(args.compress_steps, 5))
    x_bytes = B * L * Dh * 2
    w_bytes = (2 * D + dI) * Dh * 2 + 2 * Dh * 4
    o_bytes = (B * Nc * (D + dI) + B * W * D + B * Nh * D) * 2
    c_bytes = x_bytes + w_bytes + o_bytes                      # hidden read once for both caches
    c_flops = 2.0 * 2 * Dh * B * L + 2.0 * Dh * (B * Nc * (D + dI) + B * Nh * D + B * W * D)
    pool = kern_c.get("k_pool2")
    pooled_bytes = (B * Nc + B * Nh) * Dh * 2
    res = {
        "workload": cc.name, "B": B, "L": L, "Dh": Dh, "D": D, "dI": dI, "m": m, "mh": mh, "W": W,
        "hidden": "N(0,1) with 1% Student-t(3), bf16", "input_gen_s": round(gen_s, 1),
        "compress": {
            "calls": args.compress_steps, "ms_per_call": round(ms_c, 4),
            "algorithmic_bytes": c_bytes, "algorithmic_flops": c_flops,
            "GBps": round(c_bytes / (ms_c * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(c_bytes / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "kernel_us_breakdown": kern_c,
            "roofline": {"bound": "hbm", "kernel": "k_pool2",
                         "achieved": round((x_bytes + pooled_bytes) / (pool["us_per_call"] * 1e-6) / 1e9, 1)
                         if pool else None,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "algorithmic_bytes_per_launch": x_bytes + pooled_bytes,
                         "note": "one pass over the hidden rows pools both caches; bytes = hidden read once + "
                                 "pooled rows written once"},
        },
    }
    if cpu:
        res["compress"]["parity_sample"] = compress_parity(cc, X, (wkv, wik, gate, bslot), (wkv_h, gate_h, bslot_h),
                                                           kv, ik, win, kv_h)

    # the decode stack: CSA, HCA, CSA, HCA (two csa_hca_decode calls), one query per sequence, against the caches
    g = synth.parallel_bits_to_device
    pairs = []
    for layer in range(cc.layers // 2):
        pf = f"c5_l{layer}_"
        pq = dict(
            q_idx=g(0, pf + "q_idx", (B, 1, HI, dI), dI ** -0.5, 0, dev, heavy=True),
            csa_q=g(0, pf + "csa_q", (B, H, D), D ** -0.5, 0, dev, heavy=True),
            hca_q=g(0, pf + "hca_q", (B, H, D), D ** -0.5, 0, dev, heavy=True),
            w_idx=torch.from_numpy(synth.half_normal_f32(0, pf + "w_idx", (B, 1, HI), HI ** -0.5)).to(dev),
            csa_out=torch.empty((B, H, D), dtype=torch.int16, device=dev),
            hca_out=torch.empty((B, H, D), dtype=torch.int16, device=dev),
            idx=torch.empty((B, topk), dtype=torch.int32, device=dev))
        pq["args"] = b.make_decode_args(L=L, scale=D ** -0.5, csa_q=pq["csa_q"], q_idx=pq["q_idx"], w_idx=pq["w_idx"],
                                        k_idx=ik, kv=kv, kv_raw=win, idx_dtype=0, m=m, topk=topk, W=W,
                                        csa_out=pq["csa_out"], hca_q=pq["hca_q"], kv_h=kv_h, mh=mh,
                                        hca_out=pq["hca_out"], idx_out=pq["idx"])
        pairs.append(pq)
    dws = b.workspace(max(b.csa_hca_decode_ws_bytes(p["args"]) for p in pairs), dev)

    def stack():
        for p in pairs:
            b.csa_hca_decode(p["args"], ws=dws, stream=stream)

    steps = max(10, 10 * args.compress_steps)
    ms_s = timed(stack, steps)
    kern_s = breakdown(stack, min(steps, 20))
    s_bytes = 0
    for _ in pairs:
        s_bytes += B * Nc * dI * 2 + B * HI * (dI * 2 + 4) + B * (topk + W) * D * 2 + B * Nh * D * 2 + 4 * B * H * D * 2
    res["decode_stack"] = {
        "layers": cc.layers, "H": H, "topk": topk, "idx_dtype": "bf16", "calls": steps,
        "us_per_stack": round(ms_s * 1e3, 2), "queries_per_s": round(B / (ms_s * 1e-3), 1),
        "algorithmic_bytes": s_bytes, "GBps": round(s_bytes / (ms_s * 1e-3) / 1e9, 1),
        "kernel_us_breakdown": kern_s,
    }
    del X, kv, ik, win, kv_h, ws, dws, pairs
    torch.cuda.empty_cache()
    return res


def compress_parity(cc, X, wc, wh, kv, ik, win, kv_h):
    """Oracle check of a few compressed rows of sequence 0 (CSA entries 0-1 and the last, the first HCA
    entry, the window rows): max row-relative error against the 2e-2 bar."""
    import numpy as np
    import torch

    import oracle

    host = lambda t: t.cpu().numpy().view(np.uint16) if t.dtype == torch.int16 else t.cpu().numpy()
    m, mh, W, L = cc.m, cc.mh, cc.W, cc.L
    Nc = -(-L // m)
    wkv, wik, gate, bslot = (host(t) for t in wc)
    wkv_h, gate_h, bslot_h = (host(t) for t in wh)

    def bf(t):
        return (t.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def rel(got, want):
        got = got.reshape(-1, want.shape[-1])
        want = want.reshape(-1, want.shape[-1])
        return float((np.abs(got - want).max(1) / np.abs(want).max(1)).max())

    err = {}
    t0 = time.perf_counter()
    for j in (0, 1, Nc - 1):
        xs = host(X[0:1, j * m:(j + 1) * m])
        okv, oik, _ = oracle.compress(xs, wkv, wik, gate, bslot, m)
        err[f"csa_kv_{j}"] = rel(bf(kv[0, j]), okv)
        err[f"csa_ik_{j}"] = rel(bf(ik[0, j]), oik)
    xs = host(X[0:1, 0:mh])
    okh, _, _ = oracle.compress(xs, wkv_h, None, gate_h, bslot_h, mh)
    err["hca_kv_0"] = rel(bf(kv_h[0, 0]), okh)
    xs = host(X[0:1, L - W:L])
    _, _, ow = oracle.compress(xs, wkv, None, gate, bslot, m, W=W)
    err["window"] = rel(bf(win[0]), ow)
    return {"max_row_rel_err": err, "tolerance": 2e-2, "ok": bool(max(err.values()) <= 2e-2),
            "oracle_s": round(time.perf_counter() - t0, 2)}


def prefill_attn_leg(args, dev, pc, idx):
    """csa_sparse_attn over the same 8192 queries: 64 heads x 512, the selected 1024 entries plus the
    128-token window of each query (FLOPs 4 H D (k + W) per query)."""
    import torch

    from compressed_sparse_kv_compressor_amd import binding as b
    from compressed_sparse_kv_compressor_amd import synth

    Tq, H, D, W, topk, Nc, pos0 = pc.Tq, pc.H, pc.D, pc.W, pc.topk, pc.Nc, pc.pos0
    g = synth.parallel_bits_to_device
    q = g(0, "prefill_q", (1, Tq, H, D), D ** -0.5, 0, dev)
    kv = g(0, "prefill_kv", (1, Nc, D), D ** -0.5, 0, dev)
    Lr, raw0 = Tq + W - 1, pos0 - (W - 1)
    raw = g(0, "prefill_raw", (1, Lr, D), D ** -0.5, 0, dev)
    out = torch.empty((1, Tq, H, D), dtype=torch.int16, device=dev)
    ws = b.workspace(b.lib.csa_sparse_attn_ws_bytes(1, Tq, H, D, topk, W), dev)
    stream = torch.cuda.current_stream()

    def call():
        b.csa_sparse_attn(q, kv, idx, raw, raw0, pos0, W, pc.D ** -0.5, out, ws=ws, stream=stream)

    call()
    torch.cuda.synchronize()
    n = max(1, min(args.prefill_steps, 10))
    t0 = time.perf_counter()
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / n * 1e3
    flops = 4.0 * H * D * (topk + W) * Tq
    # partial rotary embedding of the same queries (rd = 64, one position per query): one read and one write
    # of every query row, out of place
    qo = torch.empty_like(q)
    qpos = torch.arange(pos0, pos0 + Tq, dtype=torch.int64, device=dev)
    b.csa_rope(q, qpos, qo, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        b.csa_rope(q, qpos, qo, stream=stream)
    torch.cuda.synchronize()
    rms = (time.perf_counter() - t0) / n * 1e3
    rbytes = 2.0 * q.numel() * 2 + qpos.numel() * 8
    rope = {"workload": f"rope_{Tq}q_{H}h_{D}", "rd": 64, "calls": n, "ms_per_call": round(rms, 4),
            "value": round(rbytes / (rms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(rbytes / (rms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_call": rbytes}
    del qo
    return {"H": H, "D": D, "W": W, "calls": n, "ms_per_call": round(ms, 4), "rope": rope,
            "value": round(flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
            "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_call": flops, "index_source": "the indexer leg's selection"}


def prefill_cpu_leg(pc, q_idx, w_idx, k_idx, gidx, rows=(0, 4095, 8191)):
    """The oracle on a few query rows of the prefill workload (bounded CPU sample),
    and a bit-exact check of the GPU's selection for those rows."""
    import numpy as np

    import oracle

    q = q_idx.cpu().numpy().view(np.uint16)
    w = w_idx.cpu().numpy()
    k = k_idx.cpu().numpy().view(np.uint16)
    g = gidx.cpu().numpy()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    ok = True
    flops = 0.0
    for t in rows:
        want, _, _, nv = oracle.index_topk(q[:, t:t + 1], w[:, t:t + 1], k, pc.L, pc.m, pc.pos0 + t, pc.topk)
        flops += 2.0 * pc.HI * pc.dI * float(nv[0, 0])
        ok = ok and bool(np.array_equal(want[0, 0], g[0, t]))
    el = time.perf_counter() - t0
    return {
        "cpu_baseline": {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                         "sample": f"query rows {list(rows)} of {pc.name}: exact indexer scores over all visible "
                                   f"entries + top-{pc.topk}", "seconds": round(el, 2)},
        "parity_sample": {"rows": list(rows), "topk_bit_exact": ok},
    }


def cpu_leg(cfg, x, gpu_out, dev):
    """The oracle on one sequence of the same workload (bounded CPU sample) and
    a parity check of the GPU's result for that sequence."""
    import numpy as np
    import torch

    import oracle

    B, H, D, L, W, topk = cfg.B, cfg.H, cfg.D, cfg.L, cfg.W, cfg.topk
    bsel = 0
    u16 = lambda t: t.cpu().numpy().view(np.uint16)
    dt = cfg.idx_dtype
    kbits = (lambda t: t.cpu().numpy()) if dt == 1 else u16
    q_idx = kbits(x["q_idx"][bsel:bsel + 1])
    w_idx = x["w_idx"][bsel:bsel + 1].cpu().numpy()
    k_idx = kbits(x["k_idx"][bsel:bsel + 1])
    csa_q = u16(x["csa_q"][bsel:bsel + 1]).reshape(1, 1, H, D)
    raw = u16(x["raw"][bsel:bsel + 1])
    hca_q = u16(x["hca_q"][bsel:bsel + 1]).reshape(1, 1, H, D)
    kv_h = u16(x["kv_h"][bsel:bsel + 1])
    p = L - 1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    idx, cnt, _, _ = oracle.index_topk(q_idx, w_idx, k_idx, L, cfg.m, p, topk, dt)
    t_index = time.perf_counter() - t0
    rows = torch.from_numpy(idx[0, 0].astype(np.int64)).to(dev)
    kv_sel = u16(x["kv"][bsel].index_select(0, rows)).reshape(1, topk, D)
    local = np.arange(topk, dtype=np.int32).reshape(1, 1, topk)
    t1 = time.perf_counter()
    o_csa, _ = oracle.sparse_attn(csa_q, kv_sel, local, raw, L - W, p, W, cfg.scale)
    o_hca, _ = oracle.dense_attn(hca_q, kv_h, L, cfg.mh, p, cfg.scale)
    t_attn = time.perf_counter() - t1
    total = t_index + t_attn

    csa_out, hca_out, gidx = gpu_out
    g_idx = gidx[bsel].cpu().numpy()

    def rel(got, want):
        g = (got.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        g = g.reshape(-1, D)
        o = want.reshape(-1, D)
        return float((np.abs(g - o).max(1) / np.abs(o).max(1)).max())

    return {
        "cpu_baseline": {"value": round(1.0 / total, 4), "unit": "queries/s", "cores": threads, "kind": "oracle",
                         "sample": f"sequence 0 of {cfg.name}: indexer over all {cfg.Nc} entries + top-{topk} + "
                                   f"CSA attention ({topk}+{W} rows) + HCA attention ({cfg.Nh} rows), 1 query",
                         "seconds": round(total, 2), "index_s": round(t_index, 2), "attn_s": round(t_attn, 2)},
        "parity_sample": {"topk_bit_exact": bool(np.array_equal(g_idx, idx[0, 0])),
                          "csa_max_row_rel_err": rel(csa_out[bsel], o_csa), "hca_max_row_rel_err": rel(hca_out[bsel], o_hca),
                          "tolerance": 2e-2},
    }


if __name__ == "__main__":
    main()

"""Workload shapes for the compressed-attention path.

Five named workloads (the shapes the method is measured on) plus down-scaled
variants with the same structure for parity tests that the CPU oracle can
finish in seconds.  Names describe the workload, not where it came from.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class DecodeCfg:
    """One interleaved CSA + HCA layer pair, one query token per sequence (p = L-1)."""
    name: str
    B: int
    L: int
    H: int
    D: int
    HI: int
    dI: int
    m: int
    mh: int
    topk: int
    W: int
    idx_dtype: int = 0      # 0 = bf16, 1 = OCP e4m3
    planted: int = 0        # planted high-relevance keys per sequence
    hca: bool = True        # run the HCA layer too

    @property
    def Nc(self):
        return (self.L + self.m - 1) // self.m

    @property
    def Nh(self):
        return (self.L + self.mh - 1) // self.mh

    @property
    def scale(self):
        return self.D ** -0.5


@dataclass(frozen=True)
class PrefillCfg:
    """Chunked prefill: Tq new query tokens at the end of an L-token context."""
    name: str
    L: int
    Tq: int
    H: int
    D: int
    HI: int
    dI: int
    m: int
    topk: int
    W: int

    @property
    def Nc(self):
        return (self.L + self.m - 1) // self.m

    @property
    def pos0(self):
        return self.L - self.Tq


@dataclass(frozen=True)
class CompressCfg:
    """Compression of B x L raw tokens (hidden Dh) into CSA (m) and HCA (mh) caches,
    then a stack of alternating CSA / HCA one-token decodes against them."""
    name: str
    B: int
    L: int
    Dh: int
    D: int
    dI: int
    HI: int
    m: int
    mh: int
    topk: int
    W: int
    H: int
    layers: int


# Single-sequence decode, 4K context, hidden 1024, 16 heads x 128, indexer 4 x 64.
DECODE_4K = DecodeCfg("decode_b1_4k", B=1, L=4096, H=16, D=128, HI=4, dI=64, m=4, mh=128,
                      topk=64, W=128)
# Batched CSA decode: 32 x 128K, 64 heads x 512, indexer 8 x 128 bf16, k = 512, 16 planted keys.
DECODE_B32_128K = DecodeCfg("decode_b32_128k", B=32, L=131072, H=64, D=512, HI=8, dI=128, m=4,
                            mh=128, topk=512, W=128, planted=16, hca=False)
# V4-Pro-shaped decode at 1M: 8 x 1,048,576, 128 heads x 512, e4m3 indexer keys 8 x 128, k = 1024.
DECODE_B8_1M = DecodeCfg("decode_b8_1m", B=8, L=1048576, H=128, D=512, HI=8, dI=128, m=4,
                         mh=128, topk=1024, W=128, idx_dtype=1)
# Chunked prefill: 8192 queries at the end of a 262,144-token context (65,536 entries).
PREFILL_8K_256K = PrefillCfg("prefill_8k_on_256k", L=262144, Tq=8192, H=64, D=512, HI=8, dI=128,
                             m=4, topk=1024, W=128)
# Compression of 4 x 64K tokens of hidden 4096 + a 4-layer alternating decode stack.
COMPRESS_B4_64K = CompressCfg("compress_b4_64k_stack4", B=4, L=65536, Dh=4096, D=512, dI=128, HI=8,
                              m=4, mh=128, topk=1024, W=128, H=128, layers=4)

WORKLOADS = {c.name: c for c in (DECODE_4K, DECODE_B32_128K, DECODE_B8_1M, PREFILL_8K_256K, COMPRESS_B4_64K)}


def scaled_decode(cfg: DecodeCfg, L: int, B: int | None = None, topk: int | None = None) -> DecodeCfg:
    """Same structure at a smaller context (for oracle-checkable parity)."""
    return replace(cfg, name=f"{cfg.name}_L{L}", L=L, B=cfg.B if B is None else B,
                   topk=cfg.topk if topk is None else topk)

"""csa_sparse_attn_noalloc (partials in the library's static scratch) against csa_sparse_attn (partials in a
caller workspace): the same kernels and split plan, so the outputs must be bitwise equal.  Two calls in a
row on the same GPU, the second with a smaller input, so the second runs on the scratch the first left
behind; and a call whose partials exceed the static size is refused before anything is launched."""
import numpy as np
import pytest
import torch

from compressed_sparse_kv_compressor_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_sparse_kv_compressor_amd import binding
    return binding


def case(seed, B, Tq, H, D, Nc, topk, W):
    q, kv = synth.attn_inputs(seed, B, Tq, H, D, Nc, "na_")
    _, raw = synth.attn_inputs(seed, B, 1, H, D, Tq + W, "na_raw_")
    g = np.random.default_rng(seed)
    pos0 = Nc * 4 - Tq
    idx = np.stack([np.stack([np.sort(g.choice(Nc, topk, replace=False)) for _ in range(Tq)]) for _ in range(B)])
    idx = idx.astype(np.int32)
    idx[:, :, -3:] = -1                       # a few unused slots
    t = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(DEV)
    return t(q), t(kv), t(idx), t(raw), pos0 - W + 1, pos0


def run_both(b, args, W, scale, H, sink=None):
    q, kv, idx, raw, raw0, pos0 = args
    B, Tq, _, D = q.shape
    outs = []
    for fn in (b.csa_sparse_attn, b.csa_sparse_attn_noalloc):
        out = torch.full((B, Tq, H, D), -1, dtype=torch.int16, device=DEV)
        lse = torch.full((B, Tq, H), float("nan"), dtype=torch.float32, device=DEV)
        fn(q, kv, idx, raw, raw0, pos0, W, scale, out, lse, sink=sink)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("H", [128, 64, 16])
def test_noalloc_matches_workspace_call_twice(b, H):
    D = 512 if H >= 64 else 128
    big = case(1, 8, 1, H, D, 20000, 1024, 128)        # many splits: the partials fill part of the scratch
    small = case(2, 2, 3, H, D, 3000, 300, 64)         # a second, smaller call reuses the scratch
    assert b.lib.csa_sparse_attn_ws_bytes(8, 1, H, D, 1024, 128) > 0
    for args, W in ((big, 128), (small, 64)):
        (o1, l1), (o2, l2) = run_both(b, args, W, D ** -0.5, H)
        assert torch.equal(o1, o2)
        assert torch.equal(l1, l2)


def test_noalloc_with_sink_matches(b):
    H, D = 128, 512
    args = case(3, 4, 1, H, D, 8000, 512, 128)
    sink = torch.from_numpy(synth.sink_logits(3, H, "na_")).to(DEV)
    (o1, l1), (o2, l2) = run_both(b, args, 128, D ** -0.5, H, sink=sink)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_refuses_oversized_partials(b):
    # 64 queries x 128 heads x 512 with many splits needs far more than the static scratch
    H, D, B, Tq, topk, W = 128, 512, 64, 1, 4096, 1024
    need = b.lib.csa_sparse_attn_ws_bytes(B, Tq, H, D, topk, W)
    assert need > (64 << 20)
    q = torch.zeros((B, Tq, H, D), dtype=torch.int16, device=DEV)
    kv = torch.zeros((B, 5000, D), dtype=torch.int16, device=DEV)
    idx = torch.zeros((B, Tq, topk), dtype=torch.int32, device=DEV)
    raw = torch.zeros((B, W, D), dtype=torch.int16, device=DEV)
    out = torch.zeros((B, Tq, H, D), dtype=torch.int16, device=DEV)
    with pytest.raises(b.CsaError, match="CSA_ERR_UNSUPPORTED"):
        b.csa_sparse_attn_noalloc(q, kv, idx, raw, 20000 - W, 20000 - 1, W, 0.04, out)
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0              # nothing was launched

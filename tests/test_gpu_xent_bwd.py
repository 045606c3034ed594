"""Parity of the vocab-parallel CE backward (vocab_parallel_xent_bwd and the
log-sum-exp merge, through the C ABI) with the fp64 oracle.

The device pipeline runs end to end: every rank's forward partials, the
log-sum-exp merge (shard_partial_sum XENT_LSE), then each rank's backward
from that lse.  The oracle takes the same inputs through its own forward
partials and merge.  Small cases compare every element; the 8.3B-shape slice
(M = 8192, h = 3072, V_r = 6400) is compared on sampled token rows of dH_r
and on contiguous blocks of vocabulary rows of dE_r (each is itself a slice,
so the oracle computes it exactly).  Tolerance: max|gpu - ref| / max|ref| <=
2e-2 per output (bf16 in and out, fp32 accumulation, G rounded to bf16).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, f64, step
from logit_gemm_shard_amd import binding as lgs
from logit_gemm_shard_amd import synth
from logit_gemm_shard_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
xo = oracle.xent


def sync():
    torch.cuda.synchronize()


def device_lse(H, E, y, b, s, t):
    """Every rank's forward partials, then the log-sum-exp merge."""
    M, h = H.shape
    V = E.shape[0]
    Vr = V // t
    stats = torch.empty(t, 3, M, dtype=F32, device=H.device)
    for r in range(t):
        lgs.vocab_parallel_xent_fwd(b, s, h, V, t, r, H, E[r * Vr:(r + 1) * Vr], y, stats[r, 0], stats[r, 1],
                                    stats[r, 2])
    lse = torch.empty(M, dtype=F32, device=H.device)
    lgs.shard_partial_sum("xent_lse", t, M, stats, 3 * M, lse)
    return lse


def oracle_lse(H64, E64, y, t):
    V = E64.shape[0]
    Vr = V // t
    parts = [xo.shard_partials(H64, E64[r * Vr:(r + 1) * Vr], y, r * Vr) for r in range(t)]
    return xo.merge_lse(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


SMALL = [  # (b, s, h, V, t): ragged token counts, slices of several tiles with tails
    (1, 300, 72, 2 * 704, 2),
    (2, 129, 136, 4 * 520, 4),
    (1, 64, 64, 8 * 136, 8),
    (1, 520, 264, 2 * 1288, 2),
    (2, 1000, 136, 24640, 1),  # wide enough that the logit GEMM splits its columns over two launches
    (1, 1, 64, 2 * 160, 2),    # a single token (dE's GEMM has K = 1)
    (1, 9, 64, 2 * 160, 2),
]


@pytest.mark.parametrize("weighted", [True, False], ids=["dloss", "unit"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_xent_bwd_all_ranks(shape, weighted):
    b, s, h, V, t = shape
    M, Vr = b * s, V // t
    d = dev()
    H, E = synth.small(41 + h, (M, h), (V, h), dtype="bf16")
    E = (E.float() * 0.5).to(BF16)
    g = torch.Generator().manual_seed(h)
    y = torch.randint(0, V, (M,), generator=g, dtype=torch.int64).to(torch.int32)
    w = torch.randn(M, generator=g) if weighted else None
    H64, E64, yn = f64(H), f64(E), y.numpy().astype(np.int64)
    w64 = None if w is None else f64(w)
    Hd, Ed, yd = H.to(d), E.to(d), y.to(d)
    wd = None if w is None else w.to(d)
    step(f"xent bwd {shape} weighted={weighted}: lse merge + every rank's backward")
    lse = device_lse(Hd, Ed, yd, b, s, t)
    dHp = torch.empty(t, M, h, dtype=BF16, device=d)
    dE = torch.empty(V, h, dtype=BF16, device=d)
    for r in range(t):
        lgs.vocab_parallel_xent_bwd(b, s, h, V, t, r, Hd, Ed[r * Vr:(r + 1) * Vr], yd, lse, dHp[r],
                                    dE[r * Vr:(r + 1) * Vr], dloss=wd)
    dH = torch.empty(M, h, dtype=BF16, device=d)
    lgs.shard_partial_sum("sum", t, M * h, dHp, M * h, dH)
    sync()
    rlse = oracle_lse(H64, E64, yn, t)
    assert_close("lse (merged)", lse, rlse, F32)
    for r in range(t):
        ref = xo.shard_backward(H64, E64[r * Vr:(r + 1) * Vr], yn, r * Vr, rlse, w64)
        assert_close(f"dH_{r} (partial)", dHp[r], ref["dH"], BF16)
        assert_close(f"dE_{r}", dE[r * Vr:(r + 1) * Vr], ref["dE"], BF16)
    full = xo.xent_backward(H64, E64, yn, w64)
    assert_close("sum_r dH_r vs unsplit dH", dH, full["dH"], BF16)
    assert_close("stacked dE_r vs unsplit dE", dE, full["dE"], BF16)


def test_xent_bwd_zero_embedding_closed_form():
    """E = 0: lse = ln V, G = (1/V - onehot) * w, dH = 0 and
    dE_j = sum_k w_k (1/V - [y_k = j]) H_k."""
    b, s, h, V, t = 1, 96, 64, 4 * 256, 4
    M, Vr = b * s, V // t
    d = dev()
    H = synth.small(3, (M, h), dtype="bf16")[0]
    E = torch.zeros(V, h, dtype=BF16)
    y = (torch.arange(M, dtype=torch.int32) * 37) % V
    step("xent bwd with E = 0")
    Hd, Ed, yd = H.to(d), E.to(d), y.to(d)
    lse = device_lse(Hd, Ed, yd, b, s, t)
    dH = torch.empty(t, M, h, dtype=BF16, device=d)
    dE = torch.empty(V, h, dtype=BF16, device=d)
    for r in range(t):
        lgs.vocab_parallel_xent_bwd(b, s, h, V, t, r, Hd, Ed[r * Vr:(r + 1) * Vr], yd, lse, dH[r],
                                    dE[r * Vr:(r + 1) * Vr])
    sync()
    assert np.abs(lse.cpu().numpy() - np.log(V)).max() < 1e-6 * np.log(V)
    assert (dH.float() == 0).all()
    yn = y.numpy()
    want = np.full((M, V), 1.0 / V)
    want[np.arange(M), yn] -= 1.0
    assert_close("dE (E = 0)", dE, want.T @ f64(H), BF16)


def test_xent_bwd_strided_outputs_equal_dense():
    """dH_r / dE_r written into wider buffers (ld > h) hold the same values."""
    b, s, h, V, t = 1, 200, 128, 2 * 384, 2
    M, Vr = b * s, V // t
    d = dev()
    H, E = synth.small(8, (M, h), (V, h), dtype="bf16")
    y = torch.randint(0, V, (M,), generator=torch.Generator().manual_seed(5)).to(torch.int32)
    Hd, Ed, yd = H.to(d), E.to(d), y.to(d)
    step("xent bwd into strided outputs")
    lse = device_lse(Hd, Ed, yd, b, s, t)
    dH = torch.empty(M, h, dtype=BF16, device=d)
    dE = torch.empty(Vr, h, dtype=BF16, device=d)
    lgs.vocab_parallel_xent_bwd(b, s, h, V, t, 1, Hd, Ed[Vr:], yd, lse, dH, dE)
    bigH = torch.full((M, h + 24), float("nan"), dtype=BF16, device=d)
    bigE = torch.full((Vr, h + 8), float("nan"), dtype=BF16, device=d)
    lgs.vocab_parallel_xent_bwd(b, s, h, V, t, 1, Hd, Ed[Vr:], yd, lse, bigH[:, 8:8 + h], bigE[:, :h])
    sync()
    assert torch.equal(bigH[:, 8:8 + h], dH) and torch.equal(bigE[:, :h], dE)
    assert torch.isnan(bigH[:, :8]).all() and torch.isnan(bigH[:, 8 + h:]).all()
    assert torch.isnan(bigE[:, h:]).all()


def test_xent_bwd_8p3b_full():
    """The 8.3B-shape slice (rank 0 and rank 7 of t = 8) in the benchmark's
    launch configuration, dloss = 1/M (the mean loss): every element of
    dH_r and dE_r, and the merged lse of every token."""
    w = WORKLOADS["xent_8p3b"]
    d = dev()
    H, E, y = synth.xent_inputs(w)
    Vr = w.v_r
    Hd, Ed, yd = H.to(d), E.to(d), y.to(d)
    dl = torch.full((w.M,), 1.0 / w.M, dtype=F32, device=d)
    step("xent_8p3b: every rank's forward + lse merge at full size")
    lse = device_lse(Hd, Ed, yd, w.b, w.s, w.t)
    H64, yn = f64(H), y.numpy().astype(np.int64)
    step("xent_8p3b: oracle lse over the whole vocabulary (host, fp64)")
    E64 = f64(E)
    rlse = oracle_lse(H64, E64, yn, w.t)
    assert_close("lse (all tokens)", lse.cpu(), rlse, F32)
    w64 = np.full(w.M, 1.0 / w.M)
    for r in (0, w.t - 1):
        a = r * Vr
        step(f"xent_8p3b: rank {r} backward at full size")
        dH = torch.empty(w.M, w.h, dtype=BF16, device=d)
        dE = torch.empty(Vr, w.h, dtype=BF16, device=d)
        lgs.vocab_parallel_xent_bwd(w.b, w.s, w.h, w.vocab, w.t, r, Hd, Ed[a:a + Vr], yd, lse, dH, dE, dloss=dl)
        sync()
        step(f"xent_8p3b: oracle backward of rank {r} (host fp64), every element")
        ref = xo.shard_backward(H64, E64[a:a + Vr], yn, a, rlse, w64)
        assert_close(f"dH_{r}", dH, ref["dH"], BF16)
        assert_close(f"dE_{r}", dE, ref["dE"], BF16)

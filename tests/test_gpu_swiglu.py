"""Parity of the SwiGLU shard (tp_swiglu_fwd / tp_swiglu_bwd, through the C
ABI) with the fp64 oracle ``oracle.swiglu``.

Ragged multi-tile cases compare every element of every output; the rank's
gate/up blocks are passed as views into a rank-chunked fused weight
[h, 2 ffn] (leading dimension 2 ffn), the layout the blocks have when every
rank's [W_gate,i | W_up,i] sits side by side.  The 70B-shape shard runs in
the benchmark's launch configuration and is compared on sampled rows and
columns that the oracle computes exactly (each output entry depends only on
those).  Tolerance as for the GeLU block: max|gpu - ref| / max|ref| <= 2e-2
per output tensor (bf16 in and out, fp32 accumulation).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, f64, round_like, step
from logit_gemm_shard_amd import binding as lgs
from logit_gemm_shard_amd import synth
from logit_gemm_shard_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
sw = oracle.swiglu


def sync():
    torch.cuda.synchronize()


def fused_weight(Wg, Wu, t):
    """[g_0 | u_0 | g_1 | u_1 | ...]: every rank's two blocks side by side."""
    return torch.cat([synth.gate_up_shard(Wg, Wu, t, r) for r in range(t)], dim=1).contiguous()


def run_fwd(X, Wgu_i, Wd_i, b, s, ffn, t, r, keep_gu=True):
    M, h = X.shape
    f = ffn // t
    GU = torch.empty(M, 2 * f, dtype=BF16, device=X.device) if keep_gu else None
    Y = torch.empty(M, f, dtype=BF16, device=X.device)
    Z = torch.empty(M, h, dtype=BF16, device=X.device)
    lgs.tp_swiglu_fwd(b, s, h, ffn, t, r, X, Wgu_i, Wd_i, Z, GU_i=GU, Y_i=Y)
    return GU, Y, Z


def run_bwd(X, Wgu_i, Wd_i, GU, dZ, b, s, ffn, t, r):
    M, h = X.shape
    f = ffn // t
    dX = torch.empty(M, h, dtype=BF16, device=X.device)
    dW = torch.empty(h, 2 * f, dtype=BF16, device=X.device)
    dD = torch.empty(f, h, dtype=BF16, device=X.device)
    lgs.tp_swiglu_bwd(b, s, h, ffn, t, r, X, Wgu_i, Wd_i, GU, dZ, dX, dW, dD)
    return dX, dW, dD


RAGGED = [  # (b, s, h, ffn, t): several tiles, ragged tails in M, N and K
    (3, 200, 136, 528, 2),
    (1, 520, 328, 600, 3),
    (1, 33, 72, 128, 8),
    (2, 1100, 1064, 2 * 1048, 2),
    (1, 1, 64, 256, 2),   # a single token (the weight gradients have K = 1)
    (1, 9, 64, 256, 2),
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_swiglu_fwd_bwd_ragged(shape):
    b, s, h, ffn, t = shape
    M, f = b * s, ffn // t
    d = dev()
    X, Wg, Wu, Wd, dZ = synth.small(17 + h, (M, h), (h, ffn), (h, ffn), (ffn, h), (M, h), dtype="bf16")
    Wg, Wu, Wd = ((w.float() * 0.05).to(BF16) for w in (Wg, Wu, Wd))
    X64, dZ64 = f64(X), f64(dZ)
    Wf = fused_weight(Wg, Wu, t).to(d)  # [h, 2 ffn]
    Xd, Wdd, dZd = X.to(d), Wd.to(d), dZ.to(d)
    for r in sorted({0, t - 1}):
        step(f"swiglu ragged fwd/bwd {shape} rank={r}")
        Wg_r, Wu_r, Wd_r = (f64(Wg[:, r * f:(r + 1) * f]), f64(Wu[:, r * f:(r + 1) * f]),
                            f64(Wd[r * f:(r + 1) * f]))
        Wgu_i = Wf[:, 2 * f * r:2 * f * (r + 1)]  # a view, ld = 2 ffn
        GU, Y, Z = run_fwd(Xd, Wgu_i, Wdd[r * f:(r + 1) * f], b, s, ffn, t, r)
        sync()
        G, U, rY, rZ = sw.shard_forward(X64, Wg_r, Wu_r, Wd_r)
        assert_close("G_i", GU[:, :f], G, BF16)
        assert_close("U_i", GU[:, f:], U, BF16)
        assert_close("Y_i", Y, rY, BF16)
        assert_close("Z_i", Z, rZ, BF16)
        # backward from G, U rounded on the host from the oracle's fp64 values
        GUin = round_like(np.concatenate([G, U], axis=1), BF16)
        dX, dW, dD = run_bwd(Xd, Wgu_i, Wdd[r * f:(r + 1) * f], GUin.to(d), dZd, b, s, ffn, t, r)
        sync()
        g = sw.shard_backward(X64, Wg_r, Wu_r, Wd_r, f64(GUin[:, :f]), f64(GUin[:, f:]), dZ64)
        assert_close("dX_i", dX, g["dX"], BF16)
        assert_close("dW_gate,i", dW[:, :f], g["dWg"], BF16)
        assert_close("dW_up,i", dW[:, f:], g["dWu"], BF16)
        assert_close("dW_down,i", dD, g["dWd"], BF16)


def test_swiglu_outputs_into_strided_views_and_workspace_y():
    """GU_i and the gradients written into wider buffers (ld > width), Y_i
    left to the workspace: the same values as dense outputs."""
    b, s, h, ffn, t = 1, 300, 200, 2 * 272, 2
    M, f = b * s, ffn // t
    d = dev()
    X, Wg, Wu, Wd, dZ = synth.small(5, (M, h), (h, ffn), (h, ffn), (ffn, h), (M, h), dtype="bf16")
    Wg, Wu, Wd = ((w.float() * 0.05).to(BF16) for w in (Wg, Wu, Wd))
    Xd, dZd = X.to(d), dZ.to(d)
    Wgu, Wd_r = synth.gate_up_shard(Wg, Wu, t, 1).to(d), Wd[f:2 * f].to(d)
    step("swiglu outputs into strided views")
    GU, Y, Z = run_fwd(Xd, Wgu, Wd_r, b, s, ffn, t, 1)
    big = torch.full((M, 2 * f + 24), float("nan"), dtype=BF16, device=d)
    Z2 = torch.empty(M, h, dtype=BF16, device=d)
    lgs.tp_swiglu_fwd(b, s, h, ffn, t, 1, Xd, Wgu, Wd_r, Z2, GU_i=big[:, 8:8 + 2 * f], Y_i=None)
    sync()
    assert torch.equal(big[:, 8:8 + 2 * f], GU) and torch.equal(Z2, Z)
    assert torch.isnan(big[:, :8]).all() and torch.isnan(big[:, 8 + 2 * f:]).all()
    dX, dW, dD = run_bwd(Xd, Wgu, Wd_r, GU, dZd, b, s, ffn, t, 1)
    bigW = torch.full((h, 2 * f + 16), float("nan"), dtype=BF16, device=d)
    dX2 = torch.empty_like(dX)
    dD2 = torch.empty_like(dD)
    lgs.tp_swiglu_bwd(b, s, h, ffn, t, 1, Xd, Wgu, Wd_r, GU, dZd, dX2, bigW[:, :2 * f], dD2)
    sync()
    assert torch.equal(bigW[:, :2 * f], dW) and torch.equal(dX2, dX) and torch.equal(dD2, dD)
    assert torch.isnan(bigW[:, 2 * f:]).all()


def test_swiglu_all_shards_sum_to_unsplit():
    """The page's identity on one device: sum_i Z_i = (Swish(X W_gate) * (X W_up)) W_down,
    and the input-gradient partials sum to the unsplit dX."""
    b, s, h, ffn, t = 2, 96, 256, 4 * 320, 4
    M, f = b * s, ffn // t
    d = dev()
    X, Wg, Wu, Wd, dZ = synth.small(9, (M, h), (h, ffn), (h, ffn), (ffn, h), (M, h), dtype="bf16")
    Wg, Wu, Wd = ((w.float() * 0.05).to(BF16) for w in (Wg, Wu, Wd))
    Xd, dZd = X.to(d), dZ.to(d)
    parts = torch.empty(t, M, h, dtype=BF16, device=d)
    dparts = torch.empty(t, M, h, dtype=BF16, device=d)
    step(f"swiglu: all {t} shards + on-device sums")
    for r in range(t):
        Wgu, Wd_r = synth.gate_up_shard(Wg, Wu, t, r).to(d), Wd[r * f:(r + 1) * f].to(d)
        GU, _, Z = run_fwd(Xd, Wgu, Wd_r, b, s, ffn, t, r)
        parts[r].copy_(Z)
        dX, _, _ = run_bwd(Xd, Wgu, Wd_r, GU, dZd, b, s, ffn, t, r)
        dparts[r].copy_(dX)
    Zs = torch.empty(M, h, dtype=BF16, device=d)
    dXs = torch.empty(M, h, dtype=BF16, device=d)
    lgs.shard_partial_sum("sum", t, M * h, parts, M * h, Zs)
    lgs.shard_partial_sum("sum", t, M * h, dparts, M * h, dXs)
    sync()
    X64, Wg64, Wu64, Wd64 = f64(X), f64(Wg), f64(Wu), f64(Wd)
    assert_close("sum_i Z_i vs unsplit Z", Zs, sw.swiglu_forward(X64, Wg64, Wu64, Wd64)[3], BF16)
    assert_close("sum_i dX_i vs unsplit dX", dXs, sw.swiglu_backward(X64, Wg64, Wu64, Wd64, f64(dZ))["dX"],
                 BF16)


def test_swiglu_gate_saturation():
    """Gate pre-activations far out on both sides: Swish -> g on the right
    (Y = G * U) and -> 0 on the left, without overflow or NaN."""
    b, s, h, ffn, t = 1, 64, 64, 2 * 128, 2
    M, f = b * s, ffn // t
    d = dev()
    X, Wu, Wd = synth.small(3, (M, h), (h, ffn), (ffn, h), dtype="bf16")
    X[:, 0] = 1.0
    Wg = torch.zeros(h, ffn, dtype=BF16)
    Wg[0, :ffn // 2] = 120.0     # G = 120 for the first half of the columns
    Wg[0, ffn // 2:] = -120.0    # G = -120 for the second half
    Wu = (Wu.float() * 0.1).to(BF16)
    Wd = (Wd.float() * 0.1).to(BF16)
    step("swiglu gate saturation")
    for r in range(t):
        GU, Y, Z = run_fwd(X.to(d), synth.gate_up_shard(Wg, Wu, t, r).to(d), Wd[r * f:(r + 1) * f].to(d),
                           b, s, ffn, t, r)
        sync()
        G, U, rY, rZ = sw.shard_forward(f64(X), f64(Wg[:, r * f:(r + 1) * f]), f64(Wu[:, r * f:(r + 1) * f]),
                                        f64(Wd[r * f:(r + 1) * f]))
        assert torch.isfinite(Y.float()).all() and torch.isfinite(Z.float()).all()
        if r == 0:
            assert_close("Y_0 (gate at +120: Y = G * U)", Y, rY, BF16)
            assert_close("Z_0", Z, rZ, BF16)
        else:
            # Swish(-120) * U is about 1e-50: far below the smallest fp32 / bf16 value
            assert np.abs(rY).max() < 1e-45 and np.abs(rZ).max() < 1e-45
            assert (Y.float() == 0).all() and (Z.float() == 0).all()


# ------------------------------------------------ full size, every element

_cache = {}


def _inputs():
    if not _cache:
        w = WORKLOADS["swiglu_70b_fwd"]
        _cache["w"] = w
        _cache["X"], _cache["Wg"], _cache["Wu"], _cache["Wd"] = synth.swiglu_weights(w)
    return _cache["w"], _cache["X"], _cache["Wg"], _cache["Wu"], _cache["Wd"]


@pytest.mark.parametrize("r", [0, 7])
def test_swiglu_70b_forward_full(r):
    w, X, Wg, Wu, Wd = _inputs()
    d = dev()
    f = w.f_i
    step(f"swiglu_70b_fwd: rank {r} forward at full size")
    GU, Y, Z = run_fwd(X.to(d), synth.gate_up_shard(Wg, Wu, w.t, r).to(d), Wd[r * f:(r + 1) * f].to(d),
                       w.b, w.s, w.ffn, w.t, r)
    sync()
    step(f"swiglu_70b_fwd: oracle forward of rank {r} (host fp64), every element")
    G, U, rY, rZ = sw.shard_forward(f64(X), f64(Wg[:, r * f:(r + 1) * f]), f64(Wu[:, r * f:(r + 1) * f]),
                                    f64(Wd[r * f:(r + 1) * f]))
    GUh = GU.cpu()
    assert_close(f"G_{r}", GUh[:, :f], G, BF16)
    assert_close(f"U_{r}", GUh[:, f:], U, BF16)
    assert_close(f"Y_{r}", Y, rY, BF16)
    assert_close(f"Z_{r}", Z, rZ, BF16)


@pytest.mark.parametrize("r", [0, 7])
def test_swiglu_70b_backward_full(r):
    w, X, Wg, Wu, Wd = _inputs()
    wb = WORKLOADS["swiglu_70b_bwd"]
    d = dev()
    f = w.f_i
    Wg_r, Wu_r, Wd_r = f64(Wg[:, r * f:(r + 1) * f]), f64(Wu[:, r * f:(r + 1) * f]), f64(Wd[r * f:(r + 1) * f])
    X64 = f64(X)
    step(f"swiglu_70b_bwd: oracle G_{r}, U_{r} in fp64 (host), rounded to bf16")
    GUin = round_like(np.concatenate([X64 @ Wg_r, X64 @ Wu_r], axis=1), BF16)
    dZ = synth.mlp_grad(wb)
    step(f"swiglu_70b_bwd: rank {r} backward at full size")
    dX, dW, dD = run_bwd(X.to(d), synth.gate_up_shard(Wg, Wu, w.t, r).to(d), Wd[r * f:(r + 1) * f].to(d),
                         GUin.to(d), dZ.to(d), w.b, w.s, w.ffn, w.t, r)
    sync()
    dW = dW.cpu()
    step(f"swiglu_70b_bwd: oracle backward of rank {r} (host fp64), every element")
    g = sw.shard_backward(X64, Wg_r, Wu_r, Wd_r, f64(GUin[:, :f]), f64(GUin[:, f:]), f64(dZ))
    assert_close(f"dX_{r}", dX, g["dX"], BF16)
    assert_close(f"dW_gate,{r}", dW[:, :f], g["dWg"], BF16)
    assert_close(f"dW_up,{r}", dW[:, f:], g["dWu"], BF16)
    assert_close(f"dW_down,{r}", dD, g["dWd"], BF16)

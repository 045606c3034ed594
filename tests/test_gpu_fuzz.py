"""Parity on seeded random shapes: the HIP path (through the C ABI) against
the fp64 oracle on every output element, over shapes drawn at import from a
fixed seed (so a failure names a reproducible case).

The shapes (MLP, CE, SwiGLU, attention projections, sums) come from
tests/fuzz_cases.py, which the debug build's bounds test also drives on the
CPU.  The hand-picked ragged cases elsewhere cover each tile shape and
launch plan on purpose; these cover the space between them: token counts from 1 to
about 1300, widths from 8 to about 1100 in steps of 8 (16-byte rows), every
rank of t in {1, 2, 3, 4, 8}, and K ranges that are not multiples of the
32-wide K step.  Tolerance as in the other parity tests (max|err| / max|ref|
2e-2 for bf16 outputs with fp32 accumulation; the integer sums exactly).
"""

import numpy as np
import pytest
import torch

import oracle
from fuzz_cases import ATTN_CASES, MLP_CASES, SPLN_CASES, SUM_CASES, SWIGLU_CASES, XENT_CASES
from gpu_util import assert_close, dev, f64, round_like, step
from logit_gemm_shard_amd import binding as lgs
from logit_gemm_shard_amd import synth

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _ids(case):
    return "x".join(map(str, case))


@pytest.mark.parametrize("case", MLP_CASES, ids=_ids)
def test_fuzz_mlp_fwd_bwd(case):
    b, s, h, ffn, t, r, act = case
    M, f = b * s, ffn // t
    d = dev()
    X, A, B, dZ = synth.small(1000 + h + ffn, (M, h), (h, ffn), (ffn, h), (M, h), dtype="bf16")
    A, B = (A.float() * 0.05).to(BF16), (B.float() * 0.05).to(BF16)
    X64, dZ64 = f64(X), f64(dZ)
    A_i, B_i = f64(A[:, r * f:(r + 1) * f]), f64(B[r * f:(r + 1) * f])
    Xd, Ad, Bd = X.to(d), A.to(d), B.to(d)
    step(f"fuzz mlp {case}")
    U = torch.empty(M, f, dtype=BF16, device=d)
    Y = torch.empty(M, f, dtype=BF16, device=d)
    Z = torch.empty(M, h, dtype=BF16, device=d)
    lgs.tp_mlp_fwd(b, s, h, ffn, t, r, Xd, Ad[:, r * f:(r + 1) * f], Bd[r * f:(r + 1) * f], Z, U_i=U, Y_i=Y,
                   act=act)
    torch.cuda.synchronize()
    rU, rY, rZ = oracle.mlp.shard_forward(X64, A_i, B_i, act)
    assert_close("U_i", U, rU, BF16)
    assert_close("Y_i", Y, rY, BF16)
    assert_close("Z_i", Z, rZ, BF16)
    Uin = round_like(rU, BF16)
    dX = torch.empty(M, h, dtype=BF16, device=d)
    dA = torch.empty(h, f, dtype=BF16, device=d)
    dB = torch.empty(f, h, dtype=BF16, device=d)
    lgs.tp_mlp_bwd(b, s, h, ffn, t, r, Xd, Ad[:, r * f:(r + 1) * f], Bd[r * f:(r + 1) * f], Uin.to(d),
                   dZ.to(d), dX, dA, dB, act=act)
    torch.cuda.synchronize()
    g = oracle.mlp.shard_backward(X64, A_i, B_i, f64(Uin), dZ64, act)
    assert_close("dX_i", dX, g["dX"], BF16)
    assert_close("dA_i", dA, g["dA"], BF16)
    assert_close("dB_i", dB, g["dB"], BF16)
    # the same backward in three parts: dX's bits always; dA's and dB's where
    # the one-launch form does not split them over the tokens
    ws = torch.empty(lgs.mlp_bwd_workspace_bytes(b, s, h, ffn, t, BF16), dtype=torch.uint8, device=d)
    dX3, dA3, dB3 = torch.empty_like(dX), torch.empty_like(dA), torch.empty_like(dB)
    lgs.tp_mlp_bwd_dgelu(b, s, h, ffn, t, r, Bd[r * f:(r + 1) * f], Uin.to(d), dZ.to(d), ws, act=act)
    lgs.tp_mlp_bwd_dx(b, s, h, ffn, t, r, Ad[:, r * f:(r + 1) * f], dX3, ws)
    lgs.tp_mlp_bwd_dw(b, s, h, ffn, t, r, Xd, dZ.to(d), dA3, dB3, ws)
    torch.cuda.synchronize()
    parts, _, tail = lgs.mlp_bwd_plan(M, h, f)
    assert torch.equal(dX3, dX), "dX: three parts vs one launch"
    for name, x, y, split in (("dA", dA3, dA, parts > 1), ("dB", dB3, dB, parts > 1 and tail == 0)):
        if split:
            assert_close(f"{name}: three parts vs one split launch", x, f64(y), BF16)
        else:
            assert torch.equal(x, y), f"{name}: three parts vs one launch"


@pytest.mark.parametrize("case", XENT_CASES, ids=_ids)
def test_fuzz_xent_fwd_all_ranks_and_bwd(case):
    b, s, h, V, t = case
    M, Vr = b * s, V // t
    d = dev()
    H, E = synth.small(2000 + h + V, (M, h), (V, h), dtype="bf16")
    E = (E.float() * 0.5).to(BF16)
    y = torch.randint(0, V, (M,), generator=torch.Generator().manual_seed(M + V), dtype=torch.int64)
    y = y.to(torch.int32)
    H64, E64, yn = f64(H), f64(E), y.numpy().astype(np.int64)
    Hd, Ed, yd = H.to(d), E.to(d), y.to(d)
    step(f"fuzz xent {case}")
    stats = torch.empty(t, 3, M, dtype=F32, device=d)
    for r in range(t):
        lgs.vocab_parallel_xent_fwd(b, s, h, V, t, r, Hd, Ed[r * Vr:(r + 1) * Vr], yd, stats[r, 0], stats[r, 1],
                                    stats[r, 2])
    loss = torch.empty(M, dtype=F32, device=d)
    lse = torch.empty(M, dtype=F32, device=d)
    lgs.shard_partial_sum("xent", t, M, stats, 3 * M, loss)
    lgs.shard_partial_sum("xent_lse", t, M, stats, 3 * M, lse)
    torch.cuda.synchronize()
    sh = stats.cpu()
    for r in range(t):
        a = r * Vr
        m, l, T, _ = oracle.xent.shard_partials(H64, E64[a:a + Vr], yn, a)
        Tn = f64(sh[r, 2])[(yn < a) | (yn >= a + Vr)]
        assert np.all(Tn == 0.0) and not np.any(np.signbit(Tn))  # not owned: exactly +0
        assert_close(f"m_{r}", sh[r, 0], m, BF16)
        assert_close(f"l_{r}", sh[r, 1], l, BF16)
        assert_close(f"T_{r}", sh[r, 2], T, BF16)
    assert_close("loss (merged)", loss, oracle.xent.naive_loss(H64, E64, yn), BF16)
    # rank 0 again through the allocation-free entry point: the same bits
    st0 = torch.empty(3, M, dtype=F32, device=d)
    lgs.vocab_parallel_xent_fwd_noalloc(b, s, h, V, t, 0, Hd, Ed[:Vr], yd, st0[0], st0[1], st0[2])
    torch.cuda.synchronize()
    assert torch.equal(st0.cpu(), sh[0]), "noalloc partials differ from the workspace call"
    # the backward of one rank from the merged lse (dloss = 1 per token)
    r = t - 1
    dH = torch.empty(M, h, dtype=BF16, device=d)
    dE = torch.empty(Vr, h, dtype=BF16, device=d)
    lgs.vocab_parallel_xent_bwd(b, s, h, V, t, r, Hd, Ed[r * Vr:(r + 1) * Vr], yd, lse, dH, dE)
    torch.cuda.synchronize()
    ref = oracle.xent.shard_backward(H64, E64[r * Vr:(r + 1) * Vr], yn, r * Vr, f64(lse))
    assert_close(f"dH_{r} (partial)", dH, ref["dH"], BF16)
    assert_close(f"dE_{r}", dE, ref["dE"], BF16)


@pytest.mark.parametrize("case", SWIGLU_CASES, ids=_ids)
def test_fuzz_swiglu_fwd_bwd(case):
    b, s, h, ffn, t, r = case
    M, f = b * s, ffn // t
    d = dev()
    X, Wg, Wu, Wd, dZ = synth.small(3000 + h + ffn, (M, h), (h, ffn), (h, ffn), (ffn, h), (M, h), dtype="bf16")
    Wg, Wu, Wd = ((w.float() * 0.05).to(BF16) for w in (Wg, Wu, Wd))
    X64, dZ64 = f64(X), f64(dZ)
    Wg_r, Wu_r, Wd_r = f64(Wg[:, r * f:(r + 1) * f]), f64(Wu[:, r * f:(r + 1) * f]), f64(Wd[r * f:(r + 1) * f])
    Wgu_i = synth.gate_up_shard(Wg, Wu, t, r).to(d)
    Wd_i = Wd[r * f:(r + 1) * f].contiguous().to(d)
    Xd = X.to(d)
    step(f"fuzz swiglu {case}")
    GU = torch.empty(M, 2 * f, dtype=BF16, device=d)
    Y = torch.empty(M, f, dtype=BF16, device=d)
    Z = torch.empty(M, h, dtype=BF16, device=d)
    lgs.tp_swiglu_fwd(b, s, h, ffn, t, r, Xd, Wgu_i, Wd_i, Z, GU_i=GU, Y_i=Y)
    torch.cuda.synchronize()
    G, U, rY, rZ = oracle.swiglu.shard_forward(X64, Wg_r, Wu_r, Wd_r)
    assert_close("G_i", GU[:, :f], G, BF16)
    assert_close("U_i", GU[:, f:], U, BF16)
    assert_close("Y_i", Y, rY, BF16)
    assert_close("Z_i", Z, rZ, BF16)
    GUin = round_like(np.concatenate([G, U], axis=1), BF16)
    dX = torch.empty(M, h, dtype=BF16, device=d)
    dW = torch.empty(h, 2 * f, dtype=BF16, device=d)
    dD = torch.empty(f, h, dtype=BF16, device=d)
    lgs.tp_swiglu_bwd(b, s, h, ffn, t, r, Xd, Wgu_i, Wd_i, GUin.to(d), dZ.to(d), dX, dW, dD)
    torch.cuda.synchronize()
    g = oracle.swiglu.shard_backward(X64, Wg_r, Wu_r, Wd_r, f64(GUin[:, :f]), f64(GUin[:, f:]), dZ64)
    assert_close("dX_i", dX, g["dX"], BF16)
    assert_close("dW_gate,i", dW[:, :f], g["dWg"], BF16)
    assert_close("dW_up,i", dW[:, f:], g["dWu"], BF16)
    assert_close("dW_down,i", dD, g["dWd"], BF16)


@pytest.mark.parametrize("case", ATTN_CASES, ids=_ids)
def test_fuzz_attn_projections(case):
    b, s, h, n_q, n_kv, d, t, r = case
    M, q, kv = b * s, n_q // t * d, n_kv // t * d
    dv = dev()
    X, Wq, Wk, Wv, Wo, A, dZ, dQ = synth.small(
        4000 + h + d, (M, h), (h, n_q * d), (h, n_kv * d), (h, n_kv * d), (n_q * d, h), (M, q), (M, h),
        (M, q + 2 * kv), dtype="bf16")
    Wq, Wk, Wv, Wo = ((w.float() * 0.05).to(BF16) for w in (Wq, Wk, Wv, Wo))
    X64 = f64(X)
    W = synth.qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, r)
    W64 = oracle.attn.qkv_shard(f64(Wq), f64(Wk), f64(Wv), n_q, n_kv, d, t, r)
    Wo_r = Wo[r * q:(r + 1) * q].contiguous()
    Xd, Wd, Wod, Ad = X.to(dv), W.to(dv), Wo_r.to(dv), A.to(dv)
    step(f"fuzz attn {case}")
    QKV = torch.empty(M, q + 2 * kv, dtype=BF16, device=dv)
    lgs.tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, r, Xd, Wd, QKV)
    Z = torch.empty(M, h, dtype=BF16, device=dv)
    lgs.tp_attn_out_fwd(b, s, h, n_q, d, t, r, Ad, Wod, Z)
    dX = torch.empty(M, h, dtype=BF16, device=dv)
    dW = torch.empty(h, q + 2 * kv, dtype=BF16, device=dv)
    lgs.tp_attn_qkv_bwd(b, s, h, n_q, n_kv, d, t, r, Xd, Wd, dQ.to(dv), dX, dW)
    dA = torch.empty(M, q, dtype=BF16, device=dv)
    dWo = torch.empty(q, h, dtype=BF16, device=dv)
    lgs.tp_attn_out_bwd(b, s, h, n_q, d, t, r, Ad, Wod, dZ.to(dv), dA, dWo)
    torch.cuda.synchronize()
    assert_close("QKV_i", QKV, oracle.attn.qkv_forward(X64, W64), BF16)
    assert_close("Z_i", Z, oracle.attn.out_forward(f64(A), f64(Wo_r)), BF16)
    g = oracle.attn.qkv_backward(X64, W64, f64(dQ))
    assert_close("dX_i", dX, g["dX"], BF16)
    assert_close("dWqkv_i", dW, g["dW"], BF16)
    g = oracle.attn.out_backward(f64(A), f64(Wo_r), f64(dZ))
    assert_close("dA_i", dA, g["dA"], BF16)
    assert_close("dWo_i", dWo, g["dW"], BF16)


@pytest.mark.parametrize("case", SUM_CASES, ids=_ids)
def test_fuzz_partial_sum_exact(case):
    """Small integers: every partial sum is exact in fp32 and in bf16."""
    t, n, to_bf16 = case
    d = dev()
    parts = torch.randint(-8, 9, (t, n), generator=torch.Generator().manual_seed(t * 100003 + n)).to(BF16)
    out = torch.empty(n, dtype=BF16 if to_bf16 else F32, device=d)
    step(f"fuzz sum {case}")
    lgs.shard_partial_sum("sum", t, n, parts.to(d), n, out)
    torch.cuda.synchronize()
    assert np.array_equal(f64(out), f64(parts).sum(axis=0))


@pytest.mark.parametrize("case", SPLN_CASES, ids=_ids)
def test_fuzz_sp_region(case):
    t, s, b, h, r, masked = case
    n = (s // t) * b
    d = dev()
    g = torch.Generator().manual_seed(5000 + h + s)
    parts = torch.randn(t, s * b, h, generator=g).to(BF16)
    res = torch.randn(n, h, generator=g).to(BF16)
    gamma = (1 + 0.1 * torch.randn(h, generator=g)).to(BF16)
    beta = (0.1 * torch.randn(h, generator=g)).to(BF16)
    keep = (torch.rand(n, h, generator=g) > 0.2).to(torch.uint8) if masked else None
    step(f"fuzz sp region {case}")
    hs = torch.empty(n, h, dtype=BF16, device=d)
    y = torch.empty(n, h, dtype=BF16, device=d)
    lgs.shard_reduce_scatter_layernorm(t, r, s, b, h, parts.to(d), s * b * h, res.to(d), gamma.to(d), beta.to(d),
                                       hs, y, keep=None if keep is None else keep.to(d), keep_scale=1.25)
    torch.cuda.synchronize()
    rh, ry = oracle.sp.exit_region([f64(p) for p in parts], s, b, t, r, f64(res), f64(gamma), f64(beta), 1e-5,
                                   None if keep is None else keep.numpy(), 1.25)
    assert_close("hs", hs, rh, BF16)
    assert_close("y", y, ry, BF16)
    # its backward from random dy and dhs, at the hs the forward stored
    dy = torch.randn(n, h, generator=g).to(BF16)
    dhs = torch.randn(n, h, generator=g).to(BF16)
    G = torch.empty(n, h, dtype=BF16, device=d)
    dz = torch.empty(n, h, dtype=BF16, device=d)
    dg, db = torch.empty(h, dtype=F32, device=d), torch.empty(h, dtype=F32, device=d)
    lgs.shard_layernorm_bwd(t, r, s, b, h, hs, dy.to(d), gamma.to(d), G, dz, dg, db, dhs=dhs.to(d),
                            keep=None if keep is None else keep.to(d), keep_scale=1.25)
    torch.cuda.synchronize()
    ref = oracle.sp.exit_region_backward(f64(hs), f64(gamma), f64(dy), f64(dhs), 1e-5,
                                         None if keep is None else keep.numpy(), 1.25)
    assert_close("g", G, ref["g"], BF16)
    assert_close("dz", dz, ref["dz"], BF16)
    assert_close("dgamma", dg, ref["dgamma"], F32)
    assert_close("dbeta", db, ref["dbeta"], F32)


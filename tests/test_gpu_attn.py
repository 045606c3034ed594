"""Parity of the attention projections under TP (tp_attn_qkv_fwd / _bwd,
tp_attn_out_fwd / _bwd, through the C ABI) with the fp64 oracle
``oracle.attn``.

Ragged multi-tile shapes compare every element.  The split identity runs on
the device: each rank's heads' outputs (the oracle's attention core on the
oracle's projections, rounded to bf16: the core is not part of the library)
go through the rank's output projection, and the on-device sum of the
partials equals the oracle's unsplit block.  The 70B-shape rank (8 query
heads and 1 KV head of 128) is compared on sampled rows and columns.
Tolerance: max|gpu - ref| / max|ref| <= 2e-2 per output (bf16 in and out,
fp32 accumulation).
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
at = oracle.attn


def sync():
    torch.cuda.synchronize()


RAGGED = [  # (b, s, h, n_q, n_kv, d, t)
    (1, 300, 136, 8, 4, 16, 2),
    (2, 130, 264, 12, 4, 24, 4),
    (1, 520, 1032, 16, 8, 64, 8),
    (1, 700, 512, 8, 8, 128, 2),
    (1, 1, 128, 4, 2, 32, 2),   # a single token
    (1, 9, 128, 4, 2, 32, 2),
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_attn_projections_ragged(shape):
    b, s, h, n_q, n_kv, d, t = shape
    M = b * s
    q, kv = n_q // t * d, n_kv // t * d
    dev_ = dev()
    X, Wq, Wk, Wv, Wo, A, dZ, dQ = synth.small(
        3 + h, (M, h), (h, n_q * d), (h, n_kv * d), (h, n_kv * d), (n_q * d, h), (M, q), (M, h), (M, q + 2 * kv),
        dtype="bf16")
    Wq, Wk, Wv, Wo = ((w.float() * 0.05).to(BF16) for w in (Wq, Wk, Wv, Wo))
    X64 = f64(X)
    Xd = X.to(dev_)
    for r in sorted({0, t - 1}):
        step(f"attn projections {shape} rank={r}")
        W = synth.qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, r)
        W64 = at.qkv_shard(f64(Wq), f64(Wk), f64(Wv), n_q, n_kv, d, t, r)
        assert np.array_equal(f64(W), W64)  # the host-side layout copy matches the oracle's shard
        Wo_r = Wo[r * q:(r + 1) * q].contiguous()
        Wd, Wod = W.to(dev_), Wo_r.to(dev_)
        QKV = torch.empty(M, q + 2 * kv, dtype=BF16, device=dev_)
        lgs.tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, r, Xd, Wd, QKV)
        Z = torch.empty(M, h, dtype=BF16, device=dev_)
        lgs.tp_attn_out_fwd(b, s, h, n_q, d, t, r, A.to(dev_), Wod, Z)
        dX = torch.empty(M, h, dtype=BF16, device=dev_)
        dW = torch.empty(h, q + 2 * kv, dtype=BF16, device=dev_)
        lgs.tp_attn_qkv_bwd(b, s, h, n_q, n_kv, d, t, r, Xd, Wd, dQ.to(dev_), dX, dW)
        dA = torch.empty(M, q, dtype=BF16, device=dev_)
        dWo = torch.empty(q, h, dtype=BF16, device=dev_)
        lgs.tp_attn_out_bwd(b, s, h, n_q, d, t, r, A.to(dev_), Wod, dZ.to(dev_), dA, dWo)
        sync()
        assert_close("QKV_i", QKV, at.qkv_forward(X64, W64), BF16)
        assert_close("Z_i", Z, at.out_forward(f64(A), f64(Wo_r)), BF16)
        g = at.qkv_backward(X64, W64, f64(dQ))
        assert_close("dX_i", dX, g["dX"], BF16)
        assert_close("dWqkv_i", dW, g["dW"], BF16)
        g = at.out_backward(f64(A), f64(Wo_r), f64(dZ))
        assert_close("dA_i", dA, g["dA"], BF16)
        assert_close("dWo_i", dWo, g["dW"], BF16)


def test_attn_qkv_split_k_every_element():
    """A deep QKV product (h = 2600) with few output tiles runs split over K
    (4 parts, the last one with a partial K tile, reduced inside the launch)
    when given its workspace: every element against the oracle, and against
    the unsplit run (same values up to the fp32 summation order)."""
    b, s, h, n_q, n_kv, d, t = 1, 600, 2600, 8, 4, 128, 2
    M, q, kv = b * s, n_q // t * d, n_kv // t * d
    dev_ = dev()
    tiles = -(-M // 256) * -(-(q + 2 * kv) // 256)  # 3 x 4 tiles of 256x256, 4 fp32 slots each
    assert lgs.attn_qkv_fwd_workspace_bytes(b, s, h, n_q, n_kv, d, t) == \
        (tiles * 4 * 256 * 256 * 4 + tiles * 4 + 255) // 256 * 256
    X, Wq, Wk, Wv = synth.small(21, (M, h), (h, n_q * d), (h, n_kv * d), (h, n_kv * d), dtype="bf16")
    Wq, Wk, Wv = ((w.float() * 0.03).to(BF16) for w in (Wq, Wk, Wv))
    W = synth.qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, 1)
    step("attn QKV split-K vs unsplit vs oracle")
    Xd, Wd = X.to(dev_), W.to(dev_)
    QKVs = torch.empty(M, q + 2 * kv, dtype=BF16, device=dev_)
    QKVu = torch.empty_like(QKVs)
    lgs.tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, 1, Xd, Wd, QKVs)
    lgs.tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, 1, Xd, Wd, QKVu, split=False)
    sync()
    ref = at.qkv_forward(f64(X), at.qkv_shard(f64(Wq), f64(Wk), f64(Wv), n_q, n_kv, d, t, 1))
    assert_close("QKV_1 split-K", QKVs, ref, BF16)
    assert_close("QKV_1 unsplit", QKVu, ref, BF16)
    assert_close("split-K vs unsplit", QKVs, f64(QKVu), BF16)


def test_attn_out_bwd_split_k_every_element():
    """The output projection's backward with dA split over K in two (few dA
    tiles, h = 4096; the halves reduced inside the launch): every element of
    dA and dW_O against the oracle and against the unsplit run."""
    b, s, h, n_q, d, t = 1, 520, 4096, 8, 128, 2
    M, q = b * s, n_q // t * d
    dev_ = dev()
    tiles = -(-M // 256) * -(-q // 256)  # 3 x 2 dA tiles of 256x256, two fp32 slots each
    assert lgs.attn_out_bwd_workspace_bytes(b, s, h, n_q, d, t) == \
        (tiles * 2 * 256 * 256 * 4 + tiles * 4 + 255) // 256 * 256
    A, Wo, dZ = synth.small(23, (M, q), (n_q * d, h), (M, h), dtype="bf16")
    Wo_r = (Wo[q:2 * q].float() * 0.05).to(BF16).contiguous()
    step("attn out-proj backward split-K vs unsplit vs oracle")
    Ad, Wod, dZd = A.to(dev_), Wo_r.to(dev_), dZ.to(dev_)
    dA, dW = torch.empty(M, q, dtype=BF16, device=dev_), torch.empty(q, h, dtype=BF16, device=dev_)
    dAu, dWu = torch.empty_like(dA), torch.empty_like(dW)
    lgs.tp_attn_out_bwd(b, s, h, n_q, d, t, 1, Ad, Wod, dZd, dA, dW)
    lgs.tp_attn_out_bwd(b, s, h, n_q, d, t, 1, Ad, Wod, dZd, dAu, dWu, split=False)
    sync()
    g = at.out_backward(f64(A), f64(Wo_r), f64(dZ))
    assert_close("dA (split-K)", dA, g["dA"], BF16)
    assert_close("dA (unsplit)", dAu, g["dA"], BF16)
    assert_close("dWo (with split dA)", dW, g["dW"], BF16)
    assert torch.equal(dW, dWu)  # dW_O takes the same path either way


def test_attn_split_identity_on_device():
    """sum over ranks of (rank's heads attended) W_O^i == the unsplit block."""
    b, s, h, n_q, n_kv, d, t = 1, 96, 256, 8, 4, 32, 4
    M, q = b * s, n_q // 4 * d
    dev_ = dev()
    X, Wq, Wk, Wv, Wo = synth.small(12, (M, h), (h, n_q * d), (h, n_kv * d), (h, n_kv * d), (n_q * d, h),
                                    dtype="bf16")
    Wq, Wk, Wv, Wo = ((w.float() * 0.05).to(BF16) for w in (Wq, Wk, Wv, Wo))
    X64, Wq64, Wk64, Wv64, Wo64 = f64(X), f64(Wq), f64(Wk), f64(Wv), f64(Wo)
    parts = torch.empty(t, M, h, dtype=BF16, device=dev_)
    step("attn: every rank's output projection of its own heads + on-device sum")
    for r in range(t):
        heads = at.attention_core(at.qkv_forward(X64, at.qkv_shard(Wq64, Wk64, Wv64, n_q, n_kv, d, t, r)),
                                  n_q // t, n_kv // t, d)
        lgs.tp_attn_out_fwd(b, s, h, n_q, d, t, r, round_like(heads, BF16).to(dev_),
                            Wo[r * q:(r + 1) * q].contiguous().to(dev_), parts[r])
    Z = torch.empty(M, h, dtype=BF16, device=dev_)
    lgs.shard_partial_sum("sum", t, M * h, parts, M * h, Z)
    sync()
    assert_close("sum_i Z_i vs unsplit attention block", Z,
                 at.block_forward(X64, Wq64, Wk64, Wv64, Wo64, n_q, n_kv, d), BF16)


def test_attn_70b_full():
    """The 70B-shape projections of ranks 0 and 7 at full size (the QKV
    product split over K as the benchmark runs it, and unsplit): every
    element of every output against the oracle."""
    w = WORKLOADS["attn_70b"]
    b, s, h, n_q, n_kv, d, t = w.b, w.s, w.h, w.n_heads, w.n_kv_heads, w.head_dim, w.t
    M, q, kv = w.M, n_q // t * d, n_kv // t * d
    dev_ = dev()
    X, Wq, Wk, Wv, Wo = synth.attn_weights(w)
    g = torch.Generator().manual_seed(w.dz_seed)
    A = synth.normal((M, q), 1.0, g, "bf16")
    dZ = synth.normal((M, h), w.dz_std, g, "bf16")
    dQ = synth.normal((M, q + 2 * kv), w.dz_std, g, "bf16")
    X64, A64, dZ64, dQ64 = f64(X), f64(A), f64(dZ), f64(dQ)
    for r in (0, t - 1):
        step(f"attn_70b: rank {r} projections, forward and backward, at full size")
        W = synth.qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, r)
        Wo_r = Wo[r * q:(r + 1) * q].contiguous()
        Xd, Wd, Wod, Ad = X.to(dev_), W.to(dev_), Wo_r.to(dev_), A.to(dev_)
        QKV = torch.empty(M, q + 2 * kv, dtype=BF16, device=dev_)
        lgs.tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, r, Xd, Wd, QKV)  # split over K (the bench's schedule)
        QKVu = torch.empty_like(QKV)
        lgs.tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, r, Xd, Wd, QKVu, split=False)
        Z = torch.empty(M, h, dtype=BF16, device=dev_)
        lgs.tp_attn_out_fwd(b, s, h, n_q, d, t, r, Ad, Wod, Z)
        dX = torch.empty(M, h, dtype=BF16, device=dev_)
        dW = torch.empty(h, q + 2 * kv, dtype=BF16, device=dev_)
        lgs.tp_attn_qkv_bwd(b, s, h, n_q, n_kv, d, t, r, Xd, Wd, dQ.to(dev_), dX, dW)
        dA = torch.empty(M, q, dtype=BF16, device=dev_)
        dWo = torch.empty(q, h, dtype=BF16, device=dev_)
        lgs.tp_attn_out_bwd(b, s, h, n_q, d, t, r, Ad, Wod, dZ.to(dev_), dA, dWo)
        sync()
        step(f"attn_70b: oracle projections of rank {r} (host fp64), every element")
        W64 = at.qkv_shard(f64(Wq), f64(Wk), f64(Wv), n_q, n_kv, d, t, r)
        rQKV = at.qkv_forward(X64, W64)
        assert_close(f"QKV_{r}", QKV, rQKV, BF16)
        assert_close(f"QKV_{r} (unsplit)", QKVu, rQKV, BF16)
        assert_close(f"Z_{r}", Z, at.out_forward(A64, f64(Wo_r)), BF16)
        gq = at.qkv_backward(X64, W64, dQ64)
        assert_close(f"dX_{r}", dX, gq["dX"], BF16)
        assert_close(f"dWqkv_{r}", dW, gq["dW"], BF16)
        go = at.out_backward(A64, f64(Wo_r), dZ64)
        assert_close(f"dA_{r}", dA, go["dA"], BF16)
        assert_close(f"dWo_{r}", dWo, go["dW"], BF16)

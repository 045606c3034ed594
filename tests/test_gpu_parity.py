"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small cases compare every element; cases spanning several tiles have ragged
tails in M, N and K.  The full workloads (8.3B-shape and 70B-shape shards,
the 51,200-entry vocabulary) run in the same launch configuration as the
benchmark and are compared with the oracle on every output element.

Tolerance: max|gpu - ref| / max|ref| per output tensor, 1e-4 for fp32 and
2e-2 for bf16 (fp32 accumulation); integer outputs (argmax ids, ownership of
the target) exactly, up to near-ties within the fp32 dot-product error bound.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, dev, f64, rel_err, round_like, step
from logit_gemm_shard_amd import binding as lgs
from logit_gemm_shard_amd import synth
from logit_gemm_shard_amd.configs import WORKLOADS

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


# ------------------------------------------------------------------ helpers

def run_fwd(X, A, B, b, s, t, r, act, with_u=True):
    """rank r's forward from full A [h, ffn] / B [ffn, h] on the device."""
    M, h = X.shape
    ffn = A.shape[1]
    f = ffn // t
    U = torch.empty(M, f, dtype=X.dtype, device=X.device) if with_u else None
    Y = torch.empty(M, f, dtype=X.dtype, device=X.device)
    Z = torch.empty(M, h, dtype=X.dtype, device=X.device)
    lgs.tp_mlp_fwd(b, s, h, ffn, t, r, X, A[:, r * f:(r + 1) * f], B[r * f:(r + 1) * f], Z, U_i=U,
                   Y_i=Y, act=act)
    return U, Y, Z


def run_bwd(X, A, B, U, dZ, b, s, t, r, act):
    M, h = X.shape
    ffn = A.shape[1]
    f = ffn // t
    dX = torch.empty(M, h, dtype=X.dtype, device=X.device)
    dA = torch.empty(h, f, dtype=X.dtype, device=X.device)
    dB = torch.empty(f, h, dtype=X.dtype, device=X.device)
    lgs.tp_mlp_bwd(b, s, h, ffn, t, r, X, A[:, r * f:(r + 1) * f], B[r * f:(r + 1) * f], U, dZ, dX,
                   dA, dB, act=act)
    return dX, dA, dB


def sync():
    torch.cuda.synchronize()


# --------------------------------------------------------- tiny fp32 (t = 2)

@pytest.mark.parametrize("act", ["erf", "tanh"])
def test_tiny_mlp_t2_f32_shards_and_sum(act):
    w = WORKLOADS["tiny_mlp_t2_f32"]
    step(f"tiny_mlp_t2_f32 act={act}: both shards + sum")
    d = dev()
    X, A, B = synth.mlp_weights(w)
    X64, A64, B64 = f64(X), f64(A), f64(B)
    Xd, Ad, Bd = X.to(d), A.to(d), B.to(d)
    parts = torch.empty(w.t, w.M, w.h, dtype=F32, device=d)
    f = w.f_i
    for r in range(w.t):
        U, Y, Z = run_fwd(Xd, Ad, Bd, w.b, w.s, w.t, r, act)
        parts[r].copy_(Z)
        sync()
        rU, rY, rZ = oracle.mlp.shard_forward(X64, A64[:, r * f:(r + 1) * f], B64[r * f:(r + 1) * f], act)
        assert_close(f"U_{r}", U, rU, F32)
        assert_close(f"Y_{r}", Y, rY, F32)
        assert_close(f"Z_{r}", Z, rZ, F32)
    Zs = torch.empty(w.M, w.h, dtype=F32, device=d)
    lgs.shard_partial_sum("sum", w.t, w.M * w.h, parts, w.M * w.h, Zs)
    sync()
    assert_close("sum_i Z_i vs unsplit Z", Zs, oracle.mlp.mlp_forward(X64, A64, B64, act)[2], F32)


# --------------------------------------------- the GEMM core, every tile shape

@pytest.mark.parametrize("layout", [(True, False), (True, True), (False, False)])
def test_gemm_core_every_tile_ragged(layout):
    ak, bk = layout
    d = dev()
    shapes = lgs.tile_shapes()
    for tid, (bm, bn) in enumerate(shapes):
        # two tiles and a ragged tail in M and N, K not a multiple of the 64-wide step
        M, N, K = 2 * bm + 24, 2 * bn + 40, 200
        step(f"gemm core tile {bm}x{bn} layout a_kmajor={ak} b_kmajor={bk} M={M} N={N} K={K}")
        a, b = synth.small(100 + tid, (M, K), (K, N), dtype="bf16")
        A = (a if ak else a.t().contiguous()).to(d)
        B = (b if not bk else b.t().contiguous()).to(d)
        C = torch.empty(M, N, dtype=BF16, device=d)
        lgs.gemm_bf16(A, B, C, a_kmajor=ak, b_kmajor=bk, tile=tid)
        sync()
        assert_close(f"C tile {bm}x{bn}", C, f64(a) @ f64(b), BF16)


# ------------------------------------------------ ragged multi-tile MLP fwd/bwd

RAGGED = [  # (b, s, h, ffn, t)
    (3, 200, 136, 528, 2),
    (1, 520, 328, 600, 3),
    (1, 33, 72, 128, 8),
    (2, 1100, 1064, 2 * 1048, 2),
]


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_mlp_fwd_bwd_ragged(shape, dtype):
    b, s, h, ffn, t = shape
    M, f = b * s, ffn // t
    d = dev()
    dn = "bf16" if dtype == BF16 else "f32"
    X, A, B, dZ = synth.small(7 + h, (M, h), (h, ffn), (ffn, h), (M, h), dtype=dn)
    A, B = (A.float() * 0.05).to(dtype), (B.float() * 0.05).to(dtype)
    X64, A64, B64, dZ64 = f64(X), f64(A), f64(B), f64(dZ)
    Xd, Ad, Bd, dZd = X.to(d), A.to(d), B.to(d), dZ.to(d)
    for act in ("erf", "tanh"):
        for r in sorted({0, t - 1}):
            step(f"ragged fwd/bwd {shape} {dn} act={act} rank={r}")
            A_i, B_i = A64[:, r * f:(r + 1) * f], B64[r * f:(r + 1) * f]
            U, Y, Z = run_fwd(Xd, Ad, Bd, b, s, t, r, act)
            sync()
            rU, rY, rZ = oracle.mlp.shard_forward(X64, A_i, B_i, act)
            assert_close("U_i", U, rU, dtype)
            assert_close("Y_i", Y, rY, dtype)
            assert_close("Z_i", Z, rZ, dtype)
            # backward from a U rounded on the host from the oracle's fp64 U
            Uin = round_like(rU, dtype)
            dX, dA, dB = run_bwd(Xd, Ad, Bd, Uin.to(d), dZd, b, s, t, r, act)
            sync()
            g = oracle.mlp.shard_backward(X64, A_i, B_i, f64(Uin), dZ64, act)
            assert_close("dX_i", dX, g["dX"], dtype)
            assert_close("dA_i", dA, g["dA"], dtype)
            assert_close("dB_i", dB, g["dB"], dtype)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 200, 136, 528, 2), (2, 1100, 1064, 2 * 1048, 2), (1, 1024, 3072, 8 * 1536, 8),
                                   (2, 300, 3584, 4 * 2048, 4)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mlp_bwd_in_three_parts(shape, dtype):
    """dgelu, then dx and dw on two streams running concurrently, against the
    oracle and against tp_mlp_bwd: the same bits, except where tp_mlp_bwd
    splits a weight gradient over the tokens inside its launch, which changes
    only the fp32 summation order (the plan comes from the library's testing
    hook).  bf16 at M = 2200, h = 1064, f = 1048 splits every dA and dB tile
    in 2 parts; at M = 600, h = 3584, f = 2048 only the last dA tiles (the
    second part ragged: 280 tokens), dB staying unsplit.  A split launch
    repeats its bits."""
    b, s, h, ffn, t = shape
    M, f = b * s, ffn // t
    d = dev()
    dn = "bf16" if dtype == BF16 else "f32"
    X, A, B, dZ = synth.small(5 + h, (M, h), (h, f), (f, h), (M, h), dtype=dn)
    A, B = (A.float() * 0.05).to(dtype), (B.float() * 0.05).to(dtype)
    X64, A64, B64, dZ64 = f64(X), f64(A), f64(B), f64(dZ)
    U = round_like(X64 @ A64, dtype)
    Xd, Ad, Bd, Ud, dZd = X.to(d), A.to(d), B.to(d), U.to(d), dZ.to(d)
    step(f"backward in three parts {shape} {dn}")
    ws = torch.empty(lgs.mlp_bwd_workspace_bytes(b, s, h, ffn, t, dtype), dtype=torch.uint8, device=d)
    dX1 = torch.empty(M, h, dtype=dtype, device=d)
    dA1 = torch.empty(h, f, dtype=dtype, device=d)
    dB1 = torch.empty(f, h, dtype=dtype, device=d)
    side = torch.cuda.Stream()
    lgs.tp_mlp_bwd_dgelu(b, s, h, ffn, t, 0, Bd, Ud, dZd, ws)
    done = torch.cuda.Event()
    done.record()
    side.wait_event(done)
    with torch.cuda.stream(side):
        lgs.tp_mlp_bwd_dw(b, s, h, ffn, t, 0, Xd, dZd, dA1, dB1, ws)
    lgs.tp_mlp_bwd_dx(b, s, h, ffn, t, 0, Ad, dX1, ws)
    torch.cuda.current_stream().wait_stream(side)
    # the one-launch backward on its own workspace, for comparison
    dX2 = torch.empty_like(dX1)
    dA2 = torch.empty_like(dA1)
    dB2 = torch.empty_like(dB1)
    lgs.tp_mlp_bwd(b, s, h, ffn, t, 0, Xd, Ad, Bd, Ud, dZd, dX2, dA2, dB2)
    sync()
    g = oracle.mlp.shard_backward(X64, A64, B64, f64(U), dZ64)
    assert_close("dX (three parts)", dX1, g["dX"], dtype)
    assert_close("dA (three parts)", dA1, g["dA"], dtype)
    assert_close("dB (three parts)", dB1, g["dB"], dtype)
    parts, _, tail = lgs.mlp_bwd_plan(M, h, f) if dtype == BF16 else (1, M, 0)
    split_a, split_b = parts > 1, parts > 1 and tail == 0
    assert (split_a, split_b) == {1064: (dtype == BF16,) * 2, 3584: (dtype == BF16, False)}.get(h, (False, False))
    assert torch.equal(dX1, dX2), "dX: three parts vs one launch"
    for name, x, y, split in (("dA", dA1, dA2, split_a), ("dB", dB1, dB2, split_b)):
        if split:
            assert_close(f"{name}: three parts vs one split launch", x, f64(y), dtype)
        else:
            assert torch.equal(x, y), f"{name}: three parts vs one launch"
    if split_a:
        dX3, dA3, dB3 = torch.empty_like(dX2), torch.empty_like(dA2), torch.empty_like(dB2)
        lgs.tp_mlp_bwd(b, s, h, ffn, t, 0, Xd, Ad, Bd, Ud, dZd, dX3, dA3, dB3)
        sync()
        assert torch.equal(dA3, dA2) and torch.equal(dB3, dB2), "a split launch repeats its bits"


def test_mlp_bwd_weight_grads_split_inside_the_launch():
    """Many tokens with small h and f make few, long dB / dA tiles; the
    grouped backward launch then splits them over the tokens into parts that
    it reduces itself (here 4 parts, the last one ragged: M = 8264 is not a
    multiple of 32).  The gradients match the oracle, and repeat bit for bit:
    the last part to finish adds the parts' partial sums in part order,
    whichever part it is."""
    b, s, h, ffn, t = 1, 8264, 776, 1040, 2
    M, f = b * s, ffn // t
    d = dev()
    X, A, B, dZ = synth.small(41, (M, h), (h, ffn), (ffn, h), (M, h), dtype="bf16")
    A, B = (A.float() * 0.05).to(BF16), (B.float() * 0.05).to(BF16)
    X64, A64, B64, dZ64 = f64(X), f64(A), f64(B), f64(dZ)
    Xd, Ad, Bd, dZd = X.to(d), A.to(d), B.to(d), dZ.to(d)
    plain = 2 * ((M * f * 2 + 255) // 256 * 256)
    assert lgs.mlp_bwd_workspace_bytes(b, s, h, ffn, t, BF16) > plain, "expected the K-split plan"
    for r in range(t):
        step(f"weight gradients split inside the launch, rank {r}")
        U = round_like(X64 @ A64[:, r * f:(r + 1) * f], BF16)
        first = None
        for rep in range(2):
            dX, dA, dB = run_bwd(Xd, Ad, Bd, U.to(d), dZd, b, s, t, r, "erf")
            sync()
            if first is None:
                g = oracle.mlp.shard_backward(X64, A64[:, r * f:(r + 1) * f], B64[r * f:(r + 1) * f], f64(U), dZ64)
                assert_close("dX_i", dX, g["dX"], BF16)
                assert_close("dA_i", dA, g["dA"], BF16)
                assert_close("dB_i", dB, g["dB"], BF16)
                first = (dX, dA, dB)
            else:
                for name, x, y in zip(("dX", "dA", "dB"), (dX, dA, dB), first):
                    assert torch.equal(x, y), f"{name}: second call differs"


def test_t1_is_the_unsplit_block():
    d = dev()
    b, s, h, ffn = 1, 300, 264, 520
    X, A, B = synth.small(5, (b * s, h), (h, ffn), (ffn, h), dtype="bf16")
    A, B = (A.float() * 0.05).to(BF16), (B.float() * 0.05).to(BF16)
    step("t=1 forward equals the unsplit block")
    U, Y, Z = run_fwd(X.to(d), A.to(d), B.to(d), b, s, 1, 0, "erf")
    sync()
    assert_close("Z (t=1)", Z, oracle.mlp.mlp_forward(f64(X), f64(A), f64(B))[2], BF16)


# ----------------------------------------------------------------- sum kernels

@pytest.mark.parametrize("t", [1, 2, 8])
@pytest.mark.parametrize("n", [8192 + 8, 1001])
@pytest.mark.parametrize("din,dout", [(BF16, BF16), (BF16, F32), (F32, F32), (F32, BF16)])
def test_partial_sum_exact_on_integers(t, n, din, dout):
    d = dev()
    step(f"partial sum t={t} n={n} {din}->{dout}")
    g = torch.Generator().manual_seed(t * 7 + n)
    parts = torch.randint(-16, 17, (t, n), generator=g).to(din)
    out = torch.full((n,), float("nan"), dtype=dout, device=d)
    lgs.shard_partial_sum("sum", t, n, parts.to(d), n, out)
    sync()
    want = oracle.mlp.partial_sum([f64(p) for p in parts])
    assert np.array_equal(f64(out), want)


def test_partial_sum_strided_blocks():
    d = dev()
    step("partial sum with a padded rank stride")
    t, n, stride = 3, 4096, 4096 + 64
    buf = torch.randint(-8, 9, (t, stride), generator=torch.Generator().manual_seed(3)).to(BF16)
    out = torch.empty(n, dtype=BF16, device=d)
    lgs.shard_partial_sum("sum", t, n, buf.to(d), stride, out)
    sync()
    assert np.array_equal(f64(out), f64(buf[:, :n]).sum(axis=0))


# ------------------------------------------------------------ cross-entropy

def run_xent_all_ranks(H, E, y, b, s, t, with_argmax=True):
    """every rank's partials into stats [t, 3, M] and argmax [t, M]."""
    M, h = H.shape
    V = E.shape[0]
    Vr = V // t
    stats = torch.empty(t, 3, M, dtype=F32, device=H.device)
    am = torch.empty(t, M, dtype=torch.int32, device=H.device)
    for r in range(t):
        lgs.vocab_parallel_xent_fwd(b, s, h, V, t, r, H, E[r * Vr:(r + 1) * Vr], y, stats[r, 0],
                                    stats[r, 1], stats[r, 2], argmax_r=am[r] if with_argmax else None)
    return stats, am


def check_argmax(H64, E64_slice, vocab_start, got_ids, rows):
    """GPU argmax ids against fp64 logits: exact unless the top two are within
    the fp32 dot-product error bound (then any id inside that band is valid)."""
    K = H64.shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    z = H64[rows] @ E64_slice.T
    bound = gamma * (np.abs(H64[rows]) @ np.abs(E64_slice).T).max(axis=1)
    got = np.asarray(got_ids)[rows] - vocab_start
    zs = np.sort(z, axis=1)
    for i in range(len(rows)):
        top = z[i].max()
        assert 0 <= got[i] < z.shape[1], (rows[i], got[i])
        if zs[i, -1] - zs[i, -2] > 2 * bound[i]:
            assert got[i] == int(np.argmax(z[i])), (rows[i], got[i], int(np.argmax(z[i])))
        else:
            assert z[i, got[i]] >= top - 2 * bound[i]


@pytest.mark.parametrize("shape", [(1, 300, 72, 1400, 2), (2, 129, 136, 4 * 520, 4), (1, 64, 64, 8 * 136, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_xent_small_all_ranks(shape):
    b, s, h, V, t = shape
    M, Vr = b * s, V // t
    d = dev()
    H, E = synth.small(11 + h, (M, h), (V, h), dtype="bf16")
    E = (E.float() * 0.5).to(BF16)
    y = torch.randint(0, V, (M,), generator=torch.Generator().manual_seed(h), dtype=torch.int64).to(torch.int32)
    H64, E64 = f64(H), f64(E)
    step(f"xent small {shape}: all ranks")
    stats, am = run_xent_all_ranks(H.to(d), E.to(d), y.to(d), b, s, t)
    loss = torch.empty(M, dtype=F32, device=d)
    lgs.shard_partial_sum("xent", t, M, stats, 3 * M, loss)
    sync()
    stats_h, am_h = stats.cpu(), am.cpu().numpy()
    yn = y.numpy().astype(np.int64)
    for r in range(t):
        a, e = r * Vr, (r + 1) * Vr
        m, l, T, ids = oracle.xent.shard_partials(H64, E64[a:e], yn, a)
        assert_close(f"m_{r}", stats_h[r, 0], m, BF16)
        assert_close(f"l_{r}", stats_h[r, 1], l, BF16)
        own = (yn >= a) & (yn < e)
        assert_close(f"T_{r} (owned)", stats_h[r, 2][own], T[own], BF16)
        # not owned: exactly +0.0
        Tn = stats_h[r, 2].numpy()[~own]
        assert np.all(Tn == 0.0) and not np.any(np.signbit(Tn))
        check_argmax(H64, E64[a:e], a, am_h[r], np.arange(M))
    assert_close("loss (merged)", loss, oracle.xent.naive_loss(H64, E64, yn), BF16)
    # exactly one rank owns every target
    owners = np.stack([(yn >= r * Vr) & (yn < (r + 1) * Vr) for r in range(t)]).sum(axis=0)
    assert np.all(owners == 1) and np.array_equal(yn // Vr, np.argmax(
        np.stack([(yn >= r * Vr) & (yn < (r + 1) * Vr) for r in range(t)]), axis=0))


def test_xent_two_launch_plan_every_element():
    """A slice wide enough that the launch plan splits its columns (the first
    8320 on 256x320 tiles in one full round, the rest on 256x256 tiles): every
    token's partials, first argmax and loss against the oracle, with a K tail
    (h = 136) and a ragged row count; targets chosen on both sides of the
    split and on its boundary."""
    d = dev()
    b, s, h, V = 2, 1000, 136, 24640
    M = b * s
    H, E = synth.small(77, (M, h), (V, h), dtype="bf16")
    E = (E.float() * 0.3).to(BF16)
    g = torch.Generator().manual_seed(11)
    y = torch.randint(0, V, (M,), generator=g, dtype=torch.int64).to(torch.int32)
    y[:6] = torch.tensor([8319, 8320, 8321, 0, V - 1, 8448], dtype=torch.int32)  # 8448: a slab edge of the second launch
    step("xent t=1, slice split over two launches: every element")
    m = torch.empty(M, dtype=F32, device=d)
    l, T, loss = torch.empty_like(m), torch.empty_like(m), torch.empty_like(m)
    am = torch.empty(M, dtype=torch.int32, device=d)
    lgs.vocab_parallel_xent_fwd(b, s, h, V, 1, 0, H.to(d), E.to(d), y.to(d), m, l, T, argmax_r=am, loss=loss)
    sync()
    H64, E64, yn = f64(H), f64(E), y.numpy().astype(np.int64)
    rm, rl, rT, _ = oracle.xent.shard_partials(H64, E64, yn, 0)
    assert_close("m (split plan)", m, rm, BF16)
    assert_close("l (split plan)", l, rl, BF16)
    assert_close("T (split plan)", T, rT, BF16)
    assert_close("loss (split plan)", loss, oracle.xent.naive_loss(H64, E64, yn), BF16)
    check_argmax(H64, E64, 0, am.cpu().numpy(), np.arange(M))


def test_xent_t1_loss_output():
    d = dev()
    b, s, h, V = 1, 200, 128, 1000
    H, E = synth.small(21, (b * s, h), (V, h), dtype="bf16")
    E = (E.float() * 0.3).to(BF16)
    y = torch.randint(0, V, (b * s,), generator=torch.Generator().manual_seed(1)).to(torch.int32)
    step("xent t=1: loss written directly")
    m = torch.empty(b * s, dtype=F32, device=d)
    l, T, loss = torch.empty_like(m), torch.empty_like(m), torch.empty_like(m)
    am = torch.empty(b * s, dtype=torch.int32, device=d)
    lgs.vocab_parallel_xent_fwd(b, s, h, V, 1, 0, H.to(d), E.to(d), y.to(d), m, l, T, argmax_r=am, loss=loss)
    sync()
    assert_close("loss (t=1)", loss, oracle.xent.naive_loss(f64(H), f64(E), y.numpy()), BF16)
    check_argmax(f64(H), f64(E), 0, am.cpu().numpy(), np.arange(b * s))


def test_xent_uniform_embedding_gives_ln_v():
    d = dev()
    b, s, h, V, t = 1, 64, 64, 8 * 640, 8
    H = synth.small(3, (b * s, h), dtype="bf16")[0].to(d)
    E = torch.zeros(V, h, dtype=BF16, device=d)
    y = torch.arange(b * s, dtype=torch.int32, device=d) * 79
    step("xent with E = 0: loss = ln V")
    stats, am = run_xent_all_ranks(H, E, y, b, s, t)
    loss = torch.empty(b * s, dtype=F32, device=d)
    lgs.shard_partial_sum("xent", t, b * s, stats, 3 * b * s, loss)
    sync()
    st = stats.cpu().numpy()
    assert np.all(st[:, 0] == 0.0) and np.all(st[:, 1] == V // t) and np.all(st[:, 2] == 0.0)
    assert np.all(am.cpu().numpy() == (np.arange(t) * (V // t))[:, None])  # ties -> lowest id
    assert np.abs(loss.cpu().numpy() - math.log(V)).max() < 1e-6 * math.log(V)


@pytest.mark.parametrize("c", [256.0, 1000.0, 4096.0])
def test_xent_shift_invariance_large_logits(c):
    """H[:, 0] = c and E[:, 0] = 1 add c to every logit: the loss must not
    change (the partials are taken relative to each slab's maximum, so
    exp never sees the raw logit).  Compared with the oracle on the same
    inputs and with the oracle's loss for the unshifted logits (H[:, 0] = 0)."""
    d = dev()
    b, s, h, V, t = 1, 160, 64, 4 * 448, 4
    H, E = synth.small(37, (b * s, h), (V, h), dtype="bf16")
    E = (E.float() * 0.5).to(BF16)
    H[:, 0] = c
    E[:, 0] = 1.0
    y = torch.randint(0, V, (b * s,), generator=torch.Generator().manual_seed(3)).to(torch.int32)
    step(f"xent with every logit shifted by {c}")
    stats, _ = run_xent_all_ranks(H.to(d), E.to(d), y.to(d), b, s, t)
    loss = torch.empty(b * s, dtype=F32, device=d)
    lgs.shard_partial_sum("xent", t, b * s, stats, 3 * b * s, loss)
    sync()
    got = loss.cpu().numpy()
    assert np.all(np.isfinite(got))
    H64, E64, yn = f64(H), f64(E), y.numpy()
    assert_close("loss (shifted logits)", got, oracle.xent.naive_loss(H64, E64, yn), BF16)
    H0 = H64.copy()
    H0[:, 0] = 0.0
    # fp32 accumulation near c keeps about 24 - log2(c) bits of each logit's fraction
    assert np.abs(got - oracle.xent.naive_loss(H0, E64, yn)).max() < 2e-2 * np.abs(got).max()
    assert np.all(stats.cpu().numpy()[:, 0] > c - 64)  # the slice maxima carry the shift


def test_xent_nan_row_stays_in_its_token():
    d = dev()
    b, s, h, V, t = 1, 96, 64, 2 * 512, 2
    H, E = synth.small(31, (b * s, h), (V, h), dtype="bf16")
    H[5, 3] = float("nan")
    y = torch.randint(0, V, (b * s,), generator=torch.Generator().manual_seed(2)).to(torch.int32)
    step("xent with a NaN in one hidden row")
    stats, _ = run_xent_all_ranks(H.to(d), E.to(d), y.to(d), b, s, t)
    loss = torch.empty(b * s, dtype=F32, device=d)
    lgs.shard_partial_sum("xent", t, b * s, stats, 3 * b * s, loss)
    sync()
    got = loss.cpu().numpy()
    assert np.isnan(got[5])
    keep = np.arange(b * s) != 5
    ref = oracle.xent.naive_loss(f64(H)[keep], f64(E), y.numpy()[keep])
    assert np.all(np.isfinite(got[keep]))
    assert_close("loss (other tokens)", got[keep], ref, BF16)


@pytest.mark.parametrize("t", [1, 3, 8, 9, 16, 21])
def test_xent_merge_kernel_matches_oracle_merge(t):
    """The combine takes ranks in chunks of eight: t past 8 merges chunks with
    the online identity; t <= 8 is one pass."""
    d = dev()
    n = 5000
    g = np.random.default_rng(4 + t)
    m = g.normal(size=(t, n)) * 5
    l = g.uniform(1, 100, size=(t, n))
    T = np.where(g.uniform(size=(t, n)) < 1 / t, g.normal(size=(t, n)), 0.0)
    parts = torch.from_numpy(np.stack([m, l, T], axis=1).astype(np.float32)).to(d)
    step(f"xent merge kernel, t={t}")
    out = torch.empty(n, dtype=F32, device=d)
    lse = torch.empty(n, dtype=F32, device=d)
    lgs.shard_partial_sum("xent", t, n, parts, 3 * n, out)
    lgs.shard_partial_sum("xent_lse", t, n, parts, 3 * n, lse)
    sync()
    p32 = parts.cpu().double().numpy()
    assert_close("merge", out, oracle.xent.merge(p32[:, 0], p32[:, 1], p32[:, 2]), F32)
    assert_close("lse", lse, oracle.xent.merge_lse(p32[:, 0], p32[:, 1]), F32)


# ------------------------------------------------------ degenerate sizes

@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("M", [1, 2, 9])
def test_single_token_and_tiny_batches(M, dtype):
    """One to nine tokens through the whole path: MLP forward and backward
    (the weight gradients then have K = M), the sums, and the fused CE with
    its combine."""
    d = dev()
    h, ffn, t, V = 64, 256, 2, 2 * 160
    dn = "bf16" if dtype == BF16 else "f32"
    X, A, B, dZ = synth.small(500 + M, (M, h), (h, ffn), (ffn, h), (M, h), dtype=dn)
    A, B = (A.float() * 0.1).to(dtype), (B.float() * 0.1).to(dtype)
    X64, A64, B64, dZ64 = f64(X), f64(A), f64(B), f64(dZ)
    Xd, Ad, Bd, dZd = X.to(d), A.to(d), B.to(d), dZ.to(d)
    f = ffn // t
    parts = torch.empty(t, M, h, dtype=dtype, device=d)
    for r in range(t):
        step(f"{M} token(s) {dn}: rank {r} forward and backward")
        U, Y, Z = run_fwd(Xd, Ad, Bd, 1, M, t, r, "erf")
        parts[r].copy_(Z)
        dX, dA, dB = run_bwd(Xd, Ad, Bd, U, dZd, 1, M, t, r, "erf")
        sync()
        A_i, B_i = A64[:, r * f:(r + 1) * f], B64[r * f:(r + 1) * f]
        rU, rY, rZ = oracle.mlp.shard_forward(X64, A_i, B_i, "erf")
        assert_close("Z_i", Z, rZ, dtype)
        ref = oracle.mlp.shard_backward(X64, A_i, B_i, f64(U), dZ64, "erf")
        assert_close("dX_i", dX, ref["dX"], dtype)
        assert_close("dA_i", dA, ref["dA"], dtype)
        assert_close("dB_i", dB, ref["dB"], dtype)
    Zs = torch.empty(M, h, dtype=dtype, device=d)
    lgs.shard_partial_sum("sum", t, M * h, parts, M * h, Zs)
    sync()
    assert_close("sum of partials", Zs, oracle.mlp.mlp_forward(X64, A64, B64, "erf")[2], dtype)
    if dtype == BF16:
        H, E = synth.small(600 + M, (M, h), (V, h), dtype="bf16")
        y = (torch.arange(M, dtype=torch.int32) * 37 + 5) % V
        step(f"{M} token(s): fused CE, {t} ranks")
        stats, _ = run_xent_all_ranks(H.to(d), E.to(d), y.to(d), 1, M, t)
        loss = torch.empty(M, dtype=F32, device=d)
        lgs.shard_partial_sum("xent", t, M, stats, 3 * M, loss)
        sync()
        assert_close("loss", loss, oracle.xent.naive_loss(f64(H), f64(E), y.numpy()), BF16)


# -------------------------------------------------- full sizes, every element
#
# The benchmarked workloads in the benchmark's launch configuration, every
# output element against the fp64 oracle (a few TFLOP of host fp64 work in
# all, seconds per test).

_cache = {}


def _mlp_inputs(name):
    if name not in _cache:
        _cache.clear()
        w = WORKLOADS[name]
        X, A, B = synth.mlp_weights(w)
        _cache[name] = (w, X, A, B)
    return _cache[name]


@pytest.mark.parametrize("name", ["mlp_8p3b_fwd", "mlp_70b_fwd"])
@pytest.mark.parametrize("which", ["rank0", "last_rank"])
def test_full_size_forward(name, which):
    w, X, A, B = _mlp_inputs(name)
    d = dev()
    f = w.f_i
    r = 0 if which == "rank0" else w.t - 1
    step(f"{name}: rank {r} forward at full size")
    U, Y, Z = run_fwd(X.to(d), A.to(d), B.to(d), w.b, w.s, w.t, r, "erf")
    sync()
    step(f"{name}: oracle forward of rank {r} (host fp64), every element")
    rU, rY, rZ = oracle.mlp.shard_forward(f64(X), f64(A[:, r * f:(r + 1) * f]), f64(B[r * f:(r + 1) * f]))
    assert_close(f"U_{r}", U, rU, BF16)
    assert_close(f"Y_{r}", Y, rY, BF16)
    assert_close(f"Z_{r}", Z, rZ, BF16)


@pytest.mark.parametrize("name", ["mlp_8p3b_fwd", "mlp_70b_fwd"])
def test_full_size_all_shards_sum_to_unsplit(name):
    """All t ranks' forward shards at full size, summed on the device: every
    element of the sum against the oracle's unsplit block ("Row-Parallel
    Linear Layer": Z = sum_i Z_i)."""
    w, X, A, B = _mlp_inputs(name)
    d = dev()
    Xd, Ad, Bd = X.to(d), A.to(d), B.to(d)
    parts = torch.empty(w.t, w.M, w.h, dtype=BF16, device=d)
    f = w.f_i
    step(f"{name}: all {w.t} ranks + on-device sum")
    Y = torch.empty(w.M, f, dtype=BF16, device=d)
    for r in range(w.t):
        lgs.tp_mlp_fwd(w.b, w.s, w.h, w.ffn, w.t, r, Xd, Ad[:, r * f:(r + 1) * f], Bd[r * f:(r + 1) * f],
                       parts[r], Y_i=Y)
    Z = torch.empty(w.M, w.h, dtype=BF16, device=d)
    lgs.shard_partial_sum("sum", w.t, w.M * w.h, parts, w.M * w.h, Z)
    sync()
    del parts, Xd, Ad, Bd
    step(f"{name}: oracle unsplit block (host fp64), every element")
    ref = oracle.mlp.mlp_forward(f64(X), f64(A), f64(B))[2]
    assert_close("sum_i Z_i vs unsplit Z", Z, ref, BF16)


@pytest.mark.parametrize("name,which", [("mlp_70b_bwd", "rank0"), ("mlp_70b_bwd", "last_rank"),
                                        ("mlp_8p3b_fwd", "rank0"), ("mlp_8p3b_fwd", "last_rank")])
def test_full_size_backward(name, which):
    """One rank's backward at full size (the 70B workload; the 8.3B shapes
    with dZ ~ N(0, 0.01) from seed 9): every element of dX_i, dA_i, dB_i."""
    w = WORKLOADS[name]
    _, X, A, B = _mlp_inputs("mlp_70b_fwd" if name == "mlp_70b_bwd" else name)
    d = dev()
    f = w.f_i
    r = 0 if which == "rank0" else w.t - 1
    A_i64, B_i64, X64 = f64(A[:, r * f:(r + 1) * f]), f64(B[r * f:(r + 1) * f]), f64(X)
    step(f"{name}: oracle U_{r} = X A_{r} in fp64 (host), rounded to bf16")
    U = round_like(X64 @ A_i64, BF16)
    dZ = synth.mlp_grad(w) if w.dz_std else synth.normal((w.M, w.h), 0.01, 9, "bf16")
    step(f"{name}: rank {r} backward at full size")
    dX, dA, dB = run_bwd(X.to(d), A.to(d), B.to(d), U.to(d), dZ.to(d), w.b, w.s, w.t, r, "erf")
    sync()
    step(f"{name}: oracle backward of rank {r} (host fp64), every element")
    g = oracle.mlp.shard_backward(X64, A_i64, B_i64, f64(U), f64(dZ))
    assert_close(f"dX_{r}", dX, g["dX"], BF16)
    assert_close(f"dA_{r}", dA, g["dA"], BF16)
    assert_close(f"dB_{r}", dB, g["dB"], BF16)


def check_argmax_given_logits(z, H64, E64_slice, vocab_start, got_ids):
    """check_argmax for every row, with the slice's fp64 logits z already
    computed.  A row whose top two logits differ by more than twice a cheap
    upper bound on its error bound (gamma_K * sum_k |h_k| max_j |e_jk|) must
    match exactly; only the remaining rows get the exact bound."""
    M, Vr = z.shape
    K = H64.shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    got = np.asarray(got_ids).astype(np.int64) - vocab_start
    assert np.all((got >= 0) & (got < Vr))
    top = z.max(axis=1)
    second = np.partition(z, Vr - 2, axis=1)[:, Vr - 2]
    loose = gamma * (np.abs(H64) @ np.abs(E64_slice).max(axis=0))
    far = (top - second) > 2 * loose
    exact = np.argmax(z, axis=1)
    assert np.array_equal(got[far], exact[far]), np.nonzero(got[far] != exact[far])[0][:8]
    near = np.nonzero(~far)[0]
    if near.size:
        bound = gamma * (np.abs(H64[near]) @ np.abs(E64_slice).T).max(axis=1)
        zn, gn = z[near], got[near]
        assert np.all(zn[np.arange(near.size), gn] >= top[near] - 2 * bound)
        sure = (top[near] - second[near]) > 2 * bound
        assert np.array_equal(gn[sure], exact[near][sure])
    return int(near.size)


def test_full_size_xent_all_ranks():
    """Every rank of the 8.3B-shape vocabulary at full size: m_r, l_r, T_r and
    the first argmax of every token against the oracle on the same logits,
    exact target ownership, and the merged loss of all 8192 tokens against
    the naive full-logit loss ("LIT-022", "Key takeaways": fused == naive)."""
    w = WORKLOADS["xent_8p3b"]
    d = dev()
    H, E, y = synth.xent_inputs(w)
    step("xent_8p3b: all 8 ranks at full size")
    stats, am = run_xent_all_ranks(H.to(d), E.to(d), y.to(d), w.b, w.s, w.t)
    loss = torch.empty(w.M, dtype=F32, device=d)
    lgs.shard_partial_sum("xent", w.t, w.M, stats, 3 * w.M, loss)
    sync()
    st, amh, yn = stats.cpu(), am.cpu().numpy(), y.numpy().astype(np.int64)
    Vr = w.v_r
    H64, E64 = f64(H), f64(E)
    for r in range(w.t):
        a = r * Vr
        step(f"xent_8p3b: oracle logits and partials of rank {r} (host fp64), every token")
        z = H64 @ E64[a:a + Vr].T
        m, l, T, _ = oracle.xent.slice_partials(z, yn, a)
        assert_close(f"m_{r}", st[r, 0], m, BF16)
        assert_close(f"l_{r}", st[r, 1], l, BF16)
        own = (yn // Vr) == r
        assert_close(f"T_{r} (owned)", st[r, 2][own], T[own], BF16)
        Tn = st[r, 2].numpy()[~own]
        assert np.all(Tn == 0.0) and not np.any(np.signbit(Tn))  # not owned: exactly +0.0
        near = check_argmax_given_logits(z, H64, E64[a:a + Vr], a, amh[r])
        print(f"    argmax_{r}: exact on every token, {near} token(s) checked against the near-tie band",
              flush=True)
        del z
    step("xent_8p3b: oracle naive full-logit loss (host fp64), every token")
    assert_close("loss (all tokens)", loss, oracle.xent.naive_loss(H64, E64, yn), BF16)
    # without the optional argmax (the training step's call) the partials are the same bits
    Hd, Ed, yd = H.to(d), E.to(d), y.to(d)
    for r in (0, w.t - 1):
        part = torch.empty(3, w.M, dtype=F32, device=d)
        lgs.vocab_parallel_xent_fwd(w.b, w.s, w.h, w.vocab, w.t, r, Hd, Ed[r * Vr:(r + 1) * Vr], yd,
                                    part[0], part[1], part[2], argmax_r=None)
        sync()
        assert torch.equal(part.cpu(), st[r]), r


# ------------------------------- streaming form of the CE reductions (testing)

def _rows_partials(Z, y, start):
    d = dev()
    M = Z.shape[0]
    out = torch.empty(3, M, dtype=F32, device=d)
    lgs.xent_rows_bf16(Z.to(d), y.to(d), start, out[0], out[1], out[2])
    sync()
    return out.cpu()


# Vr / 8 chunks per row against 448 per batch: a tail alone (1000), one full batch and a tail
# (6400, 3592), two full batches and no tail (7168), one chunk (8)
@pytest.mark.parametrize("M,Vr,start", [(300, 1000, 0), (65, 6400, 6400), (17, 3592, 0), (70, 7168, 7168),
                                        (1, 8, 3)])
def test_xent_rows_match_oracle_slice_partials(M, Vr, start):
    """bf16 logits of H E_r^T (ragged row counts, chunk counts that are not a
    multiple of the wave) -> the oracle's slice partials on the same logits."""
    h = 64
    H, E = synth.small(11, (M, h), (Vr, h), std=0.5)
    Z = round_like(f64(H) @ f64(E).T, BF16)
    g = torch.Generator().manual_seed(3)
    y = torch.randint(max(0, start - Vr // 2), start + Vr + Vr // 2, (M,), generator=g).to(torch.int32)
    step(f"xent rows M={M} Vr={Vr} start={start}")
    got = _rows_partials(Z, y, start)
    m, l, T, _ = oracle.xent.slice_partials(f64(Z), y.numpy(), start)
    assert np.array_equal(f64(got[0]), m)              # a max of bf16 values is exact
    assert np.array_equal(f64(got[2]), T)              # so is the picked logit, or +0.0
    assert not np.any(np.signbit(f64(got[2])[T == 0.0]))
    assert_close("l", got[1], l, F32)


def test_xent_rows_special_rows():
    d = dev()
    Vr = 256
    Z = torch.zeros(4, Vr, dtype=BF16)
    Z[1] = 3.0                                  # all equal: l = Vr
    Z[2, 17] = float("nan")                     # a NaN poisons the sum only
    Z[3] = float("-inf")
    Z[3, 5] = 1.0                               # one finite logit: l = 1
    y = torch.tensor([0, 1, 17, 5], dtype=torch.int32)
    step("xent rows special rows")
    got = _rows_partials(Z, y, 0).numpy()
    # exp(z - m) is evaluated as 2^(z log2e - m log2e) with one fma: equal
    # logits give 1 up to the rounding of m log2e
    assert got[0, 1] == 3.0 and abs(got[1, 1] - Vr) <= 1e-6 * Vr
    assert got[0, 2] == 0.0 and np.isnan(got[1, 2]) and np.isnan(got[2, 2])
    assert got[0, 3] == 1.0 and got[1, 3] == 1.0 and got[2, 3] == 1.0


def test_xent_rows_full_size():
    """The streaming kernel over the rank-0 slice's materialised logits
    (8192 x 6400, the benchmark's buffer shape), every row."""
    w = WORKLOADS["xent_8p3b"]
    H, E, y = synth.xent_inputs(w)
    d = dev()
    Zd = (H.to(d).float() @ E[:w.v_r].to(d).float().t().contiguous()).to(BF16)  # rank-0 slice logits
    step("xent rows at full size (8192 x 6400)")
    out = torch.empty(3, w.M, dtype=F32, device=d)
    lgs.xent_rows_bf16(Zd, y.to(d), 0, out[0], out[1], out[2])
    sync()
    m, l, T, _ = oracle.xent.slice_partials(f64(Zd.cpu()), y.numpy(), 0)
    got = out.cpu()
    assert np.array_equal(f64(got[0]), m) and np.array_equal(f64(got[2]), T)
    assert_close("l (every row)", got[1], l, F32)


# ------------------------------------------------- the epilogue's GeLU math

@pytest.mark.parametrize("act", ["erf", "tanh"])
def test_gelu_epilogue_error_bound(act):
    """fp32 path with X = I, dZ = I, B_i = 1: then U = A_i exactly, the
    backward's dA_i = GeLU'(U) and dB_i = GeLU(U)^T exactly (one nonzero
    product per sum), which isolates the device GeLU / GeLU' evaluation.
    The last row holds large magnitudes, where both forms saturate (the erf
    tail and exp(-u^2/2) underflow to 0; the tanh form's exp(2a) overflows
    or underflows): GeLU(u) must be u or 0 and GeLU'(u) 1 or 0 there."""
    d = dev()
    n = 64
    u = torch.linspace(-10.0, 10.0, n * n, dtype=F32).reshape(n, n)
    big = torch.tensor([-1e4, -1e3, -100.0, -40.0, -30.0, -20.0, -15.0, -12.0,
                        12.0, 15.0, 20.0, 30.0, 40.0, 100.0, 1e3, 1e4], dtype=F32)
    u[-1] = big.repeat(n // big.numel())
    eye = torch.eye(n, dtype=F32)
    step(f"GeLU epilogue error bound ({act})")
    U, Y, Z = run_fwd(eye.to(d), u.to(d), torch.ones(n, n, dtype=F32, device=d), 1, n, 1, 0, act)
    dX, dA, dB = run_bwd(eye.to(d), u.to(d), torch.ones(n, n, dtype=F32, device=d), u.to(d), eye.to(d),
                         1, n, 1, 0, act)
    sync()
    u64 = f64(u)
    bound = 4e-7 * np.maximum(1.0, np.abs(u64))
    assert np.array_equal(f64(U), u64)
    for name, got, ref in (("Y", f64(Y), oracle.mlp.gelu(u64, act)),
                           ("dB^T", f64(dB).T, oracle.mlp.gelu(u64, act)),
                           ("dA", f64(dA), oracle.mlp.gelu_grad(u64, act))):
        err = np.abs(got - ref)
        print(f"    {name}: max |err| = {err.max():.2e}, max |err|/bound = {(err / bound).max():.2f}", flush=True)
        assert np.all(err <= bound), name

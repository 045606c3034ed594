"""Guard bands around every output: nothing is written outside it.

Every output of the entry points (and their workspaces) lives inside a
larger buffer filled with a sentinel bit pattern: a guard band before and
after it and, for matrices, a leading dimension wider than the row, so
that the gaps between rows are guarded too.  After the call every sentinel
element must hold its bits, and the outputs must equal, bit for bit, those
of the same call into dense, exactly sized outputs.  The shapes are ragged
(partial tiles in M, N and K) so that the kernels' edge handling is what
these checks exercise.
"""

import pytest
import torch

from gpu_util import dev, step
from logit_gemm_shard_amd import binding as lgs
from logit_gemm_shard_amd import synth

pytestmark = pytest.mark.gpu

BF16, F32, I32 = torch.bfloat16, torch.float32, torch.int32
_BITS = {BF16: (torch.int16, 0x7FA5), F32: (torch.int32, 0x7FC0BEEF), I32: (torch.int32, 0x5A5A5A5A),
         torch.uint8: (torch.uint8, 0xA5)}
GUARD = 512  # elements before and after (a multiple of 128: keeps 256-byte alignment)


class Guarded:
    """An output of shape (rows, width) or (n,) inside a sentinel-filled
    buffer; `t` is the view passed to the library."""

    def __init__(self, shape, dtype, pad=24):
        d = dev()
        self.dtype = dtype
        if len(shape) == 2:
            rows, width = shape
            ld = width + pad
            self.buf = torch.empty(2 * GUARD + rows * ld, dtype=dtype, device=d)
            self.t = self.buf[GUARD:GUARD + rows * ld].view(rows, ld)[:, :width]
            inside = torch.zeros(rows, ld, dtype=torch.bool, device=d)
            inside[:, :width] = True
            self.inside = torch.cat([torch.zeros(GUARD, dtype=torch.bool, device=d), inside.reshape(-1),
                                     torch.zeros(GUARD, dtype=torch.bool, device=d)])
        else:
            (n,) = shape
            self.buf = torch.empty(2 * GUARD + n, dtype=dtype, device=d)
            self.t = self.buf[GUARD:GUARD + n]
            self.inside = torch.zeros(2 * GUARD + n, dtype=torch.bool, device=d)
            self.inside[GUARD:GUARD + n] = True
        idt, pat = _BITS[dtype]
        self.bits = self.buf.view(idt)
        if idt == torch.int16 and pat > 0x7FFF:
            pat -= 1 << 16
        self.pat = pat
        self.bits.fill_(pat)

    def check(self, name):
        bad = (self.bits != self.pat) & ~self.inside
        n = int(bad.sum())
        assert n == 0, f"{name}: {n} element(s) written outside the output (first at buffer index " \
                       f"{int(bad.nonzero()[0])})"


def workspace(nbytes):
    """A workspace of exactly nbytes with a guard band after it (256-byte aligned)."""
    return Guarded((nbytes,), torch.uint8, pad=0)


def same(name, got, ref):
    assert torch.equal(got, ref), f"{name}: differs from the call into dense outputs"


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 200, 136, 528, 2), (2, 1100, 1064, 2 * 1048, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_guard_mlp_fwd_bwd(shape, dtype):
    b, s, h, ffn, t = shape
    M, f, r = b * s, ffn // t, t - 1
    d = dev()
    dn = "bf16" if dtype == BF16 else "f32"
    X, A, B, dZ = synth.small(17 + h, (M, h), (h, ffn), (ffn, h), (M, h), dtype=dn)
    A, B = (A.float() * 0.05).to(dtype).to(d), (B.float() * 0.05).to(dtype).to(d)
    X, dZ = X.to(d), dZ.to(d)
    A_i, B_i = A[:, r * f:(r + 1) * f], B[r * f:(r + 1) * f]
    step(f"guard bands: MLP forward and backward {shape} {dn}")
    U, Y, Z = (torch.empty(M, n, dtype=dtype, device=d) for n in (f, f, h))
    lgs.tp_mlp_fwd(b, s, h, ffn, t, r, X, A_i, B_i, Z, U_i=U, Y_i=Y)
    gU, gY, gZ = Guarded((M, f), dtype), Guarded((M, f), dtype), Guarded((M, h), dtype)
    lgs.tp_mlp_fwd(b, s, h, ffn, t, r, X, A_i, B_i, gZ.t, U_i=gU.t, Y_i=gY.t)
    # Y kept in the workspace instead (the call carves it out of the workspace)
    wf = workspace(lgs.mlp_fwd_workspace_bytes(b, s, h, ffn, t, dtype, False))
    gZ2 = Guarded((M, h), dtype)
    lgs.tp_mlp_fwd(b, s, h, ffn, t, r, X, A_i, B_i, gZ2.t, workspace=wf.t)
    dX, dA, dB = torch.empty(M, h, dtype=dtype, device=d), torch.empty(h, f, dtype=dtype, device=d), \
        torch.empty(f, h, dtype=dtype, device=d)
    lgs.tp_mlp_bwd(b, s, h, ffn, t, r, X, A_i, B_i, U, dZ, dX, dA, dB)
    gdX, gdA, gdB = Guarded((M, h), dtype), Guarded((h, f), dtype), Guarded((f, h), dtype)
    wb = workspace(lgs.mlp_bwd_workspace_bytes(b, s, h, ffn, t, dtype))
    lgs.tp_mlp_bwd(b, s, h, ffn, t, r, X, A_i, B_i, U, dZ, gdX.t, gdA.t, gdB.t, workspace=wb.t)
    torch.cuda.synchronize()
    for name, g, ref in (("U", gU, U), ("Y", gY, Y), ("Z", gZ, Z), ("Z (Y in workspace)", gZ2, Z),
                         ("dX", gdX, dX), ("dA", gdA, dA), ("dB", gdB, dB)):
        g.check(name)
        same(name, g.t, ref)
    wf.check("forward workspace")
    wb.check("backward workspace")


def test_guard_mlp_bwd_three_parts():
    b, s, h, ffn, t = 2, 1100, 1064, 2 * 1048, 2
    M, f = b * s, ffn // t
    d = dev()
    X, A, B, dZ, U = synth.small(23, (M, h), (h, f), (f, h), (M, h), (M, f), dtype="bf16")
    A, B = (A.float() * 0.05).to(BF16).to(d), (B.float() * 0.05).to(BF16).to(d)
    X, dZ, U = X.to(d), dZ.to(d), U.to(d)
    step("guard bands: the backward in three parts")
    ws = workspace(lgs.mlp_bwd_workspace_bytes(b, s, h, ffn, t, BF16))
    gdX, gdA, gdB = Guarded((M, h), BF16), Guarded((h, f), BF16), Guarded((f, h), BF16)
    lgs.tp_mlp_bwd_dgelu(b, s, h, ffn, t, 0, B, U, dZ, ws.t)
    lgs.tp_mlp_bwd_dx(b, s, h, ffn, t, 0, A, gdX.t, ws.t)
    lgs.tp_mlp_bwd_dw(b, s, h, ffn, t, 0, X, dZ, gdA.t, gdB.t, ws.t)
    torch.cuda.synchronize()
    for name, g in (("dX", gdX), ("dA", gdA), ("dB", gdB)):
        g.check(name)
    ws.check("shared workspace")


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_guard_xent_fwd(noalloc):
    b, s, h, V, t = 2, 129, 136, 4 * 520, 4
    M, Vr = b * s, V // t
    d = dev()
    H, E = synth.small(13, (M, h), (V, h), dtype="bf16")
    E = (E.float() * 0.5).to(BF16)
    H, E = H.to(d), E.to(d)
    y = torch.randint(0, V, (M,), generator=torch.Generator().manual_seed(2)).to(I32).to(d)
    fn = lgs.vocab_parallel_xent_fwd_noalloc if noalloc else lgs.vocab_parallel_xent_fwd
    for r in (0, t - 1):
        step(f"guard bands: fused CE partials, rank {r} ({'noalloc' if noalloc else 'workspace'})")
        ref = [torch.empty(M, dtype=F32, device=d) for _ in range(3)] + [torch.empty(M, dtype=I32, device=d)]
        lgs.vocab_parallel_xent_fwd(b, s, h, V, t, r, H, E[r * Vr:(r + 1) * Vr], y, *ref[:3], argmax_r=ref[3])
        g = [Guarded((M,), F32) for _ in range(3)] + [Guarded((M,), I32)]
        kw, wsg = {}, None
        if not noalloc:
            wsg = workspace(lgs.xent_workspace_bytes(b, s, h, V, t))
            kw = {"workspace": wsg.t}
        fn(b, s, h, V, t, r, H, E[r * Vr:(r + 1) * Vr], y, g[0].t, g[1].t, g[2].t, argmax_r=g[3].t, **kw)
        torch.cuda.synchronize()
        for name, gg, rr in zip(("m", "l", "T", "argmax"), g, ref):
            gg.check(name)
            same(name, gg.t, rr)
        if wsg is not None:
            wsg.check("CE workspace")
    # t = 1 with the loss output
    step("guard bands: fused CE, t = 1 with the loss")
    ref = [torch.empty(M, dtype=F32, device=d) for _ in range(4)]
    lgs.vocab_parallel_xent_fwd(b, s, h, Vr, 1, 0, H, E[:Vr], y % Vr, *ref[:3], loss=ref[3])
    g = [Guarded((M,), F32) for _ in range(4)]
    fn(b, s, h, Vr, 1, 0, H, E[:Vr], y % Vr, g[0].t, g[1].t, g[2].t, loss=g[3].t)
    torch.cuda.synchronize()
    for name, gg, rr in zip(("m", "l", "T", "loss"), g, ref):
        gg.check(name)
        same(name, gg.t, rr)


def test_guard_xent_bwd():
    b, s, h, V, t = 1, 200, 136, 2 * 392, 2
    M, Vr = b * s, V // t
    d = dev()
    H, E = synth.small(8, (M, h), (V, h), dtype="bf16")
    H, E = H.to(d), E.to(d)
    y = torch.randint(0, V, (M,), generator=torch.Generator().manual_seed(5)).to(I32).to(d)
    lse = torch.randn(M, device=d).abs_().add_(3.0)
    step("guard bands: CE backward")
    dH, dE = torch.empty(M, h, dtype=BF16, device=d), torch.empty(Vr, h, dtype=BF16, device=d)
    lgs.vocab_parallel_xent_bwd(b, s, h, V, t, 1, H, E[Vr:], y, lse, dH, dE)
    gH, gE = Guarded((M, h), BF16), Guarded((Vr, h), BF16)
    ws = workspace(lgs.xent_bwd_workspace_bytes(b, s, h, V, t))
    lgs.vocab_parallel_xent_bwd(b, s, h, V, t, 1, H, E[Vr:], y, lse, gH.t, gE.t, workspace=ws.t)
    torch.cuda.synchronize()
    gH.check("dH")
    gE.check("dE")
    ws.check("CE backward workspace")
    same("dH", gH.t, dH)
    same("dE", gE.t, dE)


@pytest.mark.parametrize("n", [1001, 8192 + 8])
@pytest.mark.parametrize("din,dout", [(BF16, BF16), (F32, F32), (BF16, F32)])
def test_guard_partial_sums(n, din, dout):
    d = dev()
    t = 3
    step(f"guard bands: sum of partials t={t} n={n} {din}->{dout}")
    parts = torch.randint(-16, 17, (t, n), generator=torch.Generator().manual_seed(n)).to(din).to(d)
    ref = torch.empty(n, dtype=dout, device=d)
    lgs.shard_partial_sum("sum", t, n, parts, n, ref)
    g = Guarded((n,), dout)
    lgs.shard_partial_sum("sum", t, n, parts, n, g.t)
    torch.cuda.synchronize()
    g.check("sum")
    same("sum", g.t, ref)


@pytest.mark.parametrize("op", ["xent", "xent_lse"])
def test_guard_xent_combine(op):
    d = dev()
    t, n = 9, 1001
    gen = torch.Generator().manual_seed(9)
    parts = torch.stack([torch.randn(t, n, generator=gen), torch.rand(t, n, generator=gen) * 9 + 1,
                         torch.randn(t, n, generator=gen)], dim=1).to(d)
    step(f"guard bands: CE combine ({op})")
    ref = torch.empty(n, dtype=F32, device=d)
    lgs.shard_partial_sum(op, t, n, parts, 3 * n, ref)
    g = Guarded((n,), F32)
    lgs.shard_partial_sum(op, t, n, parts, 3 * n, g.t)
    torch.cuda.synchronize()
    g.check(op)
    same(op, g.t, ref)


def test_guard_sequence_parallel():
    d = dev()
    t, s, b, h = 4, 12, 3, 72
    n, chunk = s * b * h, s * b * h // t
    step("guard bands: reduce-scatter and all-gather")
    parts = torch.randint(-8, 9, (t, n), generator=torch.Generator().manual_seed(4)).to(BF16).to(d)
    for r in range(t):
        ref = torch.empty(chunk, dtype=BF16, device=d)
        lgs.shard_reduce_scatter(t, r, s, b, h, parts, n, ref)
        g = Guarded((chunk,), BF16)
        lgs.shard_reduce_scatter(t, r, s, b, h, parts, n, g.t)
        torch.cuda.synchronize()
        g.check(f"reduce-scatter rank {r}")
        same("reduce-scatter", g.t, ref)
    shards = torch.randn(t, chunk + 40, device=d).to(BF16)
    ref = torch.empty(n, dtype=BF16, device=d)
    lgs.shard_all_gather(t, s, b, h, shards, chunk + 40, ref)
    g = Guarded((n,), BF16)
    lgs.shard_all_gather(t, s, b, h, shards, chunk + 40, g.t)
    torch.cuda.synchronize()
    g.check("all-gather")
    same("all-gather", g.t, ref)


def test_guard_swiglu():
    b, s, h, ffn, t, r = 1, 520, 328, 3 * 208, 3, 2
    M, f = b * s, ffn // t
    d = dev()
    X, Wgu, Wd, dZ = synth.small(31, (M, h), (h, 2 * f), (f, h), (M, h), dtype="bf16")
    Wgu, Wd = (Wgu.float() * 0.05).to(BF16).to(d), (Wd.float() * 0.05).to(BF16).to(d)
    X, dZ = X.to(d), dZ.to(d)
    step("guard bands: SwiGLU forward and backward")
    GU, Y, Z = torch.empty(M, 2 * f, dtype=BF16, device=d), torch.empty(M, f, dtype=BF16, device=d), \
        torch.empty(M, h, dtype=BF16, device=d)
    lgs.tp_swiglu_fwd(b, s, h, ffn, t, r, X, Wgu, Wd, Z, GU_i=GU, Y_i=Y)
    gGU, gY, gZ = Guarded((M, 2 * f), BF16), Guarded((M, f), BF16), Guarded((M, h), BF16)
    lgs.tp_swiglu_fwd(b, s, h, ffn, t, r, X, Wgu, Wd, gZ.t, GU_i=gGU.t, Y_i=gY.t)
    dX, dW, dD = torch.empty(M, h, dtype=BF16, device=d), torch.empty(h, 2 * f, dtype=BF16, device=d), \
        torch.empty(f, h, dtype=BF16, device=d)
    lgs.tp_swiglu_bwd(b, s, h, ffn, t, r, X, Wgu, Wd, GU, dZ, dX, dW, dD)
    gdX, gdW, gdD = Guarded((M, h), BF16), Guarded((h, 2 * f), BF16), Guarded((f, h), BF16)
    ws = workspace(lgs.swiglu_bwd_workspace_bytes(b, s, h, ffn, t, BF16))
    lgs.tp_swiglu_bwd(b, s, h, ffn, t, r, X, Wgu, Wd, GU, dZ, gdX.t, gdW.t, gdD.t, workspace=ws.t)
    torch.cuda.synchronize()
    for name, g, ref in (("GU", gGU, GU), ("Y", gY, Y), ("Z", gZ, Z), ("dX", gdX, dX), ("dWgu", gdW, dW),
                         ("dWd", gdD, dD)):
        g.check(name)
        same(name, g.t, ref)
    ws.check("SwiGLU backward workspace")


@pytest.mark.parametrize("M", [300, 2072])
def test_guard_attention_projections(M):
    b, s, h, n_q, n_kv, dh, t, r = 1, M, 1032, 8, 2, 72, 2, 1
    q, kv = n_q // t * dh, n_kv // t * dh
    d = dev()
    X, W, Wo, A, dZ, dQ = synth.small(5 + M, (M, h), (h, q + 2 * kv), (q, h), (M, q), (M, h), (M, q + 2 * kv),
                                      dtype="bf16")
    W, Wo = (W.float() * 0.05).to(BF16).to(d), (Wo.float() * 0.05).to(BF16).to(d)
    X, A, dZ, dQ = X.to(d), A.to(d), dZ.to(d), dQ.to(d)
    a = (b, s, h)
    step(f"guard bands: attention projections M={M}")
    outs = {}
    for guarded in (False, True):
        mk = (lambda shp: Guarded(shp, BF16)) if guarded else (lambda shp: torch.empty(*shp, dtype=BF16, device=d))
        o = {"QKV": mk((M, q + 2 * kv)), "QKVu": mk((M, q + 2 * kv)), "Z": mk((M, h)), "dX": mk((M, h)),
             "dW": mk((h, q + 2 * kv)), "dA": mk((M, q)), "dWo": mk((q, h))}
        v = {k: (x.t if guarded else x) for k, x in o.items()}
        wq = workspace(max(1, lgs.attn_qkv_fwd_workspace_bytes(*a, n_q, n_kv, dh, t)))
        wo = workspace(max(1, lgs.attn_out_bwd_workspace_bytes(*a, n_q, dh, t)))
        lgs.tp_attn_qkv_fwd(*a, n_q, n_kv, dh, t, r, X, W, v["QKV"], workspace=wq.t)
        lgs.tp_attn_qkv_fwd(*a, n_q, n_kv, dh, t, r, X, W, v["QKVu"], split=False)
        lgs.tp_attn_out_fwd(*a, n_q, dh, t, r, A, Wo, v["Z"])
        lgs.tp_attn_qkv_bwd(*a, n_q, n_kv, dh, t, r, X, W, dQ, v["dX"], v["dW"])
        lgs.tp_attn_out_bwd(*a, n_q, dh, t, r, A, Wo, dZ, v["dA"], v["dWo"], workspace=wo.t)
        torch.cuda.synchronize()
        wq.check("QKV workspace")
        wo.check("output projection workspace")
        outs[guarded] = o
    for k, g in outs[True].items():
        g.check(k)
        same(k, g.t, outs[False][k])

"""The entry points under HIP graph capture: one rank's MLP forward, the sum
of the t partials, the MLP backward, the fused CE forward and the CE combine
are captured once (caller-supplied workspaces, so nothing allocates inside
the capture) and replayed several times, with eager runs of the same calls
and synchronisations between replays.  Every replay must reproduce the eager
outputs bit for bit: the kernels are deterministic (fixed tile order, fixed
summation order) and the library issues no memset, allocation or
synchronisation of its own.
"""

import pytest
import torch

from gpu_util import dev, step
from logit_gemm_shard_amd import binding as lgs
from logit_gemm_shard_amd import synth

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _inputs(d):
    b, s, h, ffn, t, rank, V = 1, 320, 256, 1024, 4, 1, 4 * 384
    M, f, Vr = b * s, ffn // t, V // t
    X, A, B, dZ, H, E = synth.small(71, (M, h), (h, ffn), (ffn, h), (M, h), (M, h), (V, h), dtype="bf16")
    A = (A.float() * 0.05).to(BF16)
    B = (B.float() * 0.05).to(BF16)
    E = (E.float() * 0.05).to(BF16)
    y = (torch.arange(M, dtype=torch.int32) * 131) % V
    others = synth.small(72, (t, M, h), dtype="bf16")[0]
    dxo = synth.small(73, (t, M, h), dtype="bf16")[0]
    st = synth.small(74, (t, 3, M))[0]
    st[:, 1] = st[:, 1].abs() + 1.0
    st[:, 2] = 0.0
    cfg = dict(b=b, s=s, h=h, ffn=ffn, t=t, rank=rank, V=V, M=M, f=f, Vr=Vr)
    ins = dict(X=X, A=A[:, rank * f:(rank + 1) * f].contiguous(), B=B[rank * f:(rank + 1) * f].contiguous(),
               dZ=dZ, H=H, E=E[rank * Vr:(rank + 1) * Vr].contiguous(), y=y, others=others, dxo=dxo, st=st)
    return cfg, {k: v.to(d) for k, v in ins.items()}


def _outputs(cfg, d):
    M, h, f, t = cfg["M"], cfg["h"], cfg["f"], cfg["t"]
    return dict(zparts=torch.empty(t, M, h, dtype=BF16, device=d), U=torch.empty(M, f, dtype=BF16, device=d),
                Y=torch.empty(M, f, dtype=BF16, device=d), Z=torch.empty(M, h, dtype=BF16, device=d),
                dxparts=torch.empty(t, M, h, dtype=BF16, device=d), dA=torch.empty(h, f, dtype=BF16, device=d),
                dB=torch.empty(f, h, dtype=BF16, device=d), dX=torch.empty(M, h, dtype=BF16, device=d),
                stats=torch.empty(t, 3, M, dtype=F32, device=d), loss=torch.empty(M, dtype=F32, device=d))


def _other_ranks(x, o):
    """The other ranks' partials (inputs of the sums), copied eagerly outside any capture."""
    o["zparts"].copy_(x["others"])
    o["dxparts"].copy_(x["dxo"])
    o["stats"].copy_(x["st"])


def _clear(cfg, o):
    """NaN into everything the captured calls write (this rank's parts and the results)."""
    r = cfg["rank"]
    for k in ("U", "Y", "Z", "dA", "dB", "dX", "loss"):
        o[k].fill_(float("nan"))
    o["zparts"][r].fill_(float("nan"))
    o["dxparts"][r].fill_(float("nan"))
    o["stats"][r].fill_(float("nan"))


def _run(cfg, x, o, ws, stream):
    """Library calls only (no torch work), on `stream`."""
    b, s, h, ffn, t, r, V, M = (cfg[k] for k in ("b", "s", "h", "ffn", "t", "rank", "V", "M"))
    lgs.tp_mlp_fwd(b, s, h, ffn, t, r, x["X"], x["A"], x["B"], o["zparts"][r], U_i=o["U"], Y_i=o["Y"],
                   workspace=ws["fwd"], stream=stream)
    lgs.shard_partial_sum("sum", t, M * h, o["zparts"], M * h, o["Z"], stream=stream)
    lgs.tp_mlp_bwd(b, s, h, ffn, t, r, x["X"], x["A"], x["B"], o["U"], x["dZ"], o["dxparts"][r], o["dA"],
                   o["dB"], workspace=ws["bwd"], stream=stream)
    lgs.shard_partial_sum("sum", t, M * h, o["dxparts"], M * h, o["dX"], stream=stream)
    lgs.vocab_parallel_xent_fwd(b, s, h, V, t, r, x["H"], x["E"], x["y"], o["stats"][r, 0], o["stats"][r, 1],
                                o["stats"][r, 2], workspace=ws["xent"], stream=stream)
    lgs.shard_partial_sum("xent", t, M, o["stats"], 3 * M, o["loss"], stream=stream)


def test_entry_points_replay_under_graph_capture():
    d = dev()
    cfg, x = _inputs(d)
    b, s, h, ffn, t, V = (cfg[k] for k in ("b", "s", "h", "ffn", "t", "V"))
    nfwd = lgs.lib().lgs_mlp_fwd_workspace_bytes(b, s, h, ffn, t, 1, 1)
    ws = {"fwd": torch.empty(max(nfwd, 1), dtype=torch.uint8, device=d) if nfwd else None,
          "bwd": torch.empty(lgs.mlp_bwd_workspace_bytes(b, s, h, ffn, t, BF16), dtype=torch.uint8, device=d),
          "xent": torch.empty(lgs.xent_workspace_bytes(b, s, h, V, t), dtype=torch.uint8, device=d)}
    step("graph capture: eager reference")
    ref = _outputs(cfg, d)
    _other_ranks(x, ref)
    _run(cfg, x, ref, ws, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for k, v in ref.items():
        assert torch.isfinite(v.float()).all(), k

    cap = _outputs(cfg, d)
    _other_ranks(x, cap)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        _run(cfg, x, cap, ws, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    step("graph capture: capturing")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(cfg, x, cap, ws, torch.cuda.current_stream())
    torch.cuda.synchronize()
    scratch = _outputs(cfg, d)
    _other_ranks(x, scratch)
    for rep in range(3):
        step(f"graph capture: replay {rep}")
        _clear(cfg, cap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(cap[k], ref[k]), f"replay {rep}: {k} differs from the eager result"
        _clear(cfg, scratch)  # eager work between replays
        _run(cfg, x, scratch, ws, torch.cuda.current_stream())
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(scratch[k], ref[k]), f"eager run after replay {rep}: {k}"


def test_k_split_backward_replays_under_graph_capture():
    """The backward at a shape whose weight gradients are split over the
    tokens inside the grouped launch (M = 2200, h = 1064, f = 1048: 2 parts)
    launches a counter-clearing kernel and the grouped GEMM; captured once
    and replayed, every replay equals the eager result bit for bit."""
    d = dev()
    b, s, h, ffn, t, r = 2, 1100, 1064, 2 * 1048, 2, 1
    M, f = b * s, ffn // t
    X, A, B, dZ, U = synth.small(81, (M, h), (h, f), (f, h), (M, h), (M, f), dtype="bf16")
    A = (A.float() * 0.05).to(BF16).to(d)
    B = (B.float() * 0.05).to(BF16).to(d)
    X, dZ, U = X.to(d), dZ.to(d), U.to(d)
    plain = 2 * ((M * f * 2 + 255) // 256 * 256)
    nws = lgs.mlp_bwd_workspace_bytes(b, s, h, ffn, t, BF16)
    assert nws > plain, "expected the K-split plan"
    ws = torch.empty(nws, dtype=torch.uint8, device=d)

    def outs():
        return (torch.empty(M, h, dtype=BF16, device=d), torch.empty(h, f, dtype=BF16, device=d),
                torch.empty(f, h, dtype=BF16, device=d))

    def run(o, stream):
        lgs.tp_mlp_bwd(b, s, h, ffn, t, r, X, A, B, U, dZ, *o, workspace=ws, stream=stream)

    step("K-split backward under graph capture: eager reference")
    ref = outs()
    run(ref, torch.cuda.current_stream())
    torch.cuda.synchronize()
    cap = outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(cap, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(cap, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        step(f"K-split backward under graph capture: replay {rep}")
        for x in cap:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("dX", "dA", "dB"), cap, ref):
            assert torch.equal(x, y), f"replay {rep}: {name} differs from the eager result"
        eager = outs()  # eager work between replays, on the same workspace
        run(eager, torch.cuda.current_stream())
        torch.cuda.synchronize()
        for name, x, y in zip(("dX", "dA", "dB"), eager, ref):
            assert torch.equal(x, y), f"eager run after replay {rep}: {name}"

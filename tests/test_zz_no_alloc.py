"""The allocation-free fused CE forward (vocab_parallel_xent_fwd_noalloc,
through the C ABI) against vocab_parallel_xent_fwd with a caller workspace.

Both run the same kernels, so every output must be the same bits.  Two calls
in a row, the second on a smaller input, so that the second starts with the
first call's slab partials still in the static scratch (nothing may leak from
one call into the next).  The first call is the 8.3B-shape slice at full size
(8192 tokens, 6400 columns, h = 3072: the largest the benchmark runs); the
second a ragged t = 1 case with the loss output, also checked against the
fp64 oracle.
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


def _both(b, s, h, V, t, r, H, E_r, y, with_loss):
    d = H.device
    M = b * s
    outs = []
    for noalloc in (False, True):
        m, l, T = (torch.full((M,), float("nan"), dtype=F32, device=d) for _ in range(3))
        am = torch.full((M,), -7, dtype=torch.int32, device=d)
        loss = torch.full((M,), float("nan"), dtype=F32, device=d) if with_loss else None
        fn = lgs.vocab_parallel_xent_fwd_noalloc if noalloc else lgs.vocab_parallel_xent_fwd
        fn(b, s, h, V, t, r, H, E_r, y, m, l, T, argmax_r=am, loss=loss)
        outs.append((m, l, T, am, loss))
    torch.cuda.synchronize()
    return outs


def test_noalloc_equals_workspace_call_two_calls():
    d = dev()
    w = WORKLOADS["xent_8p3b"]
    H, E, y = synth.xent_inputs(w)
    Vr, r = w.v_r, 5
    need = lgs.xent_workspace_bytes(w.b, w.s, w.h, w.vocab, w.t)
    assert need <= lgs.XENT_NOALLOC_SCRATCH_BYTES
    step(f"noalloc CE call 1: 8.3B slice at full size, rank {r} (slab partials {need} bytes)")
    ref, got = _both(w.b, w.s, w.h, w.vocab, w.t, r, H.to(d), E[r * Vr:(r + 1) * Vr].to(d), y.to(d), False)
    for name, a, b in zip(("m", "l", "T", "argmax"), ref[:4], got[:4]):
        assert torch.equal(a, b), f"{name}: noalloc differs from the workspace call"
    assert torch.isfinite(got[0]).all() and (got[1] >= 1).all()

    # the second call is smaller: 300 tokens, a K tail (h = 136), t = 1 with the loss
    b, s, h, V = 1, 300, 136, 1000
    H2, E2 = synth.small(21, (b * s, h), (V, h), dtype="bf16")
    E2 = (E2.float() * 0.3).to(BF16)
    y2 = torch.randint(0, V, (b * s,), generator=torch.Generator().manual_seed(4)).to(torch.int32)
    step("noalloc CE call 2: 300 tokens, h = 136, t = 1, loss written")
    ref, got = _both(b, s, h, V, 1, 0, H2.to(d), E2.to(d), y2.to(d), True)
    for name, a, bb in zip(("m", "l", "T", "argmax", "loss"), ref, got):
        assert torch.equal(a, bb), f"{name}: noalloc differs from the workspace call"
    yn = y2.numpy().astype(np.int64)
    rm, rl, rT, _ = oracle.xent.shard_partials(f64(H2), f64(E2), yn, 0)
    assert_close("m (noalloc)", got[0], rm, BF16)
    assert_close("l (noalloc)", got[1], rl, BF16)
    assert_close("T (noalloc)", got[2], rT, BF16)
    assert_close("loss (noalloc)", got[4], oracle.xent.naive_loss(f64(H2), f64(E2), yn), BF16)


def test_noalloc_rejects_oversize_before_launch():
    """32768 tokens at the 8.3B slice need 20 MiB of slab partials: rejected
    with LGS_ERR_UNSUPPORTED, outputs untouched."""
    d = dev()
    b, s, h, V, t = 32, 1024, 64, 51200, 8
    M, Vr = b * s, V // t
    H = torch.zeros(M, h, dtype=BF16, device=d)
    E = torch.zeros(Vr, h, dtype=BF16, device=d)
    y = torch.zeros(M, dtype=torch.int32, device=d)
    m = torch.full((M,), 3.0, dtype=F32, device=d)
    l, T = m.clone(), m.clone()
    step("noalloc CE: oversize call rejected")
    with pytest.raises(lgs.LgsError) as ei:
        lgs.vocab_parallel_xent_fwd_noalloc(b, s, h, V, t, 0, H, E, y, m, l, T)
    assert ei.value.status == lgs.LGS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (m == 3.0).all() and (l == 3.0).all() and (T == 3.0).all()

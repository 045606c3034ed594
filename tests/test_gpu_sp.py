"""Parity of the sequence-parallel stand-ins (shard_reduce_scatter,
shard_all_gather, through the C ABI) with the fp64 oracle ``oracle.sp``.

Both are exact operations here: the reduce-scatter accumulates in fp32 in
ascending rank order exactly as shard_partial_sum does, so on small-integer
data both are exact, and on any data the chunk equals the matching rows of
the all-reduce bit for bit; the all-gather is a copy.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, f64, step
from logit_gemm_shard_amd import binding as lgs

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _ints(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-16, 17, shape, generator=g).to(dtype)


@pytest.mark.parametrize("din,dout", [(BF16, BF16), (BF16, F32), (F32, F32), (F32, BF16)])
@pytest.mark.parametrize("shape", [(8, 1024, 8, 3072), (4, 96, 3, 7), (2, 2, 1, 5), (1, 16, 2, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_reduce_scatter_then_all_gather_exact(shape, din, dout):
    t, s, b, h = shape
    d = dev()
    n, c = s * b * h, (s // t) * b * h
    step(f"sp t={t} s={s} b={b} h={h} {din}->{dout}")
    parts = _ints((t, s * b, h), t * 31 + h, din)
    pd = parts.to(d)
    chunks = torch.empty(t, (s // t) * b, h, dtype=dout, device=d)
    for r in range(t):
        lgs.shard_reduce_scatter(t, r, s, b, h, pd, n, chunks[r])
    full = torch.empty(s * b, h, dtype=dout, device=d)
    lgs.shard_all_gather(t, s, b, h, chunks, c, full)
    ar = torch.empty(s * b, h, dtype=dout, device=d)
    lgs.shard_partial_sum("sum", t, n, pd, n, ar)
    torch.cuda.synchronize()
    p64 = [f64(p) for p in parts]
    for r in range(t):
        assert np.array_equal(f64(chunks[r]), oracle.sp.reduce_scatter(p64, s, b, t, r)), r
    assert np.array_equal(f64(full), oracle.sp.all_gather([f64(x) for x in chunks], s, b, t))
    assert torch.equal(full, ar)


def test_reduce_scatter_matches_all_reduce_bits_on_real_data():
    """Non-integer partials (a row-parallel exit's Z_i): every rank's chunk is
    bit-identical to its rows of the all-reduce, and the all-gather of the
    chunks to the whole all-reduce."""
    t, s, b, h = 8, 512, 2, 1024
    d = dev()
    n, c = s * b * h, (s // t) * b * h
    step("sp reduce-scatter vs all-reduce bits (bf16 partials)")
    g = torch.Generator().manual_seed(9)
    stride = n + 64  # padded rank blocks
    buf = (torch.randn(t, stride, generator=g) * 0.05).to(BF16).to(d)
    ar = torch.empty(n, dtype=BF16, device=d)
    lgs.shard_partial_sum("sum", t, n, buf, stride, ar)
    chunks = torch.empty(t, c, dtype=BF16, device=d)
    for r in range(t):
        lgs.shard_reduce_scatter(t, r, s, b, h, buf, stride, chunks[r])
    full = torch.empty(n, dtype=BF16, device=d)
    lgs.shard_all_gather(t, s, b, h, chunks, c, full)
    torch.cuda.synchronize()
    for r in range(t):
        assert torch.equal(chunks[r], ar[r * c:(r + 1) * c]), r
    assert torch.equal(full, ar)


def test_all_gather_strided_shards():
    """Shards with a padded stride (and fp32 with a chunk that is not a
    multiple of 16 bytes) land in rank order."""
    d = dev()
    for t, s, b, h, dt in ((4, 8, 3, 5, F32), (3, 6, 1, 8, BF16), (8, 64, 2, 96, BF16)):
        step(f"all-gather t={t} s={s} b={b} h={h} {dt}")
        c = (s // t) * b * h
        stride = c + 3
        shards = _ints((t, stride), 7 + h, dt).to(d)
        out = torch.empty(s * b * h, dtype=dt, device=d)
        lgs.shard_all_gather(t, s, b, h, shards, stride, out)
        torch.cuda.synchronize()
        want = oracle.sp.all_gather([f64(shards[q, :c]).reshape((s // t) * b, h) for q in range(t)], s, b, t)
        assert np.array_equal(f64(out).reshape(s * b, h), want)


# ------------------------------------------- fused SP region (RS + LayerNorm)

def _region_inputs(t, s, b, h, seed, with_mask):
    g = torch.Generator().manual_seed(seed)
    n = (s // t) * b
    parts = torch.randn(t, s * b, h, generator=g).to(BF16)
    res = torch.randn(n, h, generator=g).to(BF16)
    gamma = (1 + 0.1 * torch.randn(h, generator=g)).to(BF16)
    beta = (0.1 * torch.randn(h, generator=g)).to(BF16)
    keep = (torch.rand(n, h, generator=g) > 0.1).to(torch.uint8) if with_mask else None
    return parts, res, gamma, beta, keep


@pytest.mark.parametrize("with_mask", [False, True], ids=["nomask", "mask"])
@pytest.mark.parametrize("shape", [(8, 1024, 8, 3072), (3, 12, 3, 72), (2, 10, 5, 8), (4, 64, 2, 8192),
                                   (1, 5, 1, 16384), (2, 6, 1, 2056)], ids=lambda s: "x".join(map(str, s)))
def test_rs_layernorm_every_element(shape, with_mask):
    """Every rank's hs and y against the oracle's exit region (bf16
    tolerance); without a mask, hs bit for bit against the reduce-scatter's
    fp32 chunk plus the residual rounded once (the same fp32 sum in the same
    order)."""
    t, s, b, h = shape
    d = dev()
    n = (s // t) * b
    parts, res, gamma, beta, keep = _region_inputs(t, s, b, h, 7 * t + h, with_mask)
    scale = 1 / 0.9
    pd = parts.to(d)
    p64 = [f64(p) for p in parts]
    for r in sorted({0, t - 1}):
        step(f"rs+layernorm {shape} mask={with_mask} rank={r}")
        rd = res.to(d)
        kd = None if keep is None else keep.to(d)
        hs = torch.empty(n, h, dtype=BF16, device=d)
        y = torch.empty(n, h, dtype=BF16, device=d)
        lgs.shard_reduce_scatter_layernorm(t, r, s, b, h, pd, s * b * h, rd, gamma.to(d), beta.to(d), hs, y,
                                           keep=kd, keep_scale=scale, eps=1e-5)
        z = torch.empty(n, h, dtype=F32, device=d)
        lgs.shard_reduce_scatter(t, r, s, b, h, pd, s * b * h, z)
        torch.cuda.synchronize()
        rh, ry = oracle.sp.exit_region(p64, s, b, t, r, f64(res), f64(gamma), f64(beta), 1e-5,
                                       None if keep is None else keep.numpy(), scale)
        assert_close("hs", hs, rh, BF16)
        assert_close("y", y, ry, BF16)
        if keep is None:  # (with a mask the product and the add may contract into one fma)
            assert torch.equal(hs.cpu(), (z.cpu() + res.float()).to(BF16)), "hs: one rounding of the fp32 sum"


def test_rs_layernorm_unit_rows_and_guards():
    """With gamma = 1 and beta = 0 every output row has mean ~0 and variance
    ~1 (checked at the 8.3B chunk size on every row); outputs written into
    wider sentinel-filled buffers leave everything outside their rows alone."""
    t, s, b, h = 8, 1024, 8, 3072
    d = dev()
    n = (s // t) * b
    parts, res, _, _, _ = _region_inputs(t, s, b, h, 5, False)
    pad = 4096
    hs_buf = torch.full((n * h + 2 * pad,), float("nan"), dtype=BF16, device=d)
    y_buf = torch.full((n * h + 2 * pad,), float("nan"), dtype=BF16, device=d)
    hs, y = hs_buf[pad:pad + n * h].view(n, h), y_buf[pad:pad + n * h].view(n, h)
    step("rs+layernorm: unit rows and guard bands")
    lgs.shard_reduce_scatter_layernorm(t, 3, s, b, h, parts.to(d), s * b * h, res.to(d),
                                       torch.ones(h, dtype=BF16, device=d), torch.zeros(h, dtype=BF16, device=d),
                                       hs, y)
    torch.cuda.synchronize()
    yf = f64(y)
    assert np.abs(yf.mean(axis=1)).max() < 2e-2 and np.abs(yf.var(axis=1) - 1).max() < 2e-2
    for buf in (hs_buf, y_buf):
        assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[pad + n * h:].float()).all()
        assert torch.isfinite(buf[pad:pad + n * h].float()).all()


@pytest.mark.parametrize("with_mask,with_dhs", [(False, False), (True, True)], ids=["plain", "mask+dhs"])
@pytest.mark.parametrize("shape", [(8, 1024, 8, 3072), (3, 12, 3, 72), (2, 10, 5, 8), (4, 64, 2, 8192),
                                   (1, 5, 1, 16384), (2, 700, 1, 2056)], ids=lambda s: "x".join(map(str, s)))
def test_layernorm_bwd_every_element(shape, with_mask, with_dhs):
    """The region's backward on a rank's rows against the oracle: g and dz on
    every element (bf16 tolerance), dgamma and dbeta (fp32 tolerance); a
    second call repeats every bit (the column sums go in a fixed order)."""
    t, s, b, h = shape
    d = dev()
    n = (s // t) * b
    g_ = torch.Generator().manual_seed(9 * t + h)
    hs = torch.randn(n, h, generator=g_).to(BF16)
    dy = torch.randn(n, h, generator=g_).to(BF16)
    dhs = torch.randn(n, h, generator=g_).to(BF16) if with_dhs else None
    gamma = (1 + 0.1 * torch.randn(h, generator=g_)).to(BF16)
    keep = (torch.rand(n, h, generator=g_) > 0.1).to(torch.uint8) if with_mask else None
    step(f"layernorm bwd {shape} mask={with_mask} dhs={with_dhs}")
    outs = []
    for _ in range(2):
        G = torch.empty(n, h, dtype=BF16, device=d)
        dz = torch.empty(n, h, dtype=BF16, device=d)
        dg, db = torch.empty(h, dtype=F32, device=d), torch.empty(h, dtype=F32, device=d)
        lgs.shard_layernorm_bwd(t, t - 1, s, b, h, hs.to(d), dy.to(d), gamma.to(d), G, dz, dg, db,
                                dhs=None if dhs is None else dhs.to(d), keep=None if keep is None else keep.to(d),
                                keep_scale=1 / 0.9)
        outs.append((G, dz, dg, db))
    torch.cuda.synchronize()
    ref = oracle.sp.exit_region_backward(f64(hs), f64(gamma), f64(dy), None if dhs is None else f64(dhs), 1e-5,
                                         None if keep is None else keep.numpy(), 1 / 0.9)
    G, dz, dg, db = outs[0]
    assert_close("g", G, ref["g"], BF16)
    assert_close("dz", dz, ref["dz"], BF16)
    assert_close("dgamma", dg, ref["dgamma"], F32)
    assert_close("dbeta", db, ref["dbeta"], F32)
    for a, c in zip(outs[0], outs[1]):
        assert torch.equal(a, c)

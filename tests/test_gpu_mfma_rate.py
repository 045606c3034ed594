"""The matrix-core rate probe (lgs_test_mfma_rate), which measures the ceiling
the GEMM kernels' fractions of the bf16 peak are read against.  With
small-integer operands every accumulator is exact in fp32, so the probe's
arithmetic and the register layout of v_mfma_f32_32x32x16_bf16 it relies on
are checked bit for bit:
  A (32 x 16): lane l holds A[l % 32][8 (l // 32) + e], e = 0..7;
  B (16 x 32): lane l holds B[8 (l // 32) + e][l % 32];
  D (32 x 32): element r of lane l is D[8 (r // 4) + 4 (l // 32) + r % 4][l % 32].
Chain c ends holding iters8 * (sum_k A_k) B_c.
"""

import numpy as np
import pytest
import torch

from gpu_util import dev, step
from logit_gemm_shard_amd import binding as lgs

pytestmark = pytest.mark.gpu

LANES = np.arange(64)


def _a(frag):
    """[64, 8] lane values -> the 32 x 16 A operand."""
    A = np.zeros((32, 16))
    for l in LANES:
        A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = frag[l]
    return A


def _b(frag):
    """[64, 8] lane values -> the 16 x 32 B operand."""
    B = np.zeros((16, 32))
    for l in LANES:
        B[8 * (l // 32):8 * (l // 32) + 8, l % 32] = frag[l]
    return B


def _expected(ops, iters8):
    """[8 chains, 16 elements, 64 lanes] of one wave's accumulators."""
    S = sum(_a(ops[2 * k]) for k in range(8))
    out = np.zeros((8, 16, 64))
    for c in range(8):
        D = iters8 * (S @ _b(ops[2 * c + 1]))
        for l in LANES:
            for r in range(16):
                out[c, r, l] = D[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32]
    return out


@pytest.mark.parametrize("blocks,waves,iters8", [(3, 4, 5), (2, 8, 1), (1, 1, 0)])
def test_mfma_rate_probe_is_exact(blocks, waves, iters8):
    d = dev()
    rng = np.random.default_rng(blocks * 100 + waves)
    ops = rng.integers(-2, 3, size=(16, 64, 8)).astype(np.float32)
    out = torch.full((blocks * waves * 8192,), float("nan"), device=d)
    clocks = torch.zeros(2 * blocks * waves, dtype=torch.int64, device=d)
    step(f"mfma_rate: {blocks} block(s) x {waves} wave(s), iters8 = {iters8}")
    lgs.mfma_rate(blocks, waves, iters8, torch.tensor(ops, dtype=torch.bfloat16, device=d), out, clocks)
    torch.cuda.synchronize()
    want = _expected(ops, iters8)
    got = out.cpu().numpy().reshape(blocks * waves, 8, 16, 64)
    for w in range(blocks * waves):
        assert np.array_equal(got[w], want), w
    ck = clocks.cpu().numpy().reshape(-1, 2)
    assert np.all(ck >= 0)
    if iters8 > 0:
        assert np.all(ck[:, 0] > 0)


def test_mfma_rate_probe_rejects_bad_arguments():
    d = dev()
    ops = torch.zeros(16, 64, 8, dtype=torch.bfloat16, device=d)
    out = torch.empty(8192, device=d)
    clocks = torch.empty(2, dtype=torch.int64, device=d)
    with pytest.raises(ValueError):
        lgs.mfma_rate(1, 2, 1, ops, out, clocks)  # out too small for two waves
    with pytest.raises(lgs.LgsError):
        lgs.mfma_rate(1, 9, 1, ops, torch.empty(9 * 8192, device=d), torch.empty(18, dtype=torch.int64, device=d))

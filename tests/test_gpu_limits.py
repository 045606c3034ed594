"""The largest operands the library takes: an operand's byte span just under
2 GiB (the bound the ABI enforces, because the kernels address operands
through 32-bit buffer offsets).  The rows checked against the oracle include
the last ones, whose offsets are within 128 KiB of the bound, in both operand
orientations of the GEMM core and through the fused CE.  Inputs are drawn on
the device by torch's generator (seeded); the oracle reads the same values.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, dev, f64, step
from logit_gemm_shard_amd import binding as lgs

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
M_BIG, K_BIG = 131064, 8192  # 131064 * 8192 * 2 B = 2^31 - 128 KiB (M a multiple of 8 for M-major A)


def _draw(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(*shape, generator=g, device="cuda", dtype=F32) * scale).to(BF16)


def _rows(M):
    return np.array([0, 1, M // 2, M - 129, M - 2, M - 1])


def test_gemm_operand_at_the_2gib_bound():
    d = dev()
    assert M_BIG * K_BIG * 2 < 2 ** 31 <= M_BIG * K_BIG * 2 + 131072
    N = 64
    B = _draw((K_BIG, N), 2, 0.02)
    B64 = f64(B)
    rows = _rows(M_BIG)
    for a_kmajor in (True, False):
        step(f"GEMM with a 2 GiB - 128 KiB A operand, a_kmajor={a_kmajor}")
        A = _draw((M_BIG, K_BIG) if a_kmajor else (K_BIG, M_BIG), 1)
        C = torch.empty(M_BIG, N, dtype=BF16, device=d)
        lgs.gemm_bf16(A, B, C, a_kmajor=a_kmajor, b_kmajor=False)
        torch.cuda.synchronize()
        Arows = A[rows] if a_kmajor else A[:, rows].t()
        assert_close(f"C rows {rows.tolist()}", C[rows], f64(Arows) @ B64, BF16)
        del A, C
        torch.cuda.empty_cache()


def test_fused_xent_hidden_rows_at_the_2gib_bound():
    d = dev()
    b, s, h, V, t = 4, M_BIG // 4, K_BIG, 8 * 128, 8
    M, Vr = b * s, V // t
    step(f"fused CE with H of {M} x {h} bf16 (2 GiB - 128 KiB)")
    H = _draw((M, h), 3)
    E = _draw((V, h), 4, 0.02)
    g = torch.Generator().manual_seed(5)
    y = torch.randint(0, V, (M,), generator=g, dtype=torch.int64).to(torch.int32)
    yd = y.to(d)
    stats = torch.empty(t, 3, M, dtype=F32, device=d)
    for r in (0, t - 1):
        lgs.vocab_parallel_xent_fwd(b, s, h, V, t, r, H, E[r * Vr:(r + 1) * Vr], yd, stats[r, 0], stats[r, 1],
                                    stats[r, 2])
    torch.cuda.synchronize()
    rows = _rows(M)
    H64, E64, yn = f64(H[rows]), f64(E), y.numpy().astype(np.int64)[rows]
    st = stats.cpu()
    for r in (0, t - 1):
        m, l, T, _ = oracle.xent.shard_partials(H64, E64[r * Vr:(r + 1) * Vr], yn, r * Vr)
        assert_close(f"m_{r} rows", st[r, 0][rows], m, BF16)
        assert_close(f"l_{r} rows", st[r, 1][rows], l, BF16)
        own = (yn // Vr) == r
        if own.any():
            assert_close(f"T_{r} rows (owned)", st[r, 2][rows][own], T[own], BF16)

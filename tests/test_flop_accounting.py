"""The benchmark's FLOP convention against the worked figure a page prints.

"Megatron-LM, in depth" (aicassindra), "Overlap and memory settings": a step
of a 70B dense model over about 4.2M tokens costs about 6 x params x tokens
FLOPs (forward 2PT, backward 4PT), about 8.6 s on 512 GPUs at 400 TFLOP/s
each.  bench.py counts 2*M*N*K per GEMM: two GEMMs forward and four backward
per MLP shard, whose parameters are A_i [h, f_i] and B_i [f_i, h].
"""
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "flop_accounting.txt")


def _golden():
    for line in open(GOLDEN):
        if line.strip() and not line.lstrip().startswith("#"):
            return [float(x) for x in line.split()]
    raise AssertionError("no data line")


def test_page_figure_is_the_six_p_t_rule():
    P, T, gpus, tflops, step_flops, step_s = _golden()
    assert 6 * P * T == pytest.approx(step_flops, rel=0.01)           # printed rounded to 3 digits
    assert 6 * P * T / (gpus * tflops * 1e12) == pytest.approx(step_s, rel=0.01)


@pytest.mark.parametrize("M,h,f", [(8192, 3072, 1536), (4096, 8192, 3584), (7, 40, 24)])
def test_bench_counts_forward_2pt_and_backward_4pt(M, h, f):
    fl = bench.mlp_flops(M, h, f)
    P = 2 * h * f  # the shard's parameters
    assert fl["fwd"] == 2 * P * M
    assert fl["bwd"] == 4 * P * M
    assert fl["fwd"] + fl["bwd"] == 6 * P * M


def test_bench_logit_gemm_is_one_gemm():
    M, h, Vr = 8192, 3072, 6400
    assert bench.xent_flops(M, h, Vr) == 2 * M * h * Vr  # 322.1 GFLOP per launch
    assert bench.xent_flops(M, h, Vr) == pytest.approx(322.1e9, rel=1e-3)


def test_bench_backward_algorithmic_bytes():
    """tp_mlp_bwd at the 70B shape: X, U, dZ, dX (3 x [M, h] + [M, f]), A_i,
    B_i, dA_i, dB_i (4 x h f), and Y_i, dU_i written once and read once
    (4 x [M, f]), in bf16."""
    M, h, f = 4096, 8192, 3584
    assert bench.mlp_bwd_bytes(M, h, f) == 2 * (3 * M * h + M * f + 4 * h * f + 4 * M * f)

"""Host-side logic of bench.py (no GPU): the block-to-tile map its traffic
model uses, the model's bounds, the one-GPU guard and the kernel-time table."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("tm,tn", [(16, 14), (32, 25), (32, 20), (7, 5), (1, 1), (3, 8)])
def test_block_tile_is_a_bijection_onto_the_grid(tm, tn):
    n = tm * tn
    tiles = [bench.block_tile(p, n, tm, tn) for p in range(n)]
    assert sorted(tiles) == [(i, j) for i in range(tm) for j in range(tn)]


def test_block_tile_gives_each_xcd_a_contiguous_grouped_run():
    # 16 x 14 tiles (the 70B column-parallel GEMM on 256x256): the blocks an
    # XCD receives (ids x, x + 8, ...) walk 28 consecutive tiles of the
    # grouped order, i.e. 4 tile rows by 7 columns
    tm, tn = 16, 14
    n = tm * tn
    for x in range(8):
        ts = [bench.block_tile(p, n, tm, tn) for p in range(x, n, 8)]
        rows, cols = {t[0] for t in ts}, {t[1] for t in ts}
        assert len(ts) == 28 and len(rows) == 4 and len(cols) == 7


def test_panel_model_bounds():
    k = 6144
    # one XCD, one round holding every tile: each panel fetched exactly once
    assert bench.panel_fill_model(6, 5, 256, 320, k, xcds=1, group_m=8, cus=64) == (6 * 256 + 5 * 320) * k
    # never below one fetch of every panel, never above two panels per tile
    for tm, tn, bm, bn in ((32, 10, 256, 320), (32, 15, 256, 256), (16, 14, 256, 256)):
        got = bench.panel_fill_model(tm, tn, bm, bn, k)
        assert (tm * bm + tn * bn) * k <= got <= tm * tn * (bm + bn) * k


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_kernel_stats_table(tmp_path, capsys):
    src = tmp_path / "k.csv"
    src.write_text("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n"
                   "_ZN3lgs14gemm_pp_kernelINS_9PPProblemILi256ELi256ELb1ELb0ENS_8EpiStoreIDF16bEEEEEEvT_,"
                   "3,600000,200000,75.0,190000,210000,1\n"
                   "psum_vec_kernel,2,200000,100000,25.0,90000,110000,1\n")
    bench.kernel_stats_md(str(src), "title", "cmd")
    out = capsys.readouterr().out.splitlines()
    assert out[0] == "# title" and "cmd" in out
    rows = [l for l in out if l.startswith("| `")]
    assert rows[0] == "| `gemm_pp_kernel PPProblem 256 256 true false EpiStore bf16` | 3 | 200.0 | 190.0 | 210.0 | 75.00 |"
    assert rows[1].startswith("| `psum_vec_kernel` | 2 | 100.0 |")

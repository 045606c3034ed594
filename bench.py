"""Benchmark: one tensor-parallel rank's transformer-block shard on one MI355X.

A step is one pass of the whole path over one batch, for rank 0 of t = 8 at
the 8.3B-parameter model's shapes (b = 8, s = 1024, h = 3072, ffn = 12288,
padded vocabulary 51,200):

  1. tp_mlp_fwd               U_0 = X A_0, Y_0 = GeLU(U_0), Z_0 = Y_0 B_0
  2. shard_partial_sum(SUM)   Z = sum of the 8 ranks' partials (rank 0's just
                              written, the other 7 resident synthetic partials)
  3. tp_mlp_bwd               dY, dU = dY GeLU'(U_0), dB_0, dA_0, dX_0
  4. shard_partial_sum(SUM)   dX = sum of the 8 ranks' dX partials
  5. vocab_parallel_xent_fwd  fused logit GEMM + CE partials of slice 0
  6. shard_partial_sum(XENT)  per-token loss from the 8 ranks' partials

All inputs are resident in HBM before timing starts.  Order of work: W
warm-up steps; the per-configuration timings, the streaming CE measurement
and the clock sampling (so that the timed steps see the device settled);
then the timed region, K steps between two synchronizations, with HIP
events around the CE entry point only (its roofline is measured there);
then an untimed pass of K steps with events between every entry point for
the per-entry-point breakdown (those events cost the step about 2.5%).
Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-per-config] [--no-clock]
    python bench.py --copy-calibration   # plain copy for counter scaling
    python bench.py --blas-reference     # torch.matmul (hipBLASLt) at the same GEMM shapes
"""

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % bf16 MFMA peak for TP-shard MLP fwd+bwd; CE tokens/s"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, AMD's published figure
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
COUNTERS_FILE = os.path.join(ROOT, "profiles", "xent_8p3b_hbm_counters.txt")


def kernel_sources_digest():
    """sha256 over the HIP sources: counters are only valid for the code they were taken on."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "logit_gemm_shard_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()


def step_flops(M, h, f, Vr):
    """Algorithmic FLOPs (2*M*N*K per GEMM): forward 2 GEMMs, backward 4, plus the logit GEMM."""
    return {"mlp_fwd": 2 * 2 * M * h * f, "mlp_bwd": 4 * 2 * M * h * f, "xent": 2 * M * h * Vr}


def sample_gpu_clock(torch, run, seconds=3.0, n=4):
    """The graphics clock while `run` (one step) repeats for `seconds`: n
    readings of `amd-smi metric --clock --json` (a child process) spread over
    the run, each the mean of the XCDs' clocks; the median is reported with
    every reading.  None if the tool is missing or its output cannot be read."""
    import json
    import shutil
    import subprocess
    import threading
    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    readings = []

    def reader():
        for _ in range(n):
            delay = seconds / (n + 1)
            time.sleep(delay)
            try:
                r = subprocess.run([tool, "metric", "--clock", "--json"], capture_output=True, text=True,
                                   timeout=20)
                data = json.loads(r.stdout)
                gpus = data["gpu_data"] if isinstance(data, dict) else data
                clk = gpus[0]["clock"]
                vals = [v["clk"]["value"] for k, v in clk.items()
                        if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                if vals:
                    readings.append(sum(vals) / len(vals))
            except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.TimeoutExpired):
                pass

    th = threading.Thread(target=reader)
    t0 = time.perf_counter()
    th.start()
    k = 0
    while time.perf_counter() - t0 < seconds or th.is_alive():
        run()
        k += 1
        if k % 8 == 0:
            torch.cuda.synchronize()  # keep the queue short so the readings see steps running
        if time.perf_counter() - t0 > 4 * seconds + 30:
            break
    torch.cuda.synchronize()
    th.join()
    if not readings:
        return None
    med = sorted(readings)[len(readings) // 2]
    return {"sclk_mhz": round(med, 1), "readings_mhz": [round(x, 1) for x in readings],
            "spec_mhz": 2400, "source": "amd-smi metric --clock: median over readings taken while the "
                                        "step repeats, each the mean of the XCD graphics clocks"}


def read_counters():
    if not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256") != kernel_sources_digest():
        return None  # the kernels changed since the counters were taken
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of a known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 28  # 256 Mi floats = 1 GiB read + 1 GiB written per pass
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.neg(a, out=b)  # an elementwise kernel (a same-dtype copy_ may be a DMA, not a kernel)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "copies": 5,
                      "kernel": "torch.neg elementwise"}))


def cpu_baseline(w, xw, inputs, budget_s=10.0):
    """The fp64 oracle on the host, on a token sample of the same step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    X, A0, B0, dZ, H, E0, y = inputs
    f, h, Vr, t = w.f_i, w.h, xw.v_r, w.t
    rng = np.random.default_rng(0)

    def one_pass(m):
        Xs, dZs = X[:m].astype(np.float64), dZ[:m].astype(np.float64)
        Hs, ys = H[:m].astype(np.float64), y[:m]
        others = [rng.normal(size=(m, h)) for _ in range(t - 1)]
        stats = [(rng.normal(size=m), rng.uniform(1, 10, m), np.zeros(m)) for _ in range(t - 1)]
        t0 = time.perf_counter()
        U, Y, Z = oracle.mlp.shard_forward(Xs, A0, B0)
        oracle.mlp.partial_sum([Z] + others)
        g = oracle.mlp.shard_backward(Xs, A0, B0, U, dZs)
        oracle.mlp.partial_sum([g["dX"]] + others)
        mr, lr, Tr, _ = oracle.xent.shard_partials(Hs, E0, ys, 0)
        oracle.xent.merge(np.stack([mr] + [s[0] for s in stats]), np.stack([lr] + [s[1] for s in stats]),
                          np.stack([Tr] + [s[2] for s in stats]))
        return time.perf_counter() - t0

    # grow the token sample until one pass takes the budget, or the whole
    # step is covered; then repeat whole passes until the budget is spent
    for m in (256, 512, 1024, 2048, 4096, 8192):
        m = min(m, w.M)
        total, passes = one_pass(m), 1
        if total >= budget_s or m == w.M:
            break
    while total < budget_s:
        total += one_pass(m)
        passes += 1
    fl = sum(step_flops(m, h, f, Vr).values()) * passes
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": fl / total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "os_cpu_count": os.cpu_count(),
            "sample": f"the same step (MLP fwd+bwd, both sums, slice-0 CE, merge) on the first {m} "
                      f"of {w.M} tokens in fp64 numpy, {passes} passes: {fl / 1e9:.1f} GFLOP in {total:.2f} s"}


# The library's GEMM shapes (M, N, K) with the per-configuration entry they
# belong to, for the vendor-library reference below.
BLAS_SHAPES = [
    (4096, 8192, 3584, "70B GeLU / SwiGLU down GEMM (row-parallel)"),
    (4096, 3584, 8192, "70B GeLU column-parallel GEMM / dY"),
    (8192, 1536, 3072, "8.3B column-parallel GEMM / dY"),
    (8192, 3072, 1536, "8.3B row-parallel GEMM"),
    (8192, 6400, 3072, "8.3B CE logits (slice of t=8)"),
]


def blas_reference(reps=20):
    """torch.matmul in bf16 (hipBLASLt on ROCm) at the library's GEMM shapes:
    a vendor-library reference point for the same products (plain C = A B,
    no epilogue), timed with HIP events, next to this library's GEMM core on
    the same inputs with a plain store epilogue (the testing entry point;
    A K-contiguous, B N-contiguous, as torch.matmul of two row-major
    matrices).  The two alternate three times; the best of each is kept."""
    import torch
    from logit_gemm_shard_amd import binding as lgs
    dev = torch.device("cuda", 0)
    out = []
    for M, N, K, what in BLAS_SHAPES:
        a = torch.randn(M, K, device=dev).to(torch.bfloat16)
        b = torch.randn(K, N, device=dev).to(torch.bfloat16)
        c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        theirs, ours = [], []
        for _ in range(3):
            theirs.append(time_calls(torch, lambda: torch.matmul(a, b), reps, warmup=5))
            ours.append(time_calls(torch, lambda: lgs.gemm_bf16(a, b, c, True, False, -1), reps, warmup=5))
        t_ms, o_ms = min(theirs), min(ours)
        out.append({"M": M, "N": N, "K": K, "what": what, "us": round(t_ms * 1e3, 1),
                    "tflops": round(2 * M * N * K / t_ms / 1e9, 1), "library_us": round(o_ms * 1e3, 1),
                    "library_tflops": round(2 * M * N * K / o_ms / 1e9, 1),
                    "library_tile": "x".join(map(str, lgs.tile_shapes()[lgs.pick_tile(M, N)]))})
    print(json.dumps({"blas_reference": out, "library": "torch.matmul bf16 (hipBLASLt)"}), flush=True)


def time_calls(torch, fn, reps, warmup=3):
    """Average ms per call of fn() over reps calls, HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def per_config(torch, lgs, reps):
    """The configurations the library is specified on, each timed alone:
    the tiny fp32 block (both shards + sum), and the 70B-shape rank's forward
    and backward.  Inputs are device-side draws with the workloads'
    distributions (the kernels' cost does not depend on the values)."""
    from logit_gemm_shard_amd import synth
    from logit_gemm_shard_amd.configs import WORKLOADS
    dev = torch.device("cuda", 0)
    out = {}

    w = WORKLOADS["tiny_mlp_t2_f32"]
    X, A, B = (x.to(dev) for x in synth.mlp_weights(w))
    f = w.f_i
    Z = torch.empty(w.t, w.M, w.h, device=dev)
    Zs = torch.empty(w.M, w.h, device=dev)
    Ys = torch.empty(w.t, w.M, f, device=dev)

    shards = [(A[:, r * f:(r + 1) * f], B[r * f:(r + 1) * f], Z[r], Ys[r]) for r in range(w.t)]

    def tiny():
        for r, (Ar, Br, Zr, Yr) in enumerate(shards):
            lgs.tp_mlp_fwd(w.b, w.s, w.h, w.ffn, w.t, r, X, Ar, Br, Zr, Y_i=Yr)
        lgs.shard_partial_sum("sum", w.t, w.M * w.h, Z, w.M * w.h, Zs)
    # a launch-bound unit: replay it as one HIP graph so that the figure is the
    # device's time, not the host's launch rate
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tiny()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tiny()
    ms = time_calls(torch, graph.replay, reps)
    fl = 2 * 2 * w.M * w.h * w.ffn
    out["tiny_mlp_t2_f32"] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 3),
                              "pct_fp32_peak": round(100 * fl / ms / 1e9 / PEAK_FP32_TFLOPS, 3),
                              "note": "both shards' forward + sum, fp32, replayed as one HIP graph; launch-bound"}

    # 70B-shape rank: three input sets (555 MB of operands, more than the
    # 256 MB Infinity Cache) rotated between calls, 10 warm-up calls, then
    # `reps` calls each timed alone; median and minimum reported.
    w = WORKLOADS["mlp_70b_fwd"]
    f, bf = w.f_i, torch.bfloat16
    sets = []
    for _ in range(3):
        X = torch.randn(w.M, w.h, device=dev).to(bf)
        A0 = torch.randn(w.h, f, device=dev).mul_(0.02).to(bf)
        B0 = torch.randn(f, w.h, device=dev).mul_(synth.residual_std(w.n_blocks)).to(bf)
        sets.append((X, A0, B0))
    U = torch.empty(w.M, f, dtype=bf, device=dev)
    Y = torch.empty(w.M, f, dtype=bf, device=dev)
    Z = torch.empty(w.M, w.h, dtype=bf, device=dev)

    def fwd(i):
        X, A0, B0 = sets[i % 3]
        lgs.tp_mlp_fwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, A0, B0, Z, U_i=U, Y_i=Y)
    fl = 2 * 2 * w.M * w.h * f
    out["mlp_70b_fwd"] = _timed_report(torch, fwd, fl, reps)

    w = WORKLOADS["mlp_70b_bwd"]
    dZs = [torch.randn(w.M, w.h, device=dev).mul_(w.dz_std).to(bf) for _ in range(3)]
    dX = torch.empty(w.M, w.h, dtype=bf, device=dev)
    dA = torch.empty(w.h, f, dtype=bf, device=dev)
    dB = torch.empty(f, w.h, dtype=bf, device=dev)
    ws = torch.empty(lgs.mlp_bwd_workspace_bytes(w.b, w.s, w.h, w.ffn, w.t, bf), dtype=torch.uint8, device=dev)

    def bwd(i):
        X, A0, B0 = sets[i % 3]
        lgs.tp_mlp_bwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, A0, B0, U, dZs[i % 3], dX, dA, dB, workspace=ws)
    fl = 4 * 2 * w.M * w.h * f
    out["mlp_70b_bwd"] = _timed_report(torch, bwd, fl, reps)
    del sets, dZs, dX, dA, dB, ws, U, Y, Z

    # 70B-shape SwiGLU rank (the gated MLP of the same model): forward is the
    # paired [gate | up] GEMM (2 * M * h * 2f) and the down GEMM (2 * M * f * h);
    # backward is dY, dX, dW_gu, dW_down (2 + 4 + 4 + 2) * M * h * f.
    w = WORKLOADS["swiglu_70b_fwd"]
    f = w.f_i
    sets = []
    for _ in range(3):
        X = torch.randn(w.M, w.h, device=dev).to(bf)
        Wgu = torch.randn(w.h, 2 * f, device=dev).mul_(0.02).to(bf)
        Wd = torch.randn(f, w.h, device=dev).mul_(synth.residual_std(w.n_blocks)).to(bf)
        sets.append((X, Wgu, Wd))
    GU = torch.empty(w.M, 2 * f, dtype=bf, device=dev)
    Y = torch.empty(w.M, f, dtype=bf, device=dev)
    Z = torch.empty(w.M, w.h, dtype=bf, device=dev)

    def sfwd(i):
        X, Wgu, Wd = sets[i % 3]
        lgs.tp_swiglu_fwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, Wgu, Wd, Z, GU_i=GU, Y_i=Y)
    out["swiglu_70b_fwd"] = _timed_report(torch, sfwd, 6 * w.M * w.h * f, reps)

    w = WORKLOADS["swiglu_70b_bwd"]
    dZs = [torch.randn(w.M, w.h, device=dev).mul_(w.dz_std).to(bf) for _ in range(3)]
    dX = torch.empty(w.M, w.h, dtype=bf, device=dev)
    dWgu = torch.empty(w.h, 2 * f, dtype=bf, device=dev)
    dWd = torch.empty(f, w.h, dtype=bf, device=dev)
    ws = torch.empty(lgs.swiglu_bwd_workspace_bytes(w.b, w.s, w.h, w.ffn, w.t, bf), dtype=torch.uint8,
                     device=dev)

    def sbwd(i):
        X, Wgu, Wd = sets[i % 3]
        lgs.tp_swiglu_bwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, Wgu, Wd, GU, dZs[i % 3], dX, dWgu, dWd, workspace=ws)
    out["swiglu_70b_bwd"] = _timed_report(torch, sbwd, 12 * w.M * w.h * f, reps)
    del sets, dZs, dX, dWgu, dWd, ws, GU, Y, Z

    # 70B-shape attention projections of one rank (8 query heads, 1 KV head of
    # 128): forward = QKV (2 M h (q + 2 kv)) + W_O (2 M q h); backward = their
    # input and weight gradients (twice that).
    w = WORKLOADS["attn_70b"]
    q, kv = w.n_heads // w.t * w.head_dim, w.n_kv_heads // w.t * w.head_dim
    nqkv = q + 2 * kv
    sets = []
    for _ in range(3):
        X = torch.randn(w.M, w.h, device=dev).to(bf)
        Wqkv = torch.randn(w.h, nqkv, device=dev).mul_(0.02).to(bf)
        Wo = torch.randn(q, w.h, device=dev).mul_(synth.residual_std(w.n_blocks)).to(bf)
        A = torch.randn(w.M, q, device=dev).to(bf)
        dZ = torch.randn(w.M, w.h, device=dev).mul_(w.dz_std).to(bf)
        dQ = torch.randn(w.M, nqkv, device=dev).mul_(w.dz_std).to(bf)
        sets.append((X, Wqkv, Wo, A, dZ, dQ))
    QKV = torch.empty(w.M, nqkv, dtype=bf, device=dev)
    Z = torch.empty(w.M, w.h, dtype=bf, device=dev)
    dX = torch.empty(w.M, w.h, dtype=bf, device=dev)
    dW = torch.empty(w.h, nqkv, dtype=bf, device=dev)
    dA = torch.empty(w.M, q, dtype=bf, device=dev)
    dWo = torch.empty(q, w.h, dtype=bf, device=dev)
    a = (w.b, w.s, w.h)
    ws_qkv = torch.empty(max(1, lgs.attn_qkv_fwd_workspace_bytes(*a, w.n_heads, w.n_kv_heads, w.head_dim, w.t)),
                         dtype=torch.uint8, device=dev)

    def afwd(i):
        X, Wqkv, Wo, A, _, _ = sets[i % 3]
        lgs.tp_attn_qkv_fwd(*a, w.n_heads, w.n_kv_heads, w.head_dim, w.t, 0, X, Wqkv, QKV, workspace=ws_qkv)
        lgs.tp_attn_out_fwd(*a, w.n_heads, w.head_dim, w.t, 0, A, Wo, Z)

    ws_ob = torch.empty(max(1, lgs.attn_out_bwd_workspace_bytes(*a, w.n_heads, w.head_dim, w.t)),
                        dtype=torch.uint8, device=dev)

    def abwd(i):
        X, Wqkv, Wo, A, dZ, dQ = sets[i % 3]
        lgs.tp_attn_qkv_bwd(*a, w.n_heads, w.n_kv_heads, w.head_dim, w.t, 0, X, Wqkv, dQ, dX, dW)
        lgs.tp_attn_out_bwd(*a, w.n_heads, w.head_dim, w.t, 0, A, Wo, dZ, dA, dWo, workspace=ws_ob)
    fl = 2 * w.M * w.h * (nqkv + q)
    out["attn_70b_fwd"] = _timed_report(torch, afwd, fl, reps)
    out["attn_70b_bwd"] = _timed_report(torch, abwd, 2 * fl, reps)
    return out


def _timed_report(torch, fn, flops, reps, warmup=10):
    """fn(i) timed call by call with HIP events on the current stream."""
    for i in range(warmup):
        fn(i)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med, mn = ms[len(ms) // 2], ms[0]
    return {"ms": round(med, 4), "ms_min": round(mn, 4), "runs": reps,
            "tflops": round(flops / med / 1e9, 2), "tflops_best": round(flops / mn / 1e9, 2),
            "pct_bf16_peak": round(100 * flops / med / 1e9 / PEAK_BF16_TFLOPS, 2),
            "note": "median of per-call times, 3 rotated input sets"}


def ce_reduction_stream(torch, lgs, xw, reps=30):
    """The CE reductions alone, streamed from materialised bf16 logits of the
    rank's slice (a testing entry point; the product path fuses them into the
    logit GEMM and never writes logits).  Three logit buffers (315 MB, more
    than the 256 MB Infinity Cache) are rotated so every launch reads HBM."""
    dev = torch.device("cuda", 0)
    M, Vr = xw.M, xw.v_r
    bufs = [torch.randn(M, Vr, device=dev).to(torch.bfloat16) for _ in range(3)]
    y = torch.randint(0, xw.vocab, (M,), device=dev, dtype=torch.int32)
    out = torch.empty(3, M, device=dev)
    i = [0]

    def one():
        lgs.xent_rows_bf16(bufs[i[0] % 3], y, 0, out[0], out[1], out[2])
        i[0] += 1
    ms = time_calls(torch, one, reps, warmup=3)
    nbytes = M * Vr * 2 + M * 4 + 3 * M * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "xent_rows_kernel (lgs_test_xent_rows_bf16): CE slice reductions over "
                      f"materialised bf16 logits [{M}, {Vr}]",
            "us": round(ms * 1e3, 2), "bytes": nbytes, "achieved_GBs": round(gbs, 1),
            "peak_GBs": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the graphics clock while the step repeats (profiler runs)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-configuration timings (counter passes)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="time torch.matmul (hipBLASLt) at the library's GEMM shapes and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's shard: the library is measured on one GPU "
              "(all t ranks of the split are timed or checked on that one device); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    if args.blas_reference:
        blas_reference()
        return

    from logit_gemm_shard_amd import binding as lgs
    from logit_gemm_shard_amd import synth
    from logit_gemm_shard_amd.configs import WORKLOADS

    w, xw = WORKLOADS["mlp_8p3b_fwd"], WORKLOADS["xent_8p3b"]
    M, h, f, t, ffn = w.M, w.h, w.f_i, w.t, w.ffn
    V, Vr = xw.vocab, xw.v_r
    bf = torch.bfloat16
    dev = torch.device("cuda", 0)

    # ---------------- inputs (host, seeded) -> HBM
    X, A, B = synth.mlp_weights(w)
    dZ = synth.normal((M, h), 0.01, 6, "bf16")
    H, E, y = synth.xent_inputs(xw)
    A0, B0, E0 = A[:, :f].contiguous(), B[:f].contiguous(), E[:Vr].contiguous()
    Xd, A0d, B0d, dZd = X.to(dev), A0.to(dev), B0.to(dev), dZ.to(dev)
    Hd, E0d, yd = H.to(dev), E0.to(dev), y.to(dev)
    U = torch.empty(M, f, dtype=bf, device=dev)
    Y = torch.empty(M, f, dtype=bf, device=dev)
    zparts = torch.randn(t, M, h, device=dev).mul_(0.05).to(bf)   # ranks 1..7: "received" partials
    dxparts = torch.randn(t, M, h, device=dev).mul_(0.01).to(bf)
    Z = torch.empty(M, h, dtype=bf, device=dev)
    dX = torch.empty(M, h, dtype=bf, device=dev)
    dA = torch.empty(h, f, dtype=bf, device=dev)
    dB = torch.empty(f, h, dtype=bf, device=dev)
    stats = torch.empty(t, 3, M, dtype=torch.float32, device=dev)
    stats[:, 0].normal_()
    stats[:, 1].uniform_(1.0, 100.0)
    stats[:, 2].zero_()
    loss = torch.empty(M, dtype=torch.float32, device=dev)
    ws_bwd = torch.empty(lgs.mlp_bwd_workspace_bytes(w.b, w.s, h, ffn, t, bf), dtype=torch.uint8, device=dev)
    ws_xent = torch.empty(lgs.xent_workspace_bytes(xw.b, xw.s, h, V, t), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    names = ["mlp_fwd", "sum_z", "mlp_bwd", "sum_dx", "xent", "xent_merge"]

    def one_step(ev=None, marks=(0, 1, 2, 3, 4, 5, 6)):
        def mark(i):
            if ev is not None and i in marks:
                ev[i].record(stream)
        mark(0)
        lgs.tp_mlp_fwd(w.b, w.s, h, ffn, t, 0, Xd, A0d, B0d, zparts[0], U_i=U, Y_i=Y, stream=stream)
        mark(1)
        lgs.shard_partial_sum("sum", t, M * h, zparts, M * h, Z, stream=stream)
        mark(2)
        lgs.tp_mlp_bwd(w.b, w.s, h, ffn, t, 0, Xd, A0d, B0d, U, dZd, dxparts[0], dA, dB,
                       workspace=ws_bwd, stream=stream)
        mark(3)
        lgs.shard_partial_sum("sum", t, M * h, dxparts, M * h, dX, stream=stream)
        mark(4)
        lgs.vocab_parallel_xent_fwd(xw.b, xw.s, h, V, t, 0, Hd, E0d, yd, stats[0, 0], stats[0, 1],
                                    stats[0, 2], workspace=ws_xent, stream=stream)
        mark(5)
        lgs.shard_partial_sum("xent", t, M, stats, 3 * M, loss, stream=stream)
        mark(6)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    fl = step_flops(M, h, f, Vr)
    # The per-configuration timings, the streaming CE measurement and the clock
    # sampling run before the timed steps, so that those see the device in the
    # steady state a training run keeps it in (the first tens of steps after
    # start-up run several percent slower while clocks and caches settle).
    configs = {} if args.no_per_config else per_config(torch, lgs, reps=50)
    if not args.no_per_config:
        # CE backward of the same slice from the merged log-sum-exp, dloss = 1/M:
        # the recomputed logit GEMM with its gradient epilogue, then dH_0 = G E_0
        # and dE_0 = G^T H in one launch (3 x 2 M h V_r FLOP).
        lse = torch.empty(M, dtype=torch.float32, device=dev)
        lgs.shard_partial_sum("xent_lse", t, M, stats, 3 * M, lse)
        dl = torch.full((M,), 1.0 / M, dtype=torch.float32, device=dev)
        dH0 = torch.empty(M, h, dtype=bf, device=dev)
        dE0 = torch.empty(Vr, h, dtype=bf, device=dev)
        ws_xb = torch.empty(lgs.xent_bwd_workspace_bytes(xw.b, xw.s, h, V, t), dtype=torch.uint8, device=dev)

        def xbwd(i):
            lgs.vocab_parallel_xent_bwd(xw.b, xw.s, h, V, t, 0, Hd, E0d, yd, lse, dH0, dE0, dloss=dl,
                                        workspace=ws_xb, stream=stream)
        rep = _timed_report(torch, xbwd, 3 * fl["xent"], 50)
        rep["tokens_per_s"] = round(M / (rep["ms"] * 1e-3), 0)
        rep["note"] = "median of per-call times; one input set (the step's)"
        configs["xent_8p3b_bwd"] = rep
        del lse, dl, dH0, dE0, ws_xb
        # sequence-parallel stand-ins at the same shape (s = 1024, b = 8, h = 3072,
        # t = 8): rank 0's reduce-scatter of the 8 partials, and the all-gather of
        # 8 chunks into [s*b, h]; both pure HBM streams
        chunk = M * h // t
        rs_out = torch.empty(M // t, h, dtype=bf, device=dev)
        ag_in = torch.randn(t, M // t, h, device=dev).to(bf)
        ag_out = torch.empty(M, h, dtype=bf, device=dev)
        rs_ms = time_calls(torch, lambda: lgs.shard_reduce_scatter(t, 0, w.s, w.b, h, zparts, M * h, rs_out), 50)
        ag_ms = time_calls(torch, lambda: lgs.shard_all_gather(t, w.s, w.b, h, ag_in, chunk, ag_out), 50)
        rs_bytes, ag_bytes = (t + 1) * chunk * 2, 2 * M * h * 2
        configs["sp_8p3b"] = {
            "reduce_scatter_us": round(rs_ms * 1e3, 2),
            "reduce_scatter_GBs": round(rs_bytes / (rs_ms * 1e-3) / 1e9, 1),
            "all_gather_us": round(ag_ms * 1e3, 2),
            "all_gather_GBs": round(ag_bytes / (ag_ms * 1e-3) / 1e9, 1),
            "note": "bytes = every byte read once + written once; HBM peak 8000 GB/s"}
        del rs_out, ag_in, ag_out
        stream_ce = ce_reduction_stream(torch, lgs, xw)
    gpu_clock = None if args.no_clock else sample_gpu_clock(torch, one_step)

    # Timed region: K whole steps.  Only the CE entry point is bracketed by HIP
    # events here (its roofline is measured live); events between every entry
    # point cost the step about 2.5%, so the per-entry-point breakdown comes
    # from a second, untimed pass of K steps below.
    ce_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(ce_ev[i], marks=(4, 5))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    xent_s = sum(e[4].elapsed_time(e[5]) for e in ce_ev) / args.steps * 1e-3

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    per = {n: 0.0 for n in names}
    for ev in evs:
        for j, n in enumerate(names):
            per[n] += ev[j].elapsed_time(ev[j + 1])
    per = {n: v / args.steps for n, v in per.items()}   # ms per launch of each entry point

    total_flops = sum(fl.values())
    tflops = total_flops / (ms * 1e-3) / 1e12
    sum_bytes = (t + 1) * M * h * 2
    traffic = read_counters()
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, residual weight scaled 1/sqrt(2N), uniform targets)",
        "config": {"workload": "8.3B-shape TP shard step, rank 0 of t=8: GeLU MLP fwd+bwd "
                               "(b=8, s=1024, h=3072, ffn=12288) + sums of 8 partials + vocab-parallel "
                               "fused CE (vocab 51200) + CE merge",
                   "b": w.b, "s": w.s, "h": h, "ffn": ffn, "t": t, "rank": 0, "vocab": V},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "gpu_clock": gpu_clock,
        "timing": "value and ms_per_step: wall clock over the K timed steps (events around the CE call "
                  "only); entry_point_ms: a separate pass of K steps with events between entry points",
        "mlp_fwd_bwd_tflops": round((fl["mlp_fwd"] + fl["mlp_bwd"]) / ((per["mlp_fwd"] + per["mlp_bwd"]) * 1e-3) / 1e12, 2),
        "mlp_fwd_tflops": round(fl["mlp_fwd"] / (per["mlp_fwd"] * 1e-3) / 1e12, 2),
        "mlp_bwd_tflops": round(fl["mlp_bwd"] / (per["mlp_bwd"] * 1e-3) / 1e12, 2),
        "ce_tokens_per_s": round(M / xent_s, 0),
        "ce_tflops": round(fl["xent"] / xent_s / 1e12, 2),
        "sum_partials_gbs": round(sum_bytes / (per["sum_z"] * 1e-3) / 1e9, 1),
        "entry_point_ms": {n: round(v, 4) for n, v in per.items()},
        "roofline": {
            "kernel": "vocab_parallel_xent_fwd (fused logit GEMM + CE partials, with its slab merge)",
            "bound": "mfma",
            "achieved": round(fl["xent"] / xent_s / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fl["xent"] / xent_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    configs["mlp_8p3b_fwd"] = {"ms": round(per["mlp_fwd"], 4), "tflops": out["mlp_fwd_tflops"],
                               "pct_bf16_peak": round(100 * out["mlp_fwd_tflops"] / PEAK_BF16_TFLOPS, 2),
                               "note": "from the event pass over the step"}
    configs["xent_8p3b"] = {"ms": round(xent_s * 1e3, 4), "tflops": out["ce_tflops"],
                            "pct_bf16_peak": round(100 * out["ce_tflops"] / PEAK_BF16_TFLOPS, 2),
                            "tokens_per_s": out["ce_tokens_per_s"], "note": "from the timed steps"}
    out["per_config"] = configs
    if not args.no_per_config:
        out["ce_reduction_stream"] = stream_ce
    if not args.no_cpu_baseline:
        import numpy as np
        inputs = (X.float().numpy(), A0.float().double().numpy(), B0.float().double().numpy(),
                  dZ.float().numpy(), H.float().numpy(), E0.float().double().numpy(),
                  y.numpy().astype(np.int64))
        out["cpu_baseline"] = cpu_baseline(w, xw, inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

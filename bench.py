"""Benchmark: one tensor-parallel rank's transformer-block shard on one MI355X.

A step is one pass of the whole path for rank 0 of t = 8:

  1. tp_mlp_fwd               70B-shape GeLU MLP shard forward (b = 1, s = 4096,
                              h = 8192, ffn = 28672): U_0 = X A_0, Y_0 = GeLU(U_0),
                              Z_0 = Y_0 B_0
  2. shard_partial_sum(SUM)   Z = sum of the 8 ranks' partials [4096, 8192] (rank 0's
                              just written, the other 7 resident synthetic partials)
  3. tp_mlp_bwd               dY, dU = dY GeLU'(U_0), dB_0, dA_0, dX_0 (U_0 from step 1)
  4. shard_partial_sum(SUM)   dX = sum of the 8 ranks' dX partials
  5. vocab_parallel_xent_fwd  fused logit GEMM + CE partials of vocabulary slice 0 of
                              the 8.3B-shape model (8192 tokens, h = 3072, vocab 51200)
  6. shard_partial_sum(XENT)  per-token loss from the 8 ranks' partials

Three input sets (X, A_0, B_0, dZ, H, E_0, targets: about 400 MB each, 1.2 GB in
all, against the 256 MB Infinity Cache) rotate from step to step, so every step
reads its operands from HBM.  All inputs are resident in HBM before timing.

Order of work: W warm-up steps; the per-configuration timings, the streaming CE
measurement and the clock sampling (so that the timed steps see the device
settled); the timed region, K steps between two synchronizations, with HIP
events around the backward entry point only (its roofline is measured there);
then an untimed pass of K steps with events between every entry point for the
per-entry-point breakdown.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-per-config] [--no-clock]
    python bench.py --copy-calibration   # plain copy for counter scaling
    python bench.py --blas-reference     # torch.matmul (hipBLASLt) at the same GEMM shapes
    python bench.py --counter-summary DIR  # write the traffic summary from rocprofv3 --pmc passes in DIR
    python bench.py --kernel-stats CSV TITLE COMMAND  # markdown table from a rocprofv3 kernel_stats.csv
    python bench.py --ce-stream-workload   # the streaming CE reductions alone (counter / trace passes)
    python bench.py --ce-stream-summary DIR  # their HBM bytes and time from rocprofv3 passes under DIR
"""

import argparse
import glob
import hashlib
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
COUNTERS_FILE = os.path.join(ROOT, "profiles", "mlp_70b_bwd_hbm_counters.txt")
INFINITY_CACHE_BYTES = 256 << 20


def kernel_sources_digest():
    """sha256 over the HIP sources: counters are only valid for the code they were taken on."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "logit_gemm_shard_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()


def mlp_flops(M, h, f):
    """Algorithmic FLOPs (2 M N K per GEMM) of one rank's MLP shard: forward
    2 GEMMs, backward 4 (the 6 P T rule)."""
    return {"fwd": 2 * 2 * M * h * f, "bwd": 4 * 2 * M * h * f}


def xent_flops(M, h, Vr):
    return 2 * M * h * Vr


def mlp_bwd_bytes(M, h, f):
    """Algorithmic HBM bytes of one tp_mlp_bwd call (bf16): its two launches
    read X, A_i, B_i, U_i and dZ once, write dX_i, dA_i, dB_i once, and pass
    Y_i and dU_i from the first launch to the second (written and read once)."""
    e = 2
    inputs = M * h + h * f + f * h + M * f + M * h
    outputs = M * h + h * f + f * h
    between = 2 * (2 * M * f)
    return e * (inputs + outputs + between)


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
    """HBM bytes per tp_mlp_bwd call from the committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
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
        return float(vals["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _per_kernel(path, counter):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 CSV
    (a dispatch's value summed over its rows, e.g. over XCDs)."""
    import collections
    import csv
    by_disp, names = collections.defaultdict(float), {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        by_disp[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for k, v in by_disp.items():
        out[names[k]].append(v)
    return out


def counter_summary(d):
    """Write COUNTERS_FILE from four rocprofv3 --pmc passes under directory d:
    pmc_FETCH_SIZE and pmc_WRITE_SIZE over `bench.py --steps 2 --warmup 1
    --no-cpu-baseline --no-per-config --no-clock`, and pmc_copy_FETCH_SIZE and
    pmc_copy_WRITE_SIZE over `bench.py --copy-calibration`.  The counters are
    KiB per dispatch; each is scaled by what it reads for the plain 1 GiB copy."""
    import statistics

    def csv_of(sub):
        found = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not found:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(d, sub)}")
        return found[0]

    med = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        step = _per_kernel(csv_of(f"pmc_{c}"), c)
        copy = _per_kernel(csv_of(f"pmc_copy_{c}"), c)
        dy = [v for n, v in step.items() if "EpiGeluBwd" in n]
        grp = [v for n, v in step.items() if "gemm_pp_group3" in n]
        cp = [v for n, v in copy.items() if "neg" in n]
        if len(dy) != 1 or len(grp) != 1 or len(cp) != 1:
            raise SystemExit(f"{c}: expected one dY+GeLU' kernel, one grouped kernel and one copy kernel, "
                             f"found {len(dy)}, {len(grp)}, {len(cp)}")
        med[c] = (statistics.median(dy[0]), statistics.median(grp[0]), statistics.median(cp[0]))
    fr = (1 << 30) / (med["FETCH_SIZE"][2] * 1024)
    fw = (1 << 30) / (med["WRITE_SIZE"][2] * 1024)

    def nbytes(i):
        return med["FETCH_SIZE"][i] * 1024 * fr + med["WRITE_SIZE"][i] * 1024 * fw
    M, h, f = 4096, 8192, 3584
    alg = mlp_bwd_bytes(M, h, f)
    step_cmd = "python bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-per-config --no-clock"
    txt = f"""# HBM-side traffic of the MLP backward entry point (tp_mlp_bwd) on the
# 70B-shape workload (rank 0 of t = 8: M = 4096 tokens, h = 8192, f = 3584),
# from rocprofv3 counter passes, one counter per run:
#
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc/pmc_FETCH_SIZE -o p -- {step_cmd}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc/pmc_WRITE_SIZE -o p -- {step_cmd}
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc/pmc_copy_FETCH_SIZE -o p -- python bench.py --copy-calibration
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc/pmc_copy_WRITE_SIZE -o p -- python bench.py --copy-calibration
#   python bench.py --counter-summary rocprof_out/pmc      (writes this file)
#
# Calibration: an elementwise pass over 1 GiB (torch.neg: reads 1 GiB, writes
# 1 GiB) reads FETCH_SIZE = {med['FETCH_SIZE'][2]:.0f} KiB and WRITE_SIZE = {med['WRITE_SIZE'][2]:.0f} KiB per dispatch, so
# bytes = FETCH_SIZE x 1024 x {fr:.4f} and WRITE_SIZE x 1024 x {fw:.4f}.
#
# Per call (median over the dispatches of each kernel):
#   dY + GeLU' GEMM (writes dU_i and the recomputed Y_i): FETCH_SIZE {med['FETCH_SIZE'][0]:.0f} KiB, WRITE_SIZE {med['WRITE_SIZE'][0]:.0f} KiB -> {nbytes(0) / 1e6:.1f} MB
#   grouped dB / dA / dX launch (the last 128 dA tiles in two parts over the
#   tokens, with 64 MB of fp32 partial slots written and read back):
#                                                        FETCH_SIZE {med['FETCH_SIZE'][1]:.0f} KiB, WRITE_SIZE {med['WRITE_SIZE'][1]:.0f} KiB -> {nbytes(1) / 1e6:.1f} MB
#   algorithmic bytes of the call (X, A_i, B_i, U_i, dZ read once; dX_i, dA_i,
#   dB_i written once; Y_i and dU_i written and read once): {alg / 1e6:.1f} MB
#   (the third launch of the call, which clears the 128 split tiles' counters,
#   writes 512 bytes)
#
# The counters count every request that leaves the L2s for the memory fabric;
# they cannot separate HBM reads from hits in the 256 MB Infinity Cache in
# front of HBM.  Traffic above the algorithmic bytes is operand panels fetched
# again by the L2 of each of the 8 XCDs for its own tiles.
kernel_sources_sha256: {kernel_sources_digest()}
hbm_bytes_per_call: {nbytes(0) + nbytes(1):.0f}
"""
    open(COUNTERS_FILE, "w").write(txt)
    print(txt)
    ce_counter_summary(d, fr, fw)


STREAM_COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_stream_kernels_counters.txt")


def stream_workload(torch, lgs, calls=5):
    """The HBM-bound kernels alone, for counter passes: the sum of 8 partials
    at the 70B shape, and at the 8.3B shape (s = 1024, b = 8, h = 3072, t = 8)
    the sequence-parallel reduce-scatter, all-gather, fused region and its
    backward; `calls` calls each, successive calls on successive ranks'
    chunks as in the per-configuration timings."""
    from logit_gemm_shard_amd.configs import WORKLOADS
    dev = torch.device("cuda", 0)
    bf = torch.bfloat16

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, device=dev) * std).to(bf)
    M, h = 4096, 8192
    parts = randn(8, M, h, std=0.05)
    zs = torch.empty(M, h, dtype=bf, device=dev)
    for _ in range(calls):
        lgs.shard_partial_sum("sum", 8, M * h, parts, M * h, zs)
    torch.cuda.synchronize()
    del parts, zs
    w = WORKLOADS["mlp_8p3b_fwd"]
    t, M, h = w.t, w.M, w.h
    chunk = M * h // t
    parts = randn(t, M, h, std=0.05)
    rs_out = torch.empty(M // t, h, dtype=bf, device=dev)
    ag_in = [randn(t, M // t, h) for _ in range(3)]
    ag_out = torch.empty(M, h, dtype=bf, device=dev)
    res, dys, dhss = randn(t, M // t, h), randn(t, M // t, h), randn(t, M // t, h)
    keep = (torch.rand(t, M // t, h, device=dev) > 0.1).to(torch.uint8)
    gamma, beta = randn(h, std=0.1) + 1, randn(h, std=0.1)
    hs, ys = torch.empty(M // t, h, dtype=bf, device=dev), torch.empty(M // t, h, dtype=bf, device=dev)
    gg, dzz = torch.empty(M // t, h, dtype=bf, device=dev), torch.empty(M // t, h, dtype=bf, device=dev)
    dgam, dbet = torch.empty(h, device=dev), torch.empty(h, device=dev)
    lws = torch.empty(lgs.layernorm_bwd_workspace_bytes(t, w.s, w.b, h), dtype=torch.uint8, device=dev)
    for i in range(calls):
        lgs.shard_reduce_scatter(t, i % t, w.s, w.b, h, parts, M * h, rs_out)
    for i in range(calls):
        lgs.shard_all_gather(t, w.s, w.b, h, ag_in[i % 3], chunk, ag_out)
    for i in range(calls):
        lgs.shard_reduce_scatter_layernorm(t, i % t, w.s, w.b, h, parts, M * h, res[i % t], gamma, beta, hs, ys,
                                           keep=keep[i % t], keep_scale=1 / 0.9)
    for i in range(calls):
        lgs.shard_layernorm_bwd(t, i % t, w.s, w.b, h, res[i % t], dys[i % t], gamma, gg, dzz, dgam, dbet,
                                dhs=dhss[i % t], keep=keep[i % t], keep_scale=1 / 0.9, workspace=lws)
    torch.cuda.synchronize()
    print(json.dumps({"stream_workload": "done", "calls": calls}), flush=True)


def _per_kernel_grid(path, counter):
    """{(kernel name, grid size): [value per dispatch]} for one counter."""
    import collections
    import csv
    by_disp, keys = collections.defaultdict(float), {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        by_disp[r["Dispatch_Id"]] += float(r["Counter_Value"])
        keys[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]))
    out = collections.defaultdict(list)
    for k, v in by_disp.items():
        out[keys[k]].append(v)
    return out


def stream_summary(d):
    """Write STREAM_COUNTERS_FILE from rocprofv3 --pmc passes under directory d:
    pmc_st_FETCH_SIZE and pmc_st_WRITE_SIZE over `bench.py --stream-workload`,
    pmc_copy_FETCH_SIZE and pmc_copy_WRITE_SIZE over `bench.py --copy-calibration`."""
    import statistics

    def csv_of(sub):
        found = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not found:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(d, sub)}")
        return found[0]
    t, M83, h83 = 8, 8192, 3072
    chunk = M83 * h83 // t
    nblk = 256
    # (label, name pattern, grid size or None, algorithmic bytes)
    kernels = (
        ("sum of 8 partials, 70B [4096, 8192] (psum_vec_kernel)", "psum_vec_kernel", 8192 * 256, 9 * 4096 * 8192 * 2),
        ("SP reduce-scatter, rank rows of 8 partials (psum_vec_kernel)", "psum_vec_kernel", (chunk // 2048) * 256,
         (t + 1) * chunk * 2),
        ("SP all-gather (gather_vec_kernel)", "gather_vec_kernel", None, 2 * M83 * h83 * 2),
        ("SP region fused (rs_layernorm_kernel)", "rs_layernorm_kernel", None,
         (t + 1) * chunk * 2 + chunk + 2 * chunk * 2 + 2 * h83 * 2),
        ("SP region backward, rows (layernorm_bwd_kernel)", "layernorm_bwd_kernel", None,
         3 * chunk * 2 + chunk + 2 * chunk * 2 + h83 * 2 + nblk * 2 * h83 * 4),
        ("SP region backward, column sum (col_sum_kernel)", "col_sum_kernel", None, nblk * 2 * h83 * 4 + 2 * h83 * 4),
    )
    med, cal = {}, {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        got = _per_kernel_grid(csv_of(f"pmc_st_{c}"), c)
        copy = _per_kernel(csv_of(f"pmc_copy_{c}"), c)
        cp = [v for n, v in copy.items() if "neg" in n]
        if len(cp) != 1:
            raise SystemExit(f"{c}: expected one copy kernel, found {len(cp)}")
        cal[c] = statistics.median(cp[0])
        for label, pat, grid, _ in kernels:
            vals = [v for (n, g), v in got.items() if pat in n and (grid is None or g == grid)]
            if len(vals) != 1:
                raise SystemExit(f"{c}: {label}: expected one kernel, found {len(vals)}")
            med[(label, c)] = statistics.median(vals[0])
    fr = (1 << 30) / (cal["FETCH_SIZE"] * 1024)
    fw = (1 << 30) / (cal["WRITE_SIZE"] * 1024)
    lines = []
    for label, _, _, alg in kernels:
        rd, wr = med[(label, "FETCH_SIZE")] * 1024 * fr, med[(label, "WRITE_SIZE")] * 1024 * fw
        lines.append(f"#   {label}:\n#     read {rd / 1e6:.1f} MB + written {wr / 1e6:.1f} MB = {(rd + wr) / 1e6:.1f} MB"
                     f" against {alg / 1e6:.1f} MB algorithmic ({(rd + wr) / alg:.3f}x)")
    body = "\n".join(lines)
    txt = f"""# L2-to-fabric traffic of the HBM-bound kernels: the sum of 8 partials at the
# 70B shape and the sequence-parallel kernels at the 8.3B shape (rank chunks of
# 1024 rows x 3072; t = 8), from rocprofv3 counter passes, one counter per run:
#
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc_st/pmc_st_FETCH_SIZE -o p -- python bench.py --stream-workload
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc_st/pmc_st_WRITE_SIZE -o p -- python bench.py --stream-workload
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc_st/pmc_copy_FETCH_SIZE -o p -- python bench.py --copy-calibration
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc_st/pmc_copy_WRITE_SIZE -o p -- python bench.py --copy-calibration
#   python bench.py --stream-summary rocprof_out/pmc_st      (writes this file)
#
# Per launch (median over five), FETCH_SIZE x 1024 x {fr:.4f} and WRITE_SIZE x 1024 x {fw:.4f}
# (the calibration of the plain 1 GiB copy); algorithmic bytes: every input read once and
# every output written once (the backward's rows kernel also writes its fp32 column partials,
# which the column sum reads):
{body}
kernel_sources_sha256: {kernel_sources_digest()}
"""
    open(STREAM_COUNTERS_FILE, "w").write(txt)
    print(txt)


XENT_COUNTERS_FILE = os.path.join(ROOT, "profiles", "xent_8p3b_hbm_counters.txt")


def block_tile(pid, n, tiles_m, tiles_n, xcds=8, group_m=4):
    """The library's block-to-tile map for a launch of n blocks over a
    tiles_m x tiles_n grid: block ids are dealt to the XCDs round-robin, so
    (when n divides by the XCD count) they are renumbered to give every XCD a
    contiguous run, which then walks the tiles in groups of group_m tile rows.
    Returns (tile row, tile column)."""
    if n % xcds == 0:
        per = n // xcds
        pid = (pid % xcds) * per + pid // xcds
    width = group_m * tiles_n
    g = pid // width
    first = g * group_m
    gsz = min(tiles_m - first, group_m)
    inn = pid - g * width
    return first + inn % gsz, inn // gsz


def panel_fill_model(tiles_m, tiles_n, bm, bn, k_bytes, xcds=8, group_m=4, cus=256):
    """L2 fills of one launch if every XCD's L2 fetches, per round of its
    concurrent tiles, each operand panel those tiles cover once: blocks go to
    XCDs round-robin, each XCD owns a contiguous run of the grouped tile order
    (block_tile), and a round is `cus` blocks.  Returns bytes."""
    n = tiles_m * tiles_n
    total = 0
    for r0 in range(0, n, cus):
        for x in range(xcds):
            ts = [block_tile(p, n, tiles_m, tiles_n, xcds, group_m) for p in range(r0, min(n, r0 + cus))
                  if p % xcds == x]
            total += (len({t[0] for t in ts}) * bm + len({t[1] for t in ts}) * bn) * k_bytes
    return total


def ce_counter_summary(d, fr, fw):
    """The fused CE's share of the same counter passes (the step runs it on
    slice 0 of the 8.3B shapes), next to panel_fill_model for each of its
    two GEMM launches (K = 3072 bf16: 6144 bytes per panel row or column)."""
    import statistics

    def csv_of(sub):
        return glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)[0]
    launches = []  # (kernel name pattern, label, columns, bm, bn)
    for pat, label, cols, bm, bn in (("256, 320, true, true, lgs::EpiXent>", "256x320 launch (columns 0-2559)", 2560, 256, 320),
                                      ("256, 256, true, true, lgs::EpiXent>", "256x256 launch (columns 2560-6399)", 3840, 256, 256)):
        launches.append((pat, label, cols, bm, bn))
    med = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        step = _per_kernel(csv_of(f"pmc_{c}"), c)
        for pat, label, *_ in launches + [("xent_merge_kernel", "merge", 0, 0, 0)]:
            v = [x for n, x in step.items() if pat in n]
            if len(v) != 1:
                raise SystemExit(f"{c}: expected one CE kernel matching {pat!r}, found {len(v)}")
            med[(c, label)] = statistics.median(v[0])

    def mb(label):
        return (med[("FETCH_SIZE", label)] * 1024 * fr + med[("WRITE_SIZE", label)] * 1024 * fw) / 1e6
    k_bytes = 3072 * 2
    alg = (8192 * 3072 + 6400 * 3072) * 2 / 1e6
    rows = []
    model_total = 0.0
    for pat, label, cols, bm, bn in launches:
        model = panel_fill_model(-(-8192 // bm), -(-cols // bn), bm, bn, k_bytes) / 1e6
        model_total += model
        rows.append(f"#   {label}: FETCH_SIZE {med[('FETCH_SIZE', label)]:.0f} KiB, WRITE_SIZE "
                    f"{med[('WRITE_SIZE', label)]:.0f} KiB -> {mb(label):.1f} MB; panel model {model:.1f} MB")
    best = panel_fill_model(32, 20, 256, 320, k_bytes, group_m=8) / 1e6  # all 6400 columns
    step_cmd = "python bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-per-config --no-clock"
    nl = chr(10)
    txt = f"""# L2-to-fabric traffic of the fused CE entry point (vocab_parallel_xent_fwd) on
# the 8.3B-shape slice (rank 0 of t = 8: M = 8192 tokens, h = 3072, V_r = 6400),
# from the same rocprofv3 counter passes over the step as
# mlp_70b_bwd_hbm_counters.txt (one counter per run):
#
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc/pmc_FETCH_SIZE -o p -- {step_cmd}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc/pmc_WRITE_SIZE -o p -- {step_cmd}
#   (+ the two copy-calibration passes; python bench.py --counter-summary rocprof_out/pmc writes this file)
#
# The library's column plan for this slice: columns 0-2559 on 256x320 tiles
# (256 tiles, one round), columns 2560-6399 on 256x256 tiles (480 tiles).
# Per launch (median of the dispatches), bytes = FETCH_SIZE x 1024 x {fr:.4f} + WRITE_SIZE x 1024 x {fw:.4f},
# next to the panel model: per round of 256 blocks, each XCD's L2 fetches
# every H row panel and E_r column panel of its 32 concurrent tiles once
# (bench.panel_fill_model, from the library's block-to-tile map):
{nl.join(rows)}
#   slab merge: FETCH_SIZE {med[('FETCH_SIZE', 'merge')]:.0f} KiB, WRITE_SIZE {med[('WRITE_SIZE', 'merge')]:.0f} KiB -> {mb('merge'):.1f} MB
#   algorithmic operand bytes (H and E_r read once): {alg:.1f} MB
#
# The traffic above the algorithmic bytes is the panels that the 8 XCDs'
# separate L2s each fetch (served by the Infinity Cache, which holds H and E_r
# whole).  No tile order brings it near the algorithmic bytes: the whole slice
# on 256x320 tiles with each XCD's concurrent tiles in the most compact block
# (8 row tiles x 4 column tiles) would still fetch {best:.1f} MB, {best / alg:.1f}x
# the algorithmic bytes.
kernel_sources_sha256: {kernel_sources_digest()}
hbm_bytes_per_launch: {(sum(mb(l[1]) for l in launches) + mb('merge')) * 1e6:.0f}
"""
    open(XENT_COUNTERS_FILE, "w").write(txt)
    print(txt)



def kernel_stats_md(src, title, cmd):
    """A short markdown table of a rocprofv3 kernel_stats.csv (our mangled
    kernel names shortened to their template arguments)."""
    import csv
    import re

    def short(n):
        if n.startswith("_Z"):
            parts, i = [], 2
            while i < len(n):
                m = re.match(r"Li(\d+)E|Lb([01])E", n[i:])
                if m:
                    parts.append(m.group(1) or ("true" if m.group(2) == "1" else "false"))
                    i += m.end()
                    continue
                m = re.match(r"(\d+)", n[i:])
                if m and i > 0 and not n[i - 1].isdigit():
                    L = int(m.group(1))
                    j = i + m.end()
                    parts.append(n[j:j + L])
                    i = j + L
                    continue
                if n[i:i + 4] == "DF16":
                    parts.append("bf16")
                    i += 5
                    continue
                i += 1
            n = " ".join(p for p in parts if p != "lgs")
        n = n.replace("lgs::", "").replace("__hip_bfloat16", "bf16")
        return re.sub(r"at::native::.*", lambda m: "torch: " + m.group(0)[:70], n)

    out = [f"# {title}", "", "Command (from the repository root):", "", "```", cmd, "```", "",
           "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(src)):
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    print("\n".join(out))


def cpu_baseline(host, reps_budget_s=6.0):
    """The fp64 oracle as it stands (plain numpy, BLAS dgemm) on the host's
    cores, on the same seeded inputs as the GPU step's first input set:
      value       the whole step (70B forward and its sum of 8 partials,
                  backward and its sum, the CE slice of rank 0 and the merge of
                  8 ranks' partials), repeated while it fits the time budget;
      per_config  each configuration's unit of work alone, at full size;
      xent_full_vocab  the naive full-logit CE over all 51,200 columns.
    Input conversion to fp64 and the other ranks' partials are outside the
    timed calls."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    X, A0, B0, dZ = host["X"], host["A0"], host["B0"], host["dZ"]
    H, E, y, Vr, t = host["H"], host["E"], host["y"], host["Vr"], 8
    M, h = X.shape
    f = A0.shape[1]
    Mc, hc = H.shape
    rng = np.random.default_rng(0)
    other = rng.normal(size=(M, h)) * 0.05       # a received partial (the same values for every rank)
    st = (rng.normal(size=(t - 1, Mc)), rng.uniform(1, 100, (t - 1, Mc)), np.zeros((t - 1, Mc)))
    E0 = E[:Vr]

    def step():
        U, Y, Z = oracle.mlp.shard_forward(X, A0, B0)
        oracle.mlp.partial_sum([Z] + [other] * (t - 1))
        g = oracle.mlp.shard_backward(X, A0, B0, U, dZ)
        oracle.mlp.partial_sum([g["dX"]] + [other] * (t - 1))
        m, l, T, _ = oracle.xent.shard_partials(H, E0, y, 0)
        oracle.xent.merge(np.vstack([m[None], st[0]]), np.vstack([l[None], st[1]]), np.vstack([T[None], st[2]]))
        return U

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return time.perf_counter() - t0, r

    mf = mlp_flops(M, h, f)
    step_fl = mf["fwd"] + mf["bwd"] + xent_flops(Mc, hc, Vr)
    total, passes = 0.0, 0
    while passes == 0 or total < reps_budget_s:
        dt, U = timed(step)
        total += dt
        passes += 1
    per = {}
    X2, A2, B2 = host["X2"], host["A2_0"], host["B2_0"]
    fl2 = mlp_flops(X2.shape[0], X2.shape[1], A2.shape[1])["fwd"]
    for name, fn, fl in (
            ("mlp_8p3b_fwd", lambda: oracle.mlp.shard_forward(X2, A2, B2), fl2),
            ("mlp_70b_fwd", lambda: oracle.mlp.shard_forward(X, A0, B0), mf["fwd"]),
            ("mlp_70b_bwd", lambda: oracle.mlp.shard_backward(X, A0, B0, U, dZ), mf["bwd"]),
            ("xent_8p3b_slice", lambda: oracle.xent.shard_partials(H, E0, y, 0), xent_flops(Mc, hc, Vr)),
            ("xent_8p3b_full_vocab", lambda: oracle.xent.naive_loss(H, E, y), xent_flops(Mc, hc, E.shape[0]))):
        dt, _ = timed(fn)
        per[name] = {"s": round(dt, 3), "gflop": round(fl / 1e9, 1), "tflops": round(fl / dt / 1e12, 4)}
        if name.startswith("xent"):
            per[name]["tokens_per_s"] = round(Mc / dt, 1)
    per["xent_8p3b_full_vocab"]["note"] = ("naive full-logit CE of all 8192 tokens over the whole "
                                           "51,200-entry vocabulary (2.58 TFLOP), timed apart from slice 0")
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": round(step_fl * passes / total / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": threads,
            "sample": f"the whole step (all {M} tokens of the 70B MLP forward + backward with both sums of "
                      f"8 partials, all {Mc} tokens of CE slice 0 and the merge) in fp64 numpy, {passes} "
                      f"pass(es): {step_fl * passes / 1e9:.0f} GFLOP in {total:.2f} s",
            "per_config": per}


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


def n_sets(bytes_per_set):
    """Input sets to rotate so that together they exceed twice the Infinity Cache."""
    return max(3, -(-2 * INFINITY_CACHE_BYTES // bytes_per_set))


def settle(torch, fn, seconds=0.5):
    """Run fn(i) until `seconds` of wall time have passed.  The part's clocks
    take several milliseconds of sustained load to settle: right after light
    work, the first few hundred calls of the 8.3B forward drifted from 184 down
    to 164 us, where the same calls later took 150-152 us.  Timing starts only
    after this."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def per_config(torch, lgs, reps):
    """Every configuration the library is specified on, each timed alone, call
    by call (half a second of the first matrix-core workload to settle the
    clocks; then per configuration 10 warm-up calls and `reps` timed calls;
    median and minimum), with
    enough input sets rotated between calls to exceed twice the Infinity
    Cache.  Inputs are device draws with the workloads' distributions (the
    kernels' cost does not depend on the values)."""
    from logit_gemm_shard_amd import synth
    from logit_gemm_shard_amd.configs import WORKLOADS
    dev = torch.device("cuda", 0)
    bf = torch.bfloat16
    out = {}

    def randn(*shape, std=1.0, dtype=bf):
        x = torch.randn(*shape, device=dev)
        if std != 1.0:
            x.mul_(std)
        return x.to(dtype)

    # tiny fp32 block: both shards' forward + sum, replayed as one HIP graph
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
    del X, A, B, Z, Zs, Ys, shards, graph

    # MLP shard forward and backward at the 8.3B and 70B shapes
    for fwd_name, bwd_name in (("mlp_8p3b_fwd", "mlp_8p3b_bwd"), ("mlp_70b_fwd", "mlp_70b_bwd")):
        w = WORKLOADS[fwd_name]
        f = w.f_i
        per_set = 2 * (2 * w.M * w.h + 2 * w.h * f)
        sets = [(randn(w.M, w.h), randn(w.h, f, std=0.02), randn(f, w.h, std=synth.residual_std(w.n_blocks)),
                 randn(w.M, w.h, std=0.01)) for _ in range(n_sets(per_set))]
        U = torch.empty(w.M, f, dtype=bf, device=dev)
        Y = torch.empty(w.M, f, dtype=bf, device=dev)
        Z = torch.empty(w.M, w.h, dtype=bf, device=dev)

        def fwd(i, w=w, sets=sets, U=U, Y=Y, Z=Z):
            X, A0, B0, _ = sets[i % len(sets)]
            lgs.tp_mlp_fwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, A0, B0, Z, U_i=U, Y_i=Y)
        if fwd_name == "mlp_8p3b_fwd":  # the first matrix-core workload after the launch-bound one
            settle(torch, fwd)
        fl = mlp_flops(w.M, w.h, f)
        out[fwd_name] = _timed_report(torch, fwd, fl["fwd"], reps, len(sets))
        if bwd_name:
            wb = WORKLOADS.get(bwd_name, w)  # the 8.3B backward: the forward's shapes, dZ ~ N(0, 0.01)
            dX = torch.empty(w.M, w.h, dtype=bf, device=dev)
            dA = torch.empty(w.h, f, dtype=bf, device=dev)
            dB = torch.empty(f, w.h, dtype=bf, device=dev)
            ws = torch.empty(lgs.mlp_bwd_workspace_bytes(wb.b, wb.s, wb.h, wb.ffn, wb.t, bf), dtype=torch.uint8,
                             device=dev)

            def bwd(i, w=wb, sets=sets, U=U, dX=dX, dA=dA, dB=dB, ws=ws):
                X, A0, B0, dZ = sets[i % len(sets)]
                lgs.tp_mlp_bwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, A0, B0, U, dZ, dX, dA, dB, workspace=ws)
            out[bwd_name] = _timed_report(torch, bwd, fl["bwd"], reps, len(sets))
            del dX, dA, dB, ws
        del sets, U, Y, Z

    # the fused CE forward and backward of vocabulary slice 0 at the 8.3B shapes
    xw = WORKLOADS["xent_8p3b"]
    M, h, V, t, Vr = xw.M, xw.h, xw.vocab, xw.t, xw.v_r
    sets = [(randn(M, h), randn(Vr, h, std=0.02), torch.randint(0, V, (M,), device=dev, dtype=torch.int32))
            for _ in range(n_sets(2 * (M * h + Vr * h)))]
    stats = torch.empty(3, M, device=dev)
    ws_x = torch.empty(lgs.xent_workspace_bytes(xw.b, xw.s, h, V, t), dtype=torch.uint8, device=dev)

    def xfwd(i):
        H, E0, y = sets[i % len(sets)]
        lgs.vocab_parallel_xent_fwd(xw.b, xw.s, h, V, t, 0, H, E0, y, stats[0], stats[1], stats[2], workspace=ws_x)
    rep = _timed_report(torch, xfwd, xent_flops(M, h, Vr), reps, len(sets))
    rep["tokens_per_s"] = round(M / (rep["ms"] * 1e-3), 0)
    out["xent_8p3b"] = rep
    progress("xent_8p3b timed")
    lse = (torch.randn(M, device=dev).abs_() + 12.0)
    dl = torch.full((M,), 1.0 / M, dtype=torch.float32, device=dev)
    dH0 = torch.empty(M, h, dtype=bf, device=dev)
    dE0 = torch.empty(Vr, h, dtype=bf, device=dev)
    ws_xb = torch.empty(lgs.xent_bwd_workspace_bytes(xw.b, xw.s, h, V, t), dtype=torch.uint8, device=dev)

    def xbwd(i):
        H, E0, y = sets[i % len(sets)]
        lgs.vocab_parallel_xent_bwd(xw.b, xw.s, h, V, t, 0, H, E0, y, lse, dH0, dE0, dloss=dl, workspace=ws_xb)
    rep = _timed_report(torch, xbwd, 3 * xent_flops(M, h, Vr), reps, len(sets))
    rep["tokens_per_s"] = round(M / (rep["ms"] * 1e-3), 0)
    rep["note"] += "; dloss = 1/M: the recomputed logit GEMM with its gradient epilogue, then dH_0 and dE_0"
    out["xent_8p3b_bwd"] = rep
    progress("xent_8p3b_bwd timed")
    del sets, stats, ws_x, lse, dl, dH0, dE0, ws_xb

    # SwiGLU block (the gated MLP of the same 70B model): forward = the paired
    # [gate | up] GEMM (2 M h 2f) + the down GEMM (2 M f h); backward = dY, dX,
    # dW_gu, dW_down, (2 + 4 + 4 + 2) M h f
    w = WORKLOADS["swiglu_70b_fwd"]
    f = w.f_i
    sets = [(randn(w.M, w.h), randn(w.h, 2 * f, std=0.02), randn(f, w.h, std=synth.residual_std(w.n_blocks)),
             randn(w.M, w.h, std=0.01)) for _ in range(n_sets(2 * (2 * w.M * w.h + 3 * w.h * f)))]
    GU = torch.empty(w.M, 2 * f, dtype=bf, device=dev)
    Y = torch.empty(w.M, f, dtype=bf, device=dev)
    Z = torch.empty(w.M, w.h, dtype=bf, device=dev)

    def sfwd(i):
        X, Wgu, Wd, _ = sets[i % len(sets)]
        lgs.tp_swiglu_fwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, Wgu, Wd, Z, GU_i=GU, Y_i=Y)
    out["swiglu_70b_fwd"] = _timed_report(torch, sfwd, 6 * w.M * w.h * f, reps, len(sets))
    wb = WORKLOADS["swiglu_70b_bwd"]
    dX = torch.empty(w.M, w.h, dtype=bf, device=dev)
    dWgu = torch.empty(w.h, 2 * f, dtype=bf, device=dev)
    dWd = torch.empty(f, w.h, dtype=bf, device=dev)
    ws = torch.empty(lgs.swiglu_bwd_workspace_bytes(wb.b, wb.s, wb.h, wb.ffn, wb.t, bf), dtype=torch.uint8,
                     device=dev)

    def sbwd(i):
        X, Wgu, Wd, dZ = sets[i % len(sets)]
        lgs.tp_swiglu_bwd(wb.b, wb.s, wb.h, wb.ffn, wb.t, 0, X, Wgu, Wd, GU, dZ, dX, dWgu, dWd, workspace=ws)
    out["swiglu_70b_bwd"] = _timed_report(torch, sbwd, 12 * w.M * w.h * f, reps, len(sets))
    progress("swiglu_70b_bwd timed")
    del sets, GU, Y, Z, dX, dWgu, dWd, ws

    # attention projections of one rank (8 query heads, 1 KV head of 128):
    # forward = QKV (2 M h (q + 2 kv)) + W_O (2 M q h); backward twice that
    w = WORKLOADS["attn_70b"]
    q, kv = w.n_heads // w.t * w.head_dim, w.n_kv_heads // w.t * w.head_dim
    nqkv = q + 2 * kv
    per_set = 2 * (w.M * w.h * 2 + w.h * nqkv + q * w.h + w.M * q + w.M * nqkv)
    sets = [(randn(w.M, w.h), randn(w.h, nqkv, std=0.02), randn(q, w.h, std=synth.residual_std(w.n_blocks)),
             randn(w.M, q), randn(w.M, w.h, std=w.dz_std), randn(w.M, nqkv, std=w.dz_std))
            for _ in range(n_sets(per_set))]
    QKV = torch.empty(w.M, nqkv, dtype=bf, device=dev)
    Z = torch.empty(w.M, w.h, dtype=bf, device=dev)
    dX = torch.empty(w.M, w.h, dtype=bf, device=dev)
    dW = torch.empty(w.h, nqkv, dtype=bf, device=dev)
    dA = torch.empty(w.M, q, dtype=bf, device=dev)
    dWo = torch.empty(q, w.h, dtype=bf, device=dev)
    a = (w.b, w.s, w.h)
    ws_qkv = torch.empty(max(1, lgs.attn_qkv_fwd_workspace_bytes(*a, w.n_heads, w.n_kv_heads, w.head_dim, w.t)),
                         dtype=torch.uint8, device=dev)
    ws_ob = torch.empty(max(1, lgs.attn_out_bwd_workspace_bytes(*a, w.n_heads, w.head_dim, w.t)),
                        dtype=torch.uint8, device=dev)

    def afwd(i):
        X, Wqkv, Wo, A, _, _ = sets[i % len(sets)]
        lgs.tp_attn_qkv_fwd(*a, w.n_heads, w.n_kv_heads, w.head_dim, w.t, 0, X, Wqkv, QKV, workspace=ws_qkv)
        lgs.tp_attn_out_fwd(*a, w.n_heads, w.head_dim, w.t, 0, A, Wo, Z)

    def abwd(i):
        X, Wqkv, Wo, A, dZ, dQ = sets[i % len(sets)]
        lgs.tp_attn_qkv_bwd(*a, w.n_heads, w.n_kv_heads, w.head_dim, w.t, 0, X, Wqkv, dQ, dX, dW)
        lgs.tp_attn_out_bwd(*a, w.n_heads, w.head_dim, w.t, 0, A, Wo, dZ, dA, dWo, workspace=ws_ob)
    fl = 2 * w.M * w.h * (nqkv + q)
    out["attn_70b_fwd"] = _timed_report(torch, afwd, fl, reps, len(sets))
    out["attn_70b_bwd"] = _timed_report(torch, abwd, 2 * fl, reps, len(sets))
    progress("attn_70b_bwd timed")
    del sets, QKV, Z, dX, dW, dA, dWo, ws_qkv, ws_ob

    # the exchanges' one-device stand-ins (pure HBM streams): the sum of 8
    # partials at both shapes, and the sequence-parallel reduce-scatter and
    # all-gather at the 8.3B shape (s = 1024, b = 8, h = 3072, t = 8)
    for name, (M, h) in (("sum_partials_8p3b", (8192, 3072)), ("sum_partials_70b", (4096, 8192))):
        parts = randn(8, M, h, std=0.05)
        zs = torch.empty(M, h, dtype=bf, device=dev)
        ms = time_calls(torch, lambda: lgs.shard_partial_sum("sum", 8, M * h, parts, M * h, zs), reps)
        nb = 9 * M * h * 2
        out[name] = {"us": round(ms * 1e3, 2), "bytes": nb, "GBs": round(nb / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "note": "8 partials read once, the sum written once; one buffer (more than twice the "
                             "Infinity Cache)"}
        del parts, zs
    w = WORKLOADS["mlp_8p3b_fwd"]
    t, M, h = w.t, w.M, w.h
    chunk = M * h // t
    # successive calls take successive ranks' chunks (and rotate the gather's
    # inputs), so no call finds its bytes in the Infinity Cache
    parts = randn(t, M, h, std=0.05)
    rs_out = torch.empty(M // t, h, dtype=bf, device=dev)
    ag_in = [randn(t, M // t, h) for _ in range(6)]
    ag_out = torch.empty(M, h, dtype=bf, device=dev)
    res = randn(t, M // t, h)
    keep = (torch.rand(t, M // t, h, device=dev) > 0.1).to(torch.uint8)
    gamma, beta = randn(h, std=0.1) + 1, randn(h, std=0.1)
    hs, ys = torch.empty(M // t, h, dtype=bf, device=dev), torch.empty(M // t, h, dtype=bf, device=dev)
    i = [0]

    def rs():
        lgs.shard_reduce_scatter(t, i[0] % t, w.s, w.b, h, parts, M * h, rs_out)
        i[0] += 1

    def ag():
        lgs.shard_all_gather(t, w.s, w.b, h, ag_in[i[0] % 6], chunk, ag_out)
        i[0] += 1

    def rs_ln():
        r = i[0] % t
        lgs.shard_reduce_scatter_layernorm(t, r, w.s, w.b, h, parts, M * h, res[r], gamma, beta, hs, ys,
                                           keep=keep[r], keep_scale=1 / 0.9)
        i[0] += 1
    dys, dhss = randn(t, M // t, h), randn(t, M // t, h)
    gg, dzz = torch.empty(M // t, h, dtype=bf, device=dev), torch.empty(M // t, h, dtype=bf, device=dev)
    dgam, dbet = torch.empty(h, device=dev), torch.empty(h, device=dev)
    lws = torch.empty(lgs.layernorm_bwd_workspace_bytes(t, w.s, w.b, h), dtype=torch.uint8, device=dev)

    def ln_bwd():
        r = i[0] % t
        lgs.shard_layernorm_bwd(t, r, w.s, w.b, h, res[r], dys[r], gamma, gg, dzz, dgam, dbet, dhs=dhss[r],
                                keep=keep[r], keep_scale=1 / 0.9, workspace=lws)
        i[0] += 1
    rs_ms = time_calls(torch, rs, reps)
    ag_ms = time_calls(torch, ag, reps)
    ln_ms = time_calls(torch, rs_ln, reps)
    lb_ms = time_calls(torch, ln_bwd, reps)
    lb_bytes = 3 * chunk * 2 + chunk + 2 * chunk * 2 + h * 2 + 2 * h * 4
    rs_bytes, ag_bytes = (t + 1) * chunk * 2, 2 * M * h * 2
    ln_bytes = (t + 1) * chunk * 2 + chunk + 2 * chunk * 2 + 2 * h * 2
    out["sp_8p3b"] = {"reduce_scatter_us": round(rs_ms * 1e3, 2),
                      "reduce_scatter_GBs": round(rs_bytes / (rs_ms * 1e-3) / 1e9, 1),
                      "all_gather_us": round(ag_ms * 1e3, 2),
                      "all_gather_GBs": round(ag_bytes / (ag_ms * 1e-3) / 1e9, 1),
                      "rs_layernorm_us": round(ln_ms * 1e3, 2),
                      "rs_layernorm_GBs": round(ln_bytes / (ln_ms * 1e-3) / 1e9, 1),
                      "rs_layernorm_frac_hbm": round(ln_bytes / (ln_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "layernorm_bwd_us": round(lb_ms * 1e3, 2),
                      "layernorm_bwd_GBs": round(lb_bytes / (lb_ms * 1e-3) / 1e9, 1),
                      "note": "bytes = every byte read once + written once; HBM peak 8000 GB/s; "
                              "rs_layernorm: the 8 partials' rank rows, residual, keep mask read, hs and y "
                              "written (dropout p = 0.1); layernorm_bwd: hs, dy, dhs, mask read, g and dz "
                              "written (the fp32 column partials not counted)"}
    return out


MFMA_COUNTERS_FILE = os.path.join(ROOT, "profiles", "mfma_lds_counters_8p3b_step.md")
MFMA_PASSES = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES",
               "SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA SQ_WAVES")
# kernels of the 8.3B workload: (row label, algorithmic GFLOP, name patterns (mangled, demangled))
MFMA_KERNELS = (
    ("fwd GEMM1 + GeLU (256x192, 256 tiles)", 77.309, ("Li256ELi192ELb1ELb0ENS_10EpiGeluFwd", "256, 192, true, false, lgs::EpiGeluFwd")),
    ("fwd GEMM2 (256x192, 512 tiles)", 77.309, ("Li256ELi192ELb1ELb0ENS_8EpiStore", "256, 192, true, false, lgs::EpiStore")),
    ("dY + GeLU' (256x192, 256 tiles)", 77.309, ("Li256ELi192ELb1ELb1ENS_10EpiGeluBwd", "256, 192, true, true, lgs::EpiGeluBwd")),
    ("group3 dB, dA, dX (256x256, 528 tiles)", 231.928, ("gemm_pp_group3_kernel",)),
    ("CE logit GEMM + slabs, columns 0-2559 (256x320, 256 tiles)", 128.849,
     ("Li256ELi320ELb1ELb1ENS_7EpiXent", "256, 320, true, true, lgs::EpiXent")),
    ("CE logit GEMM + slabs, columns 2560-6399 (256x256, 480 tiles)", 193.274,
     ("Li256ELi256ELb1ELb1ENS_7EpiXent", "256, 256, true, true, lgs::EpiXent")),
)


def mfma_workload(torch, lgs, calls=5):
    """The 8.3B-shape kernels alone, for counter passes: rank 0's MLP forward
    and backward and the fused CE of slice 0, `calls` times each on three
    rotated input sets."""
    from logit_gemm_shard_amd import synth
    from logit_gemm_shard_amd.configs import WORKLOADS
    dev, bf = torch.device("cuda", 0), torch.bfloat16
    w, xw = WORKLOADS["mlp_8p3b_fwd"], WORKLOADS["xent_8p3b"]
    f = w.f_i

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, device=dev) * std).to(bf)
    sets = [(randn(w.M, w.h), randn(w.h, f, std=0.02), randn(f, w.h, std=synth.residual_std(w.n_blocks)),
             randn(w.M, w.h, std=0.01), randn(xw.M, xw.h), randn(xw.v_r, xw.h, std=0.02),
             torch.randint(0, xw.vocab, (xw.M,), device=dev, dtype=torch.int32)) for _ in range(3)]
    U, Y = torch.empty(w.M, f, dtype=bf, device=dev), torch.empty(w.M, f, dtype=bf, device=dev)
    Z, dX = torch.empty(w.M, w.h, dtype=bf, device=dev), torch.empty(w.M, w.h, dtype=bf, device=dev)
    dA, dB = torch.empty(w.h, f, dtype=bf, device=dev), torch.empty(f, w.h, dtype=bf, device=dev)
    ws = torch.empty(lgs.mlp_bwd_workspace_bytes(w.b, w.s, w.h, w.ffn, w.t, bf), dtype=torch.uint8, device=dev)
    wx = torch.empty(lgs.xent_workspace_bytes(xw.b, xw.s, xw.h, xw.vocab, xw.t), dtype=torch.uint8, device=dev)
    st = torch.empty(3, xw.M, device=dev)
    for i in range(calls):
        X, A0, B0, dZ, H, E0, y = sets[i % 3]
        lgs.tp_mlp_fwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, A0, B0, Z, U_i=U, Y_i=Y)
        lgs.tp_mlp_bwd(w.b, w.s, w.h, w.ffn, w.t, 0, X, A0, B0, U, dZ, dX, dA, dB, workspace=ws)
        lgs.vocab_parallel_xent_fwd(xw.b, xw.s, xw.h, xw.vocab, xw.t, 0, H, E0, y, st[0], st[1], st[2], workspace=wx)
    torch.cuda.synchronize()


def mfma_summary(d):
    """Write MFMA_COUNTERS_FILE from two rocprofv3 --pmc passes (MFMA_PASSES)
    over `bench.py --mfma-workload` under d/pmc_mfma_A and d/pmc_mfma_B."""
    import collections
    import csv
    import statistics
    cnt, dur, names = collections.defaultdict(list), collections.defaultdict(list), {}
    for sub in ("pmc_mfma_A", "pmc_mfma_B"):
        found = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not found:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(d, sub)}")
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        span = {}
        for r in csv.DictReader(open(found[0])):
            label = next((k[0] for k in MFMA_KERNELS if any(pat in r["Kernel_Name"] for pat in k[2])), None)
            if label is None:
                continue
            per[(label, r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
            span[(label, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        for (label, _), c in per.items():
            for k, v in c.items():
                cnt[(label, k)].append(v)
        for (label, _), v in span.items():
            dur[label].append(v)
    med = {k: statistics.median(v) for k, v in cnt.items()}
    rows1, rows2 = [], []
    for label, alg, _ in MFMA_KERNELS:
        if (label, "SQ_WAVES") not in med:
            raise SystemExit(f"no counters for {label}")
        us = statistics.median(dur[label])
        busy = med[(label, "SQ_VALU_MFMA_BUSY_CYCLES")] / 1024
        active = med[(label, "GRBM_GUI_ACTIVE")] / 8
        gflop = med[(label, "SQ_INSTS_VALU_MFMA_MOPS_BF16")] * 512 / 1e9
        waves = med[(label, "SQ_WAVES")]
        rows1.append(f"| {label} | {us:.1f} | {gflop:.3f} | {alg:.3f} | {busy / 1e3:.1f} k | {active / 1e3:.1f} k | "
                     f"{100 * busy / active:.1f}% | {active / us / 1e3:.2f} GHz |")
        rows2.append(f"| {label} | {waves:.0f} | {med[(label, 'SQ_INSTS_VALU')] / waves:.0f} | "
                     f"{med[(label, 'SQ_INSTS_MFMA')] / waves:.0f} | {med[(label, 'SQ_INSTS_LDS')] / waves:.0f} | "
                     f"{med[(label, 'SQ_LDS_BANK_CONFLICT')] / 256:.0f} |")
    cmd = "python bench.py --mfma-workload"
    txt = f"""# MFMA and LDS counters per kernel: the 8.3B-shape kernels (rank 0 of t=8)

The MLP forward and backward and the fused CE of slice 0, five calls each on three rotated input
sets (`bench.py --mfma-workload`), under two counter passes, one counter set per run:

```
rocprofv3 --pmc {MFMA_PASSES[0]} --output-format csv -d rocprof_out/pmc/pmc_mfma_A -o p -- {cmd}
rocprofv3 --pmc {MFMA_PASSES[1]} --output-format csv -d rocprof_out/pmc/pmc_mfma_B -o p -- {cmd}
python bench.py --mfma-summary rocprof_out/pmc      (writes this file)
```

Medians over the launches of each kernel. Counter values are summed over the 8 XCDs. Durations
are the dispatch timestamps of the same runs, which the counter runs serialise and slow by a
few percent.

| Kernel | µs | MFMA GFLOP (MOPs × 512) | algorithmic GFLOP | MFMA busy cycles / SIMD | active cycles / XCD | MFMA util | implied clock |
|---|---|---|---|---|---|---|---|
{chr(10).join(rows1)}

- MFMA util is rocprof's `MfmaUtil`: MFMA busy cycles summed over the 1024 SIMDs ÷
  (active cycles × 1024): the matrix cores' duty cycle at the clock the kernel actually ran
  at, independent of the 2.4 GHz figure behind the spec peak.
- The implied clock is active cycles ÷ duration; for kernels of under 100 µs the active
  count includes some time outside the dispatch window, which biases their utilisation low.

| Kernel | waves | VALU instr / wave | MFMA instr / wave | LDS instr / wave | LDS bank-conflict cycles / CU |
|---|---|---|---|---|---|
{chr(10).join(rows2)}

kernel_sources_sha256: {kernel_sources_digest()}
"""
    open(MFMA_COUNTERS_FILE, "w").write(txt)
    print(txt)


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


XR_COUNTERS_FILE = os.path.join(ROOT, "profiles", "xent_rows_8p3b_hbm_counters.txt")


def ce_stream_workload(torch, lgs):
    """The streaming CE reductions alone (the same 3 warm-up and 30 timed
    calls as the bench line), for the counter and trace passes."""
    from logit_gemm_shard_amd.configs import WORKLOADS
    r = ce_reduction_stream(torch, lgs, WORKLOADS["xent_8p3b"])
    torch.cuda.synchronize()
    print(json.dumps(r), flush=True)


def ce_stream_summary(d):
    """Write XR_COUNTERS_FILE: the streaming CE reduction kernel's HBM-side
    bytes per launch from FETCH_SIZE / WRITE_SIZE passes (scaled by the copy
    calibration passes of the counter summary) and its average duration from
    a kernel trace, all over `bench.py --ce-stream-workload`."""
    import csv
    import statistics

    def one(sub, pattern):
        found = glob.glob(os.path.join(d, sub, "**", pattern), recursive=True)
        if not found:
            raise SystemExit(f"no {pattern} under {os.path.join(d, sub)}")
        return found[0]
    med = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        xr = [v for n, v in _per_kernel(one(f"pmc/pmc_xr_{c}", "*counter_collection.csv"), c).items()
              if "xent_rows_kernel" in n]
        cp = [v for n, v in _per_kernel(one(f"pmc/pmc_copy_{c}", "*counter_collection.csv"), c).items()
              if "neg" in n]
        if len(xr) != 1 or len(cp) != 1:
            raise SystemExit(f"{c}: expected one streaming CE kernel and one copy kernel")
        med[c] = (statistics.median(xr[0]), len(xr[0]), statistics.median(cp[0]))
    fr = (1 << 30) / (med["FETCH_SIZE"][2] * 1024)
    fw = (1 << 30) / (med["WRITE_SIZE"][2] * 1024)
    rd, wr = med["FETCH_SIZE"][0] * 1024 * fr, med["WRITE_SIZE"][0] * 1024 * fw
    rows = [r for r in csv.DictReader(open(one("prof_xr", "*kernel_stats.csv"))) if "xent_rows_kernel" in r["Name"]]
    if len(rows) != 1:
        raise SystemExit("expected one streaming CE kernel in the kernel trace")
    us, calls = float(rows[0]["AverageNs"]) / 1e3, int(rows[0]["Calls"])
    M, Vr = 8192, 6400
    alg = M * Vr * 2 + M * 4 + 3 * M * 4
    wl = "python bench.py --ce-stream-workload"
    txt = f"""# HBM-side traffic and time of the streaming CE reductions (xent_rows_kernel:
# per-row max, sum of exponentials and target logit over materialised bf16
# logits of the 8.3B slice, [{M}, {Vr}]; three 105 MB buffers rotated, more than
# the 256 MB Infinity Cache), from rocprofv3 passes over the same workload:
#
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc/pmc_xr_FETCH_SIZE -o p -- {wl}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc/pmc_xr_WRITE_SIZE -o p -- {wl}
#   rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/prof_xr -o x -- {wl}
#   (the copy-calibration passes of the MLP counter summary, under rocprof_out/pmc/pmc_copy_*)
#   python bench.py --ce-stream-summary rocprof_out      (writes this file)
#
# Per launch (median over {med['FETCH_SIZE'][1]} dispatches; FETCH_SIZE x 1024 x {fr:.4f}, WRITE_SIZE x 1024 x {fw:.4f}):
#   read  {rd / 1e6:.1f} MB, written {wr / 1e6:.3f} MB (FETCH_SIZE {med['FETCH_SIZE'][0]:.0f} KiB, WRITE_SIZE {med['WRITE_SIZE'][0]:.0f} KiB)
#   algorithmic bytes: {alg / 1e6:.1f} MB (every logit read once, the targets read, m, l, T written)
#   average duration under the kernel trace: {us:.2f} us over {calls} launches
#   achieved: {(rd + wr) / us / 1e3:.1f} GB/s by the counters, {alg / us / 1e3:.1f} GB/s algorithmic
#   ({alg / us / 1e3 / PEAK_HBM_GBS:.3f} of the 8000 GB/s HBM peak)
kernel_sources_sha256: {kernel_sources_digest()}
"""
    open(XR_COUNTERS_FILE, "w").write(txt)
    print(txt)


MFMA_RATE_CASES = (  # (label, blocks, waves per block, operands)
    ("256 CUs, 2 waves per SIMD, N(0,1) x N(0,1)", 256, 8, "normal"),
    ("256 CUs, 1 wave per SIMD, N(0,1) x N(0,1)", 256, 4, "normal"),
    ("256 CUs, 2 waves per SIMD, N(0,1) x N(0,0.02) (activations x weights)", 256, 8, "weights"),
    ("256 CUs, 2 waves per SIMD, zero operands", 256, 8, "zeros"),
    ("128 CUs, 2 waves per SIMD, N(0,1) x N(0,1)", 128, 8, "normal"),
    ("64 CUs, 2 waves per SIMD, N(0,1) x N(0,1)", 64, 8, "normal"),
)


def mfma_rate_case(torch, lgs, blocks, waves, ops, iters8, reps):
    """One probe configuration: best of `reps` launches (HIP events) and the
    waves' median shader clock over their MFMA loops."""
    dev = ops.device
    out = torch.empty(blocks * waves * 8192, device=dev)
    clocks = torch.empty(2 * blocks * waves, dtype=torch.int64, device=dev)
    lgs.mfma_rate(blocks, waves, iters8 // 10, ops, out, clocks)  # warm-up
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lgs.mfma_rate(blocks, waves, iters8, ops, out, clocks)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if best is None or ms < best[0]:
            ck = clocks.cpu().view(-1, 2).double()
            best = (ms, float((ck[:, 0] / ck[:, 1]).median()) * 100.0)
    tf = blocks * waves * iters8 * 64 * 32768 / (best[0] * 1e-3) / 1e12
    return {"blocks": blocks, "waves_per_block": waves, "ms": round(best[0], 3), "tflops": round(tf, 1),
            "frac_spec_peak": round(tf / PEAK_BF16_TFLOPS, 4), "tflops_per_cu": round(tf / blocks, 3),
            "clock_mhz": round(best[1], 0)}


def mfma_rate(torch, lgs, out_path, iters8=20000, reps=3):
    """The matrix cores' bf16 rate with nothing but MFMAs to run
    (lgs_test_mfma_rate): per case, the best of `reps` launches timed with HIP
    events, and the shader clock the waves measured over their MFMA loops
    (s_memtime cycles / s_memrealtime ticks at 100 MHz, median over waves).
    Writes a markdown summary to out_path and prints it as one JSON line."""
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(11)

    def ops_of(kind):
        x = torch.randn(16, 64, 8, device=dev, generator=g)
        if kind == "weights":
            x[1::2] *= 0.02  # the B operands (pairs 2k + 1)
        elif kind == "zeros":
            x.zero_()
        return x.to(torch.bfloat16)
    rows = []
    for label, blocks, waves, kind in MFMA_RATE_CASES:
        row = mfma_rate_case(torch, lgs, blocks, waves, ops_of(kind), iters8, reps)
        rows.append({"case": label, **row})
        progress(f"mfma rate: {label}: {row['tflops']:.1f} TFLOP/s at {row['clock_mhz']:.0f} MHz")
    lines = ["# Matrix-core bf16 rate with nothing but MFMAs to run (lgs_test_mfma_rate)", "",
             "Command (from the repository root):", "", "```", f"python bench.py --mfma-rate {out_path}", "```", "",
             f"Each wave runs 8 independent accumulator chains of v_mfma_f32_32x32x16_bf16 on operands held in "
             f"registers (8 operand pairs rotating between consecutive instructions), {iters8 * 64} MFMAs per "
             f"wave; one block per compute unit. Best of {reps} launches (HIP events). The clock is the shader "
             "clock the waves counted over their MFMA loops (s_memtime cycles over s_memrealtime ticks of "
             "100 MHz, median over the waves). Spec peak: 2516.6 TFLOP/s (256 CUs at 2.4 GHz).", "",
             "| case | ms | TFLOP/s | of spec peak | TFLOP/s per busy CU | clock MHz |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['case']} | {r['ms']} | {r['tflops']} | {100 * r['frac_spec_peak']:.1f}% | "
                     f"{r['tflops_per_cu']} | {r['clock_mhz']:.0f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"mfma_rate": rows}), flush=True)


def progress(msg):
    """One line on stderr as each part of the run finishes (the JSON line on
    stdout stays the only output there)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _timed_report(torch, fn, flops, reps, nsets, warmup=10):
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
            "note": f"median of per-call times, {nsets} input sets rotated"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--ce-stream-workload", action="store_true",
                    help="run the streaming CE reductions alone (for counter and trace passes) and exit")
    ap.add_argument("--ce-stream-summary", metavar="DIR",
                    help="write the streaming CE counter summary from rocprofv3 passes under DIR and exit")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the graphics clock while the step repeats (profiler runs)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-configuration timings (counter passes)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="time torch.matmul (hipBLASLt) at the library's GEMM shapes and exit")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="write the tp_mlp_bwd traffic summary from rocprofv3 --pmc passes under DIR and exit")
    ap.add_argument("--mfma-workload", action="store_true",
                    help="run the 8.3B-shape kernels alone (for counter passes) and exit")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="write the MFMA / LDS counter summary from the passes under DIR and exit")
    ap.add_argument("--stream-workload", action="store_true",
                    help="run the HBM-bound kernels alone (for counter passes) and exit")
    ap.add_argument("--stream-summary", metavar="DIR",
                    help="write the HBM-bound kernels' counter summary from the passes under DIR and exit")
    ap.add_argument("--mfma-rate", metavar="OUT",
                    help="measure the matrix cores' rate with nothing but MFMAs to run, write a summary to OUT "
                         "and exit")
    ap.add_argument("--kernel-stats", nargs=3, metavar=("CSV", "TITLE", "COMMAND"),
                    help="print a markdown table of a rocprofv3 kernel_stats.csv and exit")
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.kernel_stats:
        kernel_stats_md(*args.kernel_stats)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.ce_stream_summary:
        ce_stream_summary(args.ce_stream_summary)
        return
    if args.stream_summary:
        stream_summary(args.stream_summary)
        return
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
    if args.mfma_workload:
        from logit_gemm_shard_amd import binding as lgs_b
        mfma_workload(torch, lgs_b)
        return
    if args.ce_stream_workload:
        from logit_gemm_shard_amd import binding as lgs_b
        ce_stream_workload(torch, lgs_b)
        return
    if args.stream_workload:
        from logit_gemm_shard_amd import binding as lgs_b
        stream_workload(torch, lgs_b)
        return
    if args.mfma_rate:
        from logit_gemm_shard_amd import binding as lgs_b
        mfma_rate(torch, lgs_b, args.mfma_rate)
        return

    from logit_gemm_shard_amd import binding as lgs
    from logit_gemm_shard_amd import synth
    from logit_gemm_shard_amd.configs import WORKLOADS

    w, wb, xw = WORKLOADS["mlp_70b_fwd"], WORKLOADS["mlp_70b_bwd"], WORKLOADS["xent_8p3b"]
    M, h, f, t, ffn = w.M, w.h, w.f_i, w.t, w.ffn
    Mc, hc, V, Vr = xw.M, xw.h, xw.vocab, xw.v_r
    bf = torch.bfloat16
    dev = torch.device("cuda", 0)

    # ---------------- inputs -> HBM.  Set 0: the workloads' seeded host draws
    # (X, A, B from the 70B seed, dZ from its own, H, E, targets from the CE
    # seed), rank 0's slices; sets 1 and 2: device draws with the same
    # distributions.
    X, A, B = synth.mlp_weights(w)
    A0, B0 = A[:, :f].contiguous(), B[:f].contiguous()
    del A, B
    dZ = synth.mlp_grad(wb)
    H, E, y = synth.xent_inputs(xw)
    E0 = E[:Vr].contiguous()
    g = torch.Generator(device=dev)
    g.manual_seed(12345)

    def draw(*shape, std=1.0):
        return (torch.randn(*shape, device=dev, generator=g) * std).to(bf)
    sets = [(X.to(dev), A0.to(dev), B0.to(dev), dZ.to(dev), H.to(dev), E0.to(dev), y.to(dev))]
    for _ in range(2):
        sets.append((draw(M, h), draw(h, f, std=0.02), draw(f, h, std=synth.residual_std(w.n_blocks)),
                     draw(M, h, std=wb.dz_std), draw(Mc, hc), draw(Vr, hc, std=0.02),
                     torch.randint(0, V, (Mc,), device=dev, dtype=torch.int32, generator=g)))
    set_bytes = sum(x.numel() * x.element_size() for x in sets[0])
    U = [torch.empty(M, f, dtype=bf, device=dev) for _ in sets]     # each set's saved U_0
    Y = torch.empty(M, f, dtype=bf, device=dev)
    zparts = draw(t, M, h, std=0.05)    # ranks 1..7: "received" partials
    dxparts = draw(t, M, h, std=0.01)
    Z = torch.empty(M, h, dtype=bf, device=dev)
    dX = torch.empty(M, h, dtype=bf, device=dev)
    dA = torch.empty(h, f, dtype=bf, device=dev)
    dB = torch.empty(f, h, dtype=bf, device=dev)
    stats = torch.empty(t, 3, Mc, dtype=torch.float32, device=dev)
    stats[:, 0].normal_()
    stats[:, 1].uniform_(1.0, 100.0)
    stats[:, 2].zero_()
    loss = torch.empty(Mc, dtype=torch.float32, device=dev)
    ws_bwd = torch.empty(lgs.mlp_bwd_workspace_bytes(w.b, w.s, h, ffn, t, bf), dtype=torch.uint8, device=dev)
    ws_xent = torch.empty(lgs.xent_workspace_bytes(xw.b, xw.s, hc, V, t), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    names = ["mlp_fwd", "sum_z", "mlp_bwd", "sum_dx", "xent", "xent_merge"]
    counter = [0]

    def one_step(ev=None, marks=(0, 1, 2, 3, 4, 5, 6)):
        k = counter[0] % len(sets)
        counter[0] += 1
        Xk, Ak, Bk, dZk, Hk, Ek, yk = sets[k]

        def mark(i):
            if ev is not None and i in marks:
                ev[i].record(stream)
        mark(0)
        lgs.tp_mlp_fwd(w.b, w.s, h, ffn, t, 0, Xk, Ak, Bk, zparts[0], U_i=U[k], Y_i=Y, stream=stream)
        mark(1)
        lgs.shard_partial_sum("sum", t, M * h, zparts, M * h, Z, stream=stream)
        mark(2)
        lgs.tp_mlp_bwd(w.b, w.s, h, ffn, t, 0, Xk, Ak, Bk, U[k], dZk, dxparts[0], dA, dB,
                       workspace=ws_bwd, stream=stream)
        mark(3)
        lgs.shard_partial_sum("sum", t, M * h, dxparts, M * h, dX, stream=stream)
        mark(4)
        lgs.vocab_parallel_xent_fwd(xw.b, xw.s, hc, V, t, 0, Hk, Ek, yk, stats[0, 0], stats[0, 1],
                                    stats[0, 2], workspace=ws_xent, stream=stream)
        mark(5)
        lgs.shard_partial_sum("xent", t, Mc, stats, 3 * Mc, loss, stream=stream)
        mark(6)

    side = torch.cuda.Stream()  # default priority, like every stream here

    def one_step_overlapped():
        """The same step with the backward in three parts (tp_mlp_bwd_dgelu,
        _dx, _dw) and the sum of the dX partials, the stand-in for f*'s
        all-reduce, on a second stream beside the weight-gradient GEMMs,
        which do not read it."""
        k = counter[0] % len(sets)
        counter[0] += 1
        Xk, Ak, Bk, dZk, Hk, Ek, yk = sets[k]
        lgs.tp_mlp_fwd(w.b, w.s, h, ffn, t, 0, Xk, Ak, Bk, zparts[0], U_i=U[k], Y_i=Y, stream=stream)
        lgs.shard_partial_sum("sum", t, M * h, zparts, M * h, Z, stream=stream)
        lgs.tp_mlp_bwd_dgelu(w.b, w.s, h, ffn, t, 0, Bk, U[k], dZk, ws_bwd, stream=stream)
        lgs.tp_mlp_bwd_dx(w.b, w.s, h, ffn, t, 0, Ak, dxparts[0], ws_bwd, stream=stream)
        side.wait_stream(stream)
        lgs.shard_partial_sum("sum", t, M * h, dxparts, M * h, dX, stream=side)
        lgs.tp_mlp_bwd_dw(w.b, w.s, h, ffn, t, 0, Xk, dZk, dA, dB, ws_bwd, stream=stream)
        stream.wait_stream(side)
        lgs.vocab_parallel_xent_fwd(xw.b, xw.s, hc, V, t, 0, Hk, Ek, yk, stats[0, 0], stats[0, 1],
                                    stats[0, 2], workspace=ws_xent, stream=stream)
        lgs.shard_partial_sum("xent", t, Mc, stats, 3 * Mc, loss, stream=stream)

    for _ in range(max(args.warmup, len(sets))):
        one_step()
    torch.cuda.synchronize()
    progress("inputs resident, warm-up steps done")

    mf = mlp_flops(M, h, f)
    fl_x = xent_flops(Mc, hc, Vr)
    # The per-configuration timings, the streaming CE measurement and the clock
    # sampling run before the timed steps, so that those see the device in the
    # steady state a training run keeps it in.
    configs = {} if args.no_per_config else per_config(torch, lgs, reps=50)
    stream_ce = None if args.no_per_config else ce_reduction_stream(torch, lgs, xw)
    gpu_clock = None if args.no_clock else sample_gpu_clock(torch, one_step)
    # the matrix cores' rate on this part with nothing but MFMAs to run (all
    # CUs, random operands): the ceiling the roofline fraction is read against
    ceiling = None
    if not args.no_per_config:
        ops = torch.randn(16, 64, 8, device=dev, generator=torch.Generator(device=dev).manual_seed(11)).to(bf)
        ceiling = mfma_rate_case(torch, lgs, 256, 8, ops, 20000, 3)
    progress("per-configuration timings, CE stream, clock and matrix-core ceiling done")

    # Timed region: K whole steps.  Only the backward entry point is bracketed
    # by HIP events here (its roofline is measured live); events between every
    # entry point cost the step a few percent, so the per-entry-point
    # breakdown comes from a second, untimed pass of K steps below.
    bw_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    counter[0] = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(bw_ev[i], marks=(2, 3))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    progress(f"{args.steps} timed steps: {ms:.3f} ms per step")
    bwd_s = sum(e[2].elapsed_time(e[3]) for e in bw_ev) / args.steps * 1e-3

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    per = {n: 0.0 for n in names}
    for ev in evs:
        for j, n in enumerate(names):
            per[n] += ev[j].elapsed_time(ev[j + 1])
    per = {n: v / args.steps for n, v in per.items()}   # ms per call of each entry point

    # The overlapped schedule of the same step, timed the same way (wall clock
    # over K steps after warm-up steps of its own).
    for _ in range(max(args.warmup, len(sets))):
        one_step_overlapped()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step_overlapped()
    torch.cuda.synchronize()
    ms_ov = (time.perf_counter() - t0) * 1e3 / args.steps
    progress(f"{args.steps} overlapped steps: {ms_ov:.3f} ms per step")

    total_flops = mf["fwd"] + mf["bwd"] + fl_x
    tflops = total_flops / (ms * 1e-3) / 1e12
    mlp_s = (per["mlp_fwd"] + per["mlp_bwd"]) * 1e-3
    sum_bytes = (t + 1) * M * h * 2
    bwd_tf = mf["bwd"] / bwd_s / 1e12
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
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, residual weight scaled 1/sqrt(2N), "
                "dZ ~ N(0,0.01), uniform targets)",
        "config": {"workload": "70B-shape TP shard step, rank 0 of t=8: GeLU MLP fwd+bwd (b=1, s=4096, h=8192, "
                               "ffn=28672) with the sums of 8 partials, plus the vocab-parallel fused CE of "
                               "slice 0 (8.3B shapes: 8192 tokens, h=3072, vocab 51200) and its merge",
                   "b": w.b, "s": w.s, "h": h, "ffn": ffn, "t": t, "rank": 0,
                   "ce": {"tokens": Mc, "h": hc, "vocab": V},
                   "input_sets": f"{len(sets)} rotated, {len(sets) * set_bytes / 1e9:.2f} GB of operands in all "
                                 "(Infinity Cache 0.27 GB): each step reads its operands from HBM"},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "gpu_clock": gpu_clock,
        "timing": "value and ms_per_step: wall clock over the K timed steps, FLOPs of the MLP forward and "
                  "backward and the CE logit GEMM (GEMM FLOPs only, 2MNK each); entry_point_ms: a separate "
                  "pass of K steps with events between entry points",
        "mlp_fwd_bwd_tflops": round((mf["fwd"] + mf["bwd"]) / mlp_s / 1e12, 2),
        "mlp_fwd_bwd_pct_bf16_peak": round(100 * (mf["fwd"] + mf["bwd"]) / mlp_s / 1e12 / PEAK_BF16_TFLOPS, 2),
        "mlp_fwd_tflops": round(mf["fwd"] / (per["mlp_fwd"] * 1e-3) / 1e12, 2),
        "mlp_bwd_tflops": round(mf["bwd"] / (per["mlp_bwd"] * 1e-3) / 1e12, 2),
        "ce_tokens_per_s": round(Mc / (per["xent"] * 1e-3), 0),
        "ce_tflops": round(fl_x / (per["xent"] * 1e-3) / 1e12, 2),
        "sum_partials_gbs": round(sum_bytes / (per["sum_z"] * 1e-3) / 1e9, 1),
        "entry_point_ms": {n: round(v, 4) for n, v in per.items()},
        "overlapped_step": {
            "ms_per_step": round(ms_ov, 4),
            "tflops": round(total_flops / (ms_ov * 1e-3) / 1e12, 2),
            "vs_value": round(ms / ms_ov, 4),
            "note": "the same work with the backward as tp_mlp_bwd_dgelu, tp_mlp_bwd_dx, tp_mlp_bwd_dw and the "
                    "sum of the dX partials (the stand-in for f*'s all-reduce) on a second stream beside the "
                    "weight-gradient GEMMs; the weight-gradient launch then shares the chip with the sum, so "
                    "the roofline above is taken on the serial step"},
        "roofline": {
            "kernel": "tp_mlp_bwd at the 70B shape: the dY+GeLU' GEMM, a 128-counter clear and the grouped "
                      "dB/dA/dX GEMM with its last 128 dA tiles split in two over the tokens (three launches, "
                      "962.1 GFLOP per call), timed with HIP events around the entry point",
            "bound": "mfma",
            "achieved": round(bwd_tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": read_counters(),
            "algorithmic_bytes": mlp_bwd_bytes(M, h, f),
        },
    }
    if ceiling is not None:
        out["mfma_ceiling"] = {
            "tflops": ceiling["tflops"], "clock_mhz": ceiling["clock_mhz"],
            "frac_spec_peak": ceiling["frac_spec_peak"],
            "roofline_achieved_frac_of_ceiling": round(bwd_tf / ceiling["tflops"], 4),
            "note": "lgs_test_mfma_rate on all 256 CUs, two waves per SIMD, N(0,1) operands in registers: "
                    "the most the matrix cores deliver on this part with real data (the power limit holds the "
                    "clock well under the 2.4 GHz of the spec peak); measured in this run"}
    out["per_config"] = configs
    if stream_ce is not None:
        out["ce_reduction_stream"] = stream_ce
    if not args.no_cpu_baseline:
        w2 = WORKLOADS["mlp_8p3b_fwd"]
        X2, A2, B2 = synth.mlp_weights(w2)
        host = {"X": X.double().numpy(), "A0": A0.double().numpy(), "B0": B0.double().numpy(),
                "dZ": dZ.double().numpy(), "H": H.double().numpy(), "E": E.double().numpy(),
                "y": y.numpy().astype("int64"), "Vr": Vr, "X2": X2.double().numpy(),
                "A2_0": A2[:, :w2.f_i].double().numpy(), "B2_0": B2[:w2.f_i].double().numpy()}
        del X2, A2, B2
        progress("CPU oracle baseline starts")
        out["cpu_baseline"] = cpu_baseline(host)
        progress("CPU oracle baseline done")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

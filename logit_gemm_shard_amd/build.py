"""Build liblgs.so (the HIP kernels + the C ABI) in-tree for gfx950.

    python -m logit_gemm_shard_amd.build [--jobs N] [--verbose]

Each ``csrc/*.hip`` file is compiled by hipcc in parallel into
``logit_gemm_shard_amd/_build/``, then linked into
``logit_gemm_shard_amd/liblgs.so``.  Always rebuilds.
"""

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblgs.so")
ARCH = "gfx950"

# Packed fp32 ops (v_pk_*_f32) are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: ROCm is required to build liblgs.so")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(jobs=None, verbose=False, extra_flags=()):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cc = hipcc()
    objs = []
    cmds = []
    for src in srcs:
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON, *DEVICE_FLAGS, *extra_flags, "-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(lambda c: _run(c, verbose), cmds):
            if out.strip() and verbose:
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())

"""Build liblgs.so (the HIP kernels + the C ABI) in-tree for gfx950.

    python -m logit_gemm_shard_amd.build [--jobs N] [--verbose]

Each ``csrc/*.hip`` file is compiled by hipcc in parallel into
``logit_gemm_shard_amd/_build/``, then linked into
``logit_gemm_shard_amd/liblgs.so``.  The same sources compiled with
``-DLGS_DEBUG`` (objects in ``_build_debug/``) give ``liblgs_debug.so``, whose
launchers check every device span a kernel touches against the buffers the
entry point validated (used by the tests only).  Always rebuilds.
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
LIB = os.path.join(PKG, "liblgs.so")
LIB_DEBUG = os.path.join(PKG, "liblgs_debug.so")
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


def _objects(debug, extra_flags):
    build_dir = os.path.join(PKG, "_build_debug" if debug else "_build")
    os.makedirs(build_dir, exist_ok=True)
    flags = [*COMMON, *DEVICE_FLAGS, *extra_flags] + (["-DLGS_DEBUG"] if debug else [])
    objs, cmds = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *flags, "-c", src, "-o", obj])
    return objs, cmds


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)


def build(jobs=None, verbose=False, extra_flags=(), debug=True):
    """Compile and link liblgs.so, and (debug=True) liblgs_debug.so too."""
    variants = [(False, LIB)] + ([(True, LIB_DEBUG)] if debug else [])
    plan = [(_objects(d, extra_flags), lib) for d, lib in variants]
    cmds = [c for (objs, cs), _ in plan for c in cs]
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(lambda c: _run(c, verbose), cmds):
            if out.strip() and verbose:
                print(out)
    for (objs, _), lib in plan:
        _link(objs, lib, verbose)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())

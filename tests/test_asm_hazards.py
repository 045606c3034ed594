"""The compiled kernels never touch an asm LDS read's destination before its
wait (see tests/asm_hazards.py).  Compiles every csrc/*.hip to gfx950
assembly with the library's flags (CPU only: hipcc cross-compiles), and
checks the checker itself on a small kernel that does make the mistake."""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

import asm_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "logit_gemm_shard_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc (ROCm) is required")

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
         "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S"]

# A kernel that reads an asm LDS result before waiting for it.
BAD = r"""
#include <hip/hip_runtime.h>
typedef short s16x4 __attribute__((ext_vector_type(4)));
__global__ void bad(int* out) {
  __shared__ short lds[1024];
  lds[threadIdx.x] = (short)threadIdx.x;
  __syncthreads();
  const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) short*)(lds + 4 * (threadIdx.x & 15));
  s16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
  out[threadIdx.x] = v[0] + v[3];
}
"""


def _asm(src, tmp, name):
    out = os.path.join(tmp, name + ".s")
    subprocess.run([HIPCC, *FLAGS, src, "-o", out], check=True, capture_output=True)
    return open(out).read()


def test_checker_catches_an_early_read(tmp_path):
    src = tmp_path / "bad.hip"
    src.write_text(BAD)
    text = _asm(str(src), str(tmp_path), "bad")
    assert asm_hazards.count_asm_reads(text) == 1
    assert asm_hazards.hazards(text), "the checker missed a read used before its wait"


def test_library_kernels_have_no_early_asm_read_use(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        texts = list(ex.map(lambda p: _asm(p, str(tmp_path), os.path.basename(p)[:-4]), srcs))
    reads = sum(asm_hazards.count_asm_reads(t) for t in texts)
    assert reads > 100  # the GEMM cores' transpose reads are all in there
    bad = set()
    for t in texts:
        bad |= asm_hazards.hazards(t)
    assert not bad, sorted(bad)[:5]

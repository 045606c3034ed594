"""The debug build's host-side bounds checks (no GPU needed).

liblgs_debug.so (the same sources built with -DLGS_DEBUG) records the device
spans each entry point validated and, before every kernel launch, checks that
every span the kernel reads or writes lies inside one of them.  With its dry
run switched on it makes no HIP call, so these tests drive every entry point
at the benchmark's full shapes, at ragged shapes and with padded leading
dimensions through fake device addresses (64 GiB apart, never dereferenced).
A failed check aborts the process, so the calls run in a child process.
"""

import ctypes
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r'''
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
from logit_gemm_shard_amd import binding
L = ctypes.CDLL(binding.LIB_DEBUG_PATH)
for name, res, args in binding.SIGNATURES:
    fn = getattr(L, name); fn.restype = res; fn.argtypes = args
assert L.lgs_test_debug_build() == 1 and L.lgs_test_set_dry_run(1) == 0
BF, F32 = 1, 0
nxt = [0]
def buf():
    nxt[0] += 1
    return nxt[0] << 36          # 64 GiB apart, 16-byte (and 256-byte) aligned
calls = []
def call(name, *a):
    before = L.lgs_test_debug_checks()
    st = getattr(L, name)(*a)
    if st != 0:
        raise SystemExit(f"{name}{a}: status {st}: {L.lgs_last_error().decode()}")
    calls.append((name, L.lgs_test_debug_checks() - before))
def ws(n):
    return (buf(), n) if n else (None, 0)

def mlp(b, s, h, ffn, t, dt, pad=0):
    f, M = ffn // t, b * s
    for r in sorted({0, t - 1}):
        X, A, B, U, Y, Z = (buf() for _ in range(6))
        # A_i, B_i inside full [h, ffn] / [ffn, h] matrices, other matrices with ld = width + pad
        esz = 2 if dt == BF else 4
        A_i, B_i = A + r * f * esz, B + r * f * h * esz
        call("tp_mlp_fwd", b, s, h, ffn, t, r, dt, 0, X, h + pad, A_i, ffn, B_i, h, U, f + pad, Y, f + pad,
             Z, h + pad, None, 0, None)
        w, n = ws(L.lgs_mlp_fwd_workspace_bytes(b, s, h, ffn, t, dt, 0))
        call("tp_mlp_fwd", b, s, h, ffn, t, r, dt, 1, X, h, A_i, ffn, B_i, h, None, 0, None, 0, Z, h, w, n, None)
        dZ, dX, dA, dB = (buf() for _ in range(4))
        w, n = ws(L.lgs_mlp_bwd_workspace_bytes(b, s, h, ffn, t, dt))
        call("tp_mlp_bwd", b, s, h, ffn, t, r, dt, 0, X, h + pad, A_i, ffn, B_i, h, U, f + pad, dZ, h + pad,
             dX, h + pad, dA, f + pad, dB, h + pad, w, n, None)
        call("tp_mlp_bwd_dgelu", b, s, h, ffn, t, r, dt, 1, B_i, h, U, f, dZ, h, w, n, None)
        call("tp_mlp_bwd_dx", b, s, h, ffn, t, r, dt, A_i, ffn, dX, h, w, n, None)
        call("tp_mlp_bwd_dw", b, s, h, ffn, t, r, dt, X, h, dZ, h, dA, f, dB, h, w, n, None)

def swiglu(b, s, h, ffn, t, pad=0):
    f, M = ffn // t, b * s
    X, W, Wd, GU, Y, Z, dZ, dX, dW, dD = (buf() for _ in range(10))
    call("tp_swiglu_fwd", b, s, h, ffn, t, t - 1, BF, X, h + pad, W, 2 * f + pad, Wd, h, GU, 2 * f + pad, Y,
         f + pad, Z, h + pad, None, 0, None)
    w, n = ws(L.lgs_swiglu_fwd_workspace_bytes(b, s, h, ffn, t, BF, 0))
    call("tp_swiglu_fwd", b, s, h, ffn, t, 0, BF, X, h, W, 2 * f, Wd, h, None, 0, None, 0, Z, h, w, n, None)
    w, n = ws(L.lgs_swiglu_bwd_workspace_bytes(b, s, h, ffn, t, BF))
    call("tp_swiglu_bwd", b, s, h, ffn, t, 0, BF, X, h + pad, W, 2 * f + pad, Wd, h + pad, GU, 2 * f + pad,
         dZ, h + pad, dX, h + pad, dW, 2 * f + pad, dD, h + pad, w, n, None)

def xent(b, s, h, V, t, pad=0):
    M, Vr = b * s, V // t
    H, E, y, m, l, T, am, loss = (buf() for _ in range(8))
    for r in sorted({0, t - 1}):
        w, n = ws(L.lgs_xent_workspace_bytes(b, s, h, V, t, BF))
        call("vocab_parallel_xent_fwd", b, s, h, V, t, r, BF, H, h + pad, E + 2 * r * Vr * (h + pad), h + pad, y,
             m, l, T, am, None, w, n, None)
        call("vocab_parallel_xent_fwd", b, s, h, V, t, r, BF, H, h, E, h, y, m, l, T, None, None, w, n, None)
        if L.lgs_xent_workspace_bytes(b, s, h, V, t, BF) <= binding.XENT_NOALLOC_SCRATCH_BYTES:
            call("vocab_parallel_xent_fwd_noalloc", b, s, h, V, t, r, BF, H, h, E, h, y, m, l, T, am, None, None)
        lse, dl, dH, dE = (buf() for _ in range(4))
        w, n = ws(L.lgs_xent_bwd_workspace_bytes(b, s, h, V, t, BF))
        call("vocab_parallel_xent_bwd", b, s, h, V, t, r, BF, H, h + pad, E, h + pad, y, lse, dl, dH, h + pad,
             dE, h + pad, w, n, None)
        call("vocab_parallel_xent_bwd", b, s, h, V, t, r, BF, H, h, E, h, y, lse, None, dH, h, dE, h, w, n, None)
    w, n = ws(L.lgs_xent_workspace_bytes(b, s, h, Vr, 1, BF))
    call("vocab_parallel_xent_fwd", b, s, h, Vr, 1, 0, BF, H, h, E, h, y, m, l, T, am, loss, w, n, None)
    parts, out = buf(), buf()
    for op, per in ((1, 3), (2, 2)):
        call("shard_partial_sum", op, t, M, F32, F32, parts, per * M + 16, out, None)

def sums(t, n, stride):
    for din in (BF, F32):
        for dout in (BF, F32):
            call("shard_partial_sum", 0, t, n, din, dout, buf(), stride, buf(), None)

def sp(t, s, b, h):
    for r in range(t):
        call("shard_reduce_scatter", t, r, s, b, h, BF, BF, buf(), s * b * h, buf(), None)
        if h % 8 == 0:
            for keep in (None, buf()):
                call("shard_reduce_scatter_layernorm", t, r, s, b, h, BF, buf(), s * b * h + 8 * r, buf(), keep,
                     1.25, buf(), buf(), 1e-5, buf(), buf(), None)
                w, nw = ws(L.lgs_layernorm_bwd_workspace_bytes(t, s, b, h, BF))
                call("shard_layernorm_bwd", t, r, s, b, h, BF, buf(), buf(), keep and buf(), keep, 1.25, buf(), 1e-5,
                     buf(), buf(), buf(), buf(), w, nw, None)
    call("shard_all_gather", t, s, b, h, BF, buf(), (s // t) * b * h + 40, buf(), None)

def attn(b, s, h, nq, nkv, d, t, pad=0):
    M, q, kv = b * s, nq // t * d, nkv // t * d
    X, W, QKV, A, Wo, Z, dQ, dX, dW, dZ, dA, dWo = (buf() for _ in range(12))
    for r in sorted({0, t - 1}):
        w, n = ws(L.lgs_attn_qkv_fwd_workspace_bytes(b, s, h, nq, nkv, d, t, BF))
        call("tp_attn_qkv_fwd", b, s, h, nq, nkv, d, t, r, BF, X, h + pad, W, q + 2 * kv + pad, QKV,
             q + 2 * kv + pad, w, n, None)
        call("tp_attn_qkv_fwd", b, s, h, nq, nkv, d, t, r, BF, X, h, W, q + 2 * kv, QKV, q + 2 * kv, None, 0, None)
        call("tp_attn_qkv_bwd", b, s, h, nq, nkv, d, t, r, BF, X, h, W, q + 2 * kv, dQ, q + 2 * kv, dX, h, dW,
             q + 2 * kv, None)
        call("tp_attn_out_fwd", b, s, h, nq, d, t, r, BF, A, q + pad, Wo, h + pad, Z, h + pad, None)
        w, n = ws(L.lgs_attn_out_bwd_workspace_bytes(b, s, h, nq, d, t, BF))
        call("tp_attn_out_bwd", b, s, h, nq, d, t, r, BF, A, q, Wo, h, dZ, h, dA, q, dWo, h, w, n, None)
        call("tp_attn_out_bwd", b, s, h, nq, d, t, r, BF, A, q, Wo, h, dZ, h, dA, q, dWo, h, None, 0, None)

def testing_entry_points():
    for tile in range(L.lgs_test_num_tiles()):
        for ak, bk in ((1, 0), (1, 1), (0, 0)):
            M, N, K = 600, 456, 200
            A, B, C = buf(), buf(), buf()
            call("lgs_test_gemm_bf16", tile, ak, bk, M, N, K, A, K if ak else M, B, K if bk else N, C, N + 8, None)
    call("lgs_test_xent_rows_bf16", 8192, 6400, 0, buf(), 6400, buf(), buf(), buf(), buf(), None)
    call("lgs_test_xent_rows_bf16", 65, 1000, 3000, buf(), 1024, buf(), buf(), buf(), buf(), None)

# the benchmark's and the tests' full shapes
mlp(2, 64, 256, 1024, 2, F32)                 # tiny block, fp32
mlp(8, 1024, 3072, 12288, 8, BF)              # 8.3B
mlp(1, 4096, 8192, 28672, 8, BF)              # 70B
mlp(2, 1100, 1064, 2 * 1048, 2, BF)           # backward split over tokens: 2 parts
mlp(1, 8264, 776, 1040, 2, BF)                # 4 parts, ragged last part
mlp(3, 200, 136, 528, 2, BF, pad=24)          # ragged, padded leading dimensions
mlp(1, 33, 72, 128, 8, F32, pad=8)
mlp(1, 9, 64, 256, 2, BF)
swiglu(1, 4096, 8192, 28672, 8)
swiglu(1, 520, 328, 3 * 208, 3, pad=24)
xent(8, 1024, 3072, 51200, 8)                 # 8.3B vocabulary
xent(2, 1000, 136, 24640, 1)                  # slice split over two launches
xent(2, 129, 136, 4 * 520, 4, pad=8)
sums(8, 4096 * 8192, 4096 * 8192)
sums(3, 1001, 1024)
sp(8, 1024, 8, 3072)
sp(4, 12, 3, 72)
sp(2, 6, 1, 16384)
sp(3, 9, 2, 2056)
attn(1, 4096, 8192, 64, 8, 128, 8)
attn(1, 2072, 1032, 8, 2, 72, 2, pad=8)
testing_entry_points()
# the randomized parity tests' shapes
sys.path.insert(0, sys.argv[1] + "/tests")
from fuzz_cases import ATTN_CASES, MLP_CASES, SPLN_CASES, SUM_CASES, SWIGLU_CASES, XENT_CASES
for b, s, h, ffn, t, _, _ in MLP_CASES:
    mlp(b, s, h, ffn, t, BF)
for b, s, h, V, t in XENT_CASES:
    xent(b, s, h, V, t)
for b, s, h, ffn, t, _ in SWIGLU_CASES:
    swiglu(b, s, h, ffn, t)
for t, n, _ in SUM_CASES:
    sums(t, n, n)
for b, s, h, nq, nkv, d, t, _ in ATTN_CASES:
    attn(b, s, h, nq, nkv, d, t)
for t, s, b, h, _, _ in SPLN_CASES:
    sp(t, s, b, h)
print(json.dumps({"calls": len(calls), "checks": L.lgs_test_debug_checks(),
                  "min_checks_per_call": min(c for _, c in calls)}))
'''


@pytest.fixture(scope="module")
def debug_lib():
    from logit_gemm_shard_amd import binding
    if not os.path.exists(binding.LIB_DEBUG_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.LIB_DEBUG_PATH


def _run(code, *args):
    return subprocess.run([sys.executable, "-c", code, ROOT, *args], capture_output=True, text=True,
                          timeout=300)


def test_debug_and_product_builds_export_the_same_symbols(debug_lib):
    from logit_gemm_shard_amd import binding
    names = []
    for path in (binding.LIB_PATH, debug_lib):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                             check=True).stdout
        names.append({l.split()[-1] for l in out.splitlines() if " T " in l})
    assert names[0] == names[1]
    assert ctypes.CDLL(debug_lib).lgs_test_debug_build() == 1
    assert binding.lib().lgs_test_debug_build() == 0
    assert binding.lib().lgs_test_set_dry_run(1) == -1     # the product build has no dry run
    assert binding.lib().lgs_test_debug_checks() == 0


def test_every_entry_point_keeps_its_launches_inside_the_validated_buffers(debug_lib):
    r = _run(DRIVER)
    assert r.returncode == 0, r.stderr[-3000:] + r.stdout[-2000:]
    summary = json.loads(r.stdout.strip().splitlines()[-1])
    print(summary)
    assert summary["calls"] > 150
    assert summary["min_checks_per_call"] >= 3   # every call ran its launchers' checks
    assert summary["checks"] > 1500


CHECK = r'''
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from logit_gemm_shard_amd import binding
L = ctypes.CDLL(binding.LIB_DEBUG_PATH)
L.lgs_test_debug_span.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t]
A = 1 << 40
off, n = int(sys.argv[2]), int(sys.argv[3])
print("returned", L.lgs_test_debug_span(A, 4096, A + off, n), flush=True)
'''


@pytest.mark.parametrize("off,n,inside", [(0, 4096, True), (96, 4000, True), (4095, 1, True), (0, 0, True),
                                          (96, 4001, False), (-16, 16, False), (4096, 1, False),
                                          (1 << 20, 8, False)])
def test_a_span_outside_the_validated_buffers_aborts(debug_lib, off, n, inside):
    r = _run(CHECK, str(off), str(n))
    if inside:
        assert r.returncode == 0 and "returned 0" in r.stdout, r.stderr
    else:
        assert r.returncode != 0 and "outside every validated buffer" in r.stderr, (r.returncode, r.stderr)

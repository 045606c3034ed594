"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

* liblgs.so loads and exports every function include/lgs.h declares, and
  nothing else under the library's names;
* every validation rule returns its status code before any HIP call (the
  pointers passed here are fake and would fault if anything were enqueued).
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("lgs.h", "lgs_testing.h")]

FAKE = 0x10000  # 64 KiB-aligned fake device address: never dereferenced


@pytest.fixture(scope="module")
def L():
    from logit_gemm_shard_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.lib()


def declared_functions():
    names = []
    for hdr in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ("tp_mlp_fwd", "tp_mlp_bwd", "vocab_parallel_xent_fwd", "shard_partial_sum",
               "tp_swiglu_fwd", "tp_swiglu_bwd"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    from logit_gemm_shard_amd import binding
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in lgs.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    ours = {n for n in exported if n.startswith(("lgs_", "tp_", "vocab_", "shard_"))}
    assert ours == set(declared_functions())
    # the binding knows every declared function
    assert {n for n, _, _ in binding.SIGNATURES} == set(declared_functions())


def test_status_strings(L):
    assert L.lgs_version() >= 100
    for st in range(5):
        assert L.lgs_status_string(st)
    assert L.lgs_status_string(99) == b"unknown status"


def _fwd(L, **kw):
    a = dict(b=2, s=64, h=256, ffn=1024, t=2, rank=0, dtype=1, act=0, X=FAKE, ldx=256, A=FAKE,
             lda=1024, B=FAKE, ldb=256, U=None, ldu=0, Y=FAKE, ldy=512, Z=FAKE, ldz=256, ws=None,
             ws_bytes=0, stream=None)
    a.update(kw)
    return L.tp_mlp_fwd(a["b"], a["s"], a["h"], a["ffn"], a["t"], a["rank"], a["dtype"], a["act"],
                        a["X"], a["ldx"], a["A"], a["lda"], a["B"], a["ldb"], a["U"], a["ldu"],
                        a["Y"], a["ldy"], a["Z"], a["ldz"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(b=0), 1), (dict(s=-1), 1), (dict(h=0), 1), (dict(t=0), 1),
    (dict(rank=2), 1), (dict(rank=-1), 1),
    (dict(ffn=1001), 1),                      # not divisible by t
    (dict(dtype=7), 2), (dict(act=5), 2),
    (dict(h=252, ldx=252, ldb=252, ldz=252), 2),  # h % 8
    (dict(ffn=1020, ldy=510, lda=1020), 2),   # ffn/t % 8
    (dict(X=None), 1), (dict(A=None), 1), (dict(B=None), 1), (dict(Z=None), 1),
    (dict(ldx=255), 1), (dict(lda=500), 1), (dict(ldz=8), 1),
    (dict(X=FAKE + 2), 2),                    # bf16 needs 16-byte alignment
    (dict(ldx=260), 2),                       # bf16 ld % 8
    (dict(Y=None), 3),                        # needs a workspace
    (dict(Y=None, ws=FAKE, ws_bytes=10), 3),
    (dict(Y=None, ws=FAKE + 16, ws_bytes=1 << 20), 2),
    (dict(b=1 << 16, s=1 << 16), 1),          # more than INT_MAX tokens
])
def test_mlp_fwd_validation(L, kw, code):
    assert _fwd(L, **kw) == code
    assert L.lgs_last_error()


def test_mlp_fwd_fp32_alignment_rules(L):
    # fp32 needs only 4-byte alignment and no ld multiple
    assert _fwd(L, dtype=0, X=FAKE + 2) == 2
    assert _fwd(L, dtype=0, ldx=257, X=None) == 1


def test_mlp_bwd_validation(L):
    def bwd(**kw):
        a = dict(b=1, s=16, h=64, ffn=128, t=2, rank=1, dtype=1, act=0, ws=FAKE, ws_bytes=1 << 20)
        a.update(kw)
        p = [FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64]
        for i, v in kw.get("mats", {}).items():
            p[i] = v
        return L.tp_mlp_bwd(a["b"], a["s"], a["h"], a["ffn"], a["t"], a["rank"], a["dtype"],
                            a["act"], *p, a["ws"], a["ws_bytes"], None)
    assert bwd(rank=2) == 1
    assert bwd(mats={6: None}) == 1          # U_i required
    assert bwd(mats={3: 32}) == 1            # lda < ffn/t = 64 ... (lda is index 3)
    assert bwd(ws=None) == 3
    assert bwd(ws_bytes=100) == 3
    need = L.lgs_mlp_bwd_workspace_bytes(1, 16, 64, 128, 2, 1)
    assert need == 2 * 2048
    assert bwd(ws_bytes=need - 1) == 3


def test_mlp_bwd_workspace_holds_the_weight_gradient_split(L):
    """Y_i and dU_i, plus, for bf16 shapes whose dB / dA tiles are few and
    long (many tokens, small h and f), the K-split partial sums (fp32, one
    256x256 slot per tile and part) and one counter per tile; the same for
    the split tiles alone where only the last dA tiles are split (the 70B
    shape: 448 + 448 + 512 blocks, the last 128 dA tiles in 2 parts)."""
    def plain(b, s, ffn, t, el):
        return 2 * (((b * s * (ffn // t) * el) + 255) // 256 * 256)
    L.lgs_mlp_bwd_workspace_bytes.restype = ctypes.c_size_t
    # the 8.3B shape: not split
    assert L.lgs_mlp_bwd_workspace_bytes(8, 1024, 3072, 12288, 8, 1) == plain(8, 1024, 12288, 8, 2)
    tail = 128 * 2 * 256 * 256 * 4 + 512
    assert L.lgs_mlp_bwd_workspace_bytes(1, 4096, 8192, 28672, 8, 1) == plain(1, 4096, 28672, 8, 2) + tail
    # M = 8264 tokens, h = 776, f = 520: 3 x 4 tiles each for dB and dA, 4 parts
    tiles, parts = 2 * 3 * 4, 4
    split = tiles * parts * 256 * 256 * 4 + 256
    assert L.lgs_mlp_bwd_workspace_bytes(1, 8264, 776, 1040, 2, 1) == plain(1, 8264, 1040, 2, 2) + split
    # fp32 never splits
    assert L.lgs_mlp_bwd_workspace_bytes(1, 8264, 776, 1040, 2, 0) == plain(1, 8264, 1040, 2, 4)


def _swiglu_fwd(L, **kw):
    # f = ffn / t = 64: Wgu_i is [h, 2f] = [64, 128]
    a = dict(b=1, s=16, h=64, ffn=128, t=2, rank=0, dtype=1, X=FAKE, ldx=64, W=FAKE, ldw=128,
             D=FAKE, ldd=64, GU=None, ldgu=0, Y=FAKE, ldy=64, Z=FAKE, ldz=64, ws=None, ws_bytes=0)
    a.update(kw)
    return L.tp_swiglu_fwd(a["b"], a["s"], a["h"], a["ffn"], a["t"], a["rank"], a["dtype"], a["X"],
                           a["ldx"], a["W"], a["ldw"], a["D"], a["ldd"], a["GU"], a["ldgu"], a["Y"],
                           a["ldy"], a["Z"], a["ldz"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=0), 1), (dict(rank=2), 1), (dict(ffn=129), 1),  # ffn % t
    (dict(dtype=0), 2),                       # bf16 only
    (dict(dtype=5), 2),
    (dict(ffn=120, ldy=64), 2),               # ffn/t = 60 not a multiple of 8
    (dict(ldw=64), 1),                        # Wgu_i holds 2f = 128 columns
    (dict(GU=FAKE, ldgu=64), 1),              # so does GU_i
    (dict(GU=FAKE + 8, ldgu=128), 2),         # 16-byte alignment
    (dict(W=None), 1), (dict(D=None), 1), (dict(Z=None), 1),
    (dict(Y=None), 3), (dict(Y=None, ws=FAKE, ws_bytes=100), 3),
])
def test_swiglu_fwd_validation(L, kw, code):
    assert _swiglu_fwd(L, **kw) == code
    assert L.lgs_last_error()


def test_swiglu_bwd_validation(L):
    def bwd(**kw):
        a = dict(b=1, s=16, h=64, ffn=128, t=2, rank=1, dtype=1, ws=FAKE, ws_bytes=1 << 20)
        a.update(kw)
        # X, Wgu_i, Wd_i, GU_i, dZ, dX_i, dWgu_i, dWd_i with their ld
        p = [FAKE, 64, FAKE, 128, FAKE, 64, FAKE, 128, FAKE, 64, FAKE, 64, FAKE, 128, FAKE, 64]
        for i, v in kw.get("mats", {}).items():
            p[i] = v
        return L.tp_swiglu_bwd(a["b"], a["s"], a["h"], a["ffn"], a["t"], a["rank"], a["dtype"], *p,
                               a["ws"], a["ws_bytes"], None)
    assert bwd(rank=2) == 1
    assert bwd(dtype=0) == 2
    assert bwd(mats={6: None}) == 1          # GU_i required
    assert bwd(mats={7: 64}) == 1            # ldgu < 2f
    assert bwd(mats={13: 96}) == 1           # lddwgu < 2f
    assert bwd(ws=None) == 3
    # Y_i [16, 64] and dGU_i [16, 128] bf16, each rounded up to 256 bytes
    need = L.lgs_swiglu_bwd_workspace_bytes(1, 16, 64, 128, 2, 1)
    assert need == 2048 + 4096
    assert bwd(ws_bytes=need - 1) == 3
    assert L.lgs_swiglu_fwd_workspace_bytes(1, 16, 64, 128, 2, 1, 1) == 0
    assert L.lgs_swiglu_fwd_workspace_bytes(1, 16, 64, 128, 2, 1, 0) == 2048


def test_mlp_bwd_parts_validation(L):
    # (b, s, h, ffn, t, rank, dtype, act, B, ldb, U, ldu, dZ, lddz, ws, ws_bytes, stream)
    dg = lambda **k: L.tp_mlp_bwd_dgelu(1, 16, 64, 128, 2, k.get("rank", 1), 1, k.get("act", 0), FAKE, 64,
                                        k.get("U", FAKE), 64, FAKE, 64, k.get("ws", FAKE), k.get("wsb", 1 << 20),
                                        None)
    assert dg(rank=2) == 1 and dg(act=9) == 2 and dg(U=None) == 1
    assert dg(ws=None) == 3 and dg(wsb=100) == 3 and dg(ws=FAKE + 16) == 2
    dx = L.tp_mlp_bwd_dx(1, 16, 64, 128, 2, 0, 1, FAKE, 32, FAKE, 64, None, 0, None)
    assert dx == 1                          # lda < ffn/t = 64
    dx = L.tp_mlp_bwd_dx(1, 16, 64, 128, 2, 0, 1, FAKE, 64, FAKE, 64, None, 0, None)
    assert dx == 3                          # the shared workspace is required
    dw = L.tp_mlp_bwd_dw(1, 16, 64, 128, 2, 0, 1, FAKE, 64, FAKE, 64, FAKE, 64, None, 64, FAKE, 1 << 20, None)
    assert dw == 1                          # dB_i required


def test_xent_validation(L):
    def xe(**kw):
        a = dict(b=2, s=8, h=64, vocab=1024, t=4, rank=0, dtype=1, H=FAKE, ldh=64, E=FAKE, lde=64,
                 y=FAKE, m=FAKE, l=FAKE, T=FAKE, am=None, loss=None, ws=FAKE, ws_bytes=1 << 24)
        a.update(kw)
        return L.vocab_parallel_xent_fwd(a["b"], a["s"], a["h"], a["vocab"], a["t"], a["rank"],
                                         a["dtype"], a["H"], a["ldh"], a["E"], a["lde"], a["y"],
                                         a["m"], a["l"], a["T"], a["am"], a["loss"], a["ws"],
                                         a["ws_bytes"], None)
    assert xe(vocab=1022) == 1
    assert xe(rank=4) == 1
    assert xe(dtype=0) == 2
    assert xe(h=60, ldh=60, lde=60) == 2
    assert xe(loss=FAKE) == 1               # loss only for the whole vocabulary
    assert xe(y=None) == 1
    assert xe(ws=None) == 3
    assert xe(ws_bytes=16) == 3
    assert xe(lde=32) == 1
    # one 16-byte entry per token and slab written: the 8.3B slice (6400 columns)
    # runs 2560 columns on 256x320 tiles (16 slabs of 160) and 3840 on 256x256
    # (30 slabs of 128)
    assert L.lgs_xent_workspace_bytes(8, 1024, 3072, 51200, 8, 1) == 46 * 8192 * 16


def test_xent_noalloc_validation(L):
    """The allocation-free CE forward applies the same argument rules, and
    rejects calls whose slab partials exceed its static scratch, before any
    HIP call."""
    def xn(**kw):
        a = dict(b=2, s=8, h=64, vocab=1024, t=4, rank=0, dtype=1, H=FAKE, ldh=64, E=FAKE, lde=64,
                 y=FAKE, m=FAKE, l=FAKE, T=FAKE, am=None, loss=None)
        a.update(kw)
        return L.vocab_parallel_xent_fwd_noalloc(a["b"], a["s"], a["h"], a["vocab"], a["t"],
                                                 a["rank"], a["dtype"], a["H"], a["ldh"], a["E"],
                                                 a["lde"], a["y"], a["m"], a["l"], a["T"], a["am"],
                                                 a["loss"], None)
    assert xn(vocab=1022) == 1
    assert xn(rank=4) == 1
    assert xn(dtype=0) == 2
    assert xn(loss=FAKE) == 1
    assert xn(y=None) == 1
    assert xn(lde=32) == 1
    from logit_gemm_shard_amd import binding
    cap = binding.XENT_NOALLOC_SCRATCH_BYTES
    # 8192 tokens at the 8.3B slice fit (6 MiB); 32768 do not (23 MiB)
    assert L.lgs_xent_workspace_bytes(8, 1024, 3072, 51200, 8, 1) <= cap
    assert L.lgs_xent_workspace_bytes(32, 1024, 3072, 51200, 8, 1) > cap
    big = xn(b=32, s=1024, h=3072, vocab=51200, t=8, ldh=3072, lde=3072)
    assert big == 2 and b"static scratch" in L.lgs_last_error()


def test_xent_bwd_validation(L):
    def xb(**kw):
        a = dict(b=2, s=8, h=64, vocab=1024, t=4, rank=0, dtype=1, H=FAKE, ldh=64, E=FAKE, lde=64,
                 y=FAKE, lse=FAKE, w=None, dH=FAKE, lddh=64, dE=FAKE, ldde=64, ws=FAKE, ws_bytes=1 << 24)
        a.update(kw)
        return L.vocab_parallel_xent_bwd(a["b"], a["s"], a["h"], a["vocab"], a["t"], a["rank"],
                                         a["dtype"], a["H"], a["ldh"], a["E"], a["lde"], a["y"],
                                         a["lse"], a["w"], a["dH"], a["lddh"], a["dE"], a["ldde"],
                                         a["ws"], a["ws_bytes"], None)
    assert xb(vocab=1022) == 1
    assert xb(rank=4) == 1
    assert xb(dtype=0) == 2
    assert xb(vocab=4 * 260) == 2           # vocab/t = 260 not a multiple of 8
    assert xb(lse=None) == 1 and xb(y=None) == 1
    assert xb(dE=None) == 1 and xb(ldde=32) == 1
    assert xb(w=FAKE + 2) == 2              # dloss 4-byte aligned when given
    assert xb(ws=None) == 3
    # G is M x vocab/t bf16: 16 tokens x 256 entries x 2 B
    need = L.lgs_xent_bwd_workspace_bytes(2, 8, 64, 1024, 4, 1)
    assert need == 16 * 256 * 2
    assert xb(ws_bytes=need - 1) == 3
    assert xb(b=1 << 12, s=1 << 12, h=8, ldh=8, lde=8, lddh=8, ldde=8, vocab=8 * 1024, t=1) == 2  # G over 2 GiB
    assert b"G" in L.lgs_last_error()


def test_partial_sum_validation(L):
    assert L.shard_partial_sum(0, 0, 16, 1, 1, FAKE, 16, FAKE, None) == 1
    assert L.shard_partial_sum(0, 2, -1, 1, 1, FAKE, 16, FAKE, None) == 1
    assert L.shard_partial_sum(0, 2, 16, 1, 1, FAKE, 8, FAKE, None) == 1   # stride < n
    assert L.shard_partial_sum(0, 2, 16, 3, 1, FAKE, 16, FAKE, None) == 2
    assert L.shard_partial_sum(9, 2, 16, 1, 1, FAKE, 16, FAKE, None) == 2
    assert L.shard_partial_sum(1, 2, 16, 1, 0, FAKE, 48, FAKE, None) == 2  # xent is fp32
    assert L.shard_partial_sum(1, 2, 16, 0, 0, FAKE, 40, FAKE, None) == 1  # stride < 3n
    assert L.shard_partial_sum(0, 2, 16, 1, 1, None, 16, FAKE, None) == 1
    # n == 0 is a no-op and touches nothing
    assert L.shard_partial_sum(0, 3, 0, 1, 1, None, 0, None, None) == 0
    # the log-sum-exp merge reads two planes per rank block
    assert L.shard_partial_sum(2, 2, 16, 0, 0, FAKE, 31, FAKE, None) == 1   # stride < 2n
    assert L.shard_partial_sum(2, 2, 16, 1, 0, FAKE, 48, FAKE, None) == 2   # fp32 only
    assert L.shard_partial_sum(3, 2, 16, 0, 0, FAKE, 48, FAKE, None) == 2   # no op 3


def test_attn_validation(L):
    def qf(**kw):
        a = dict(b=1, s=16, h=64, nq=8, nkv=4, d=8, t=2, rank=0, dtype=1, X=FAKE, ldx=64, W=FAKE,
                 ldw=64, Y=FAKE, ldy=64)  # q = 4*8 = 32, kv = 2*8 = 16: 64 columns
        a.update(kw)
        return L.tp_attn_qkv_fwd(a["b"], a["s"], a["h"], a["nq"], a["nkv"], a["d"], a["t"], a["rank"],
                                 a["dtype"], a["X"], a["ldx"], a["W"], a["ldw"], a["Y"], a["ldy"],
                                 a.get("ws"), a.get("wsb", 0), None)
    assert qf(nq=7) == 1                    # n_q % t
    assert qf(nkv=3, t=1) == 1              # n_q % n_kv
    assert qf(nkv=1) == 1                   # n_kv % t
    assert qf(d=12) == 2                    # head_dim % 8
    assert qf(dtype=0) == 2
    assert qf(ldw=48) == 1 and qf(ldy=56) == 1  # widths q + 2 kv = 64
    assert qf(rank=2) == 1
    assert qf(nq=7, ws=FAKE + 64, wsb=1 << 20) == 1  # shape errors come first
    assert qf(d=12, ws=FAKE + 64, wsb=1 << 20) == 2
    # the split-K workspace: none for small shapes; for the 70B rank (4096 x
    # 1280 outputs, K = 8192: 80 tiles of 256x256 in 3 parts over K) one fp32
    # 256x256 slot per tile and part, and one counter per tile
    ws = L.lgs_attn_qkv_fwd_workspace_bytes
    assert ws(1, 16, 64, 8, 4, 8, 2, 1) == 0
    assert ws(1, 4096, 8192, 64, 8, 128, 8, 1) == (80 * 3 * 256 * 256 * 4 + 80 * 4 + 255) // 256 * 256
    assert ws(1, 4096, 8192, 64, 8, 128, 8, 0) == 0  # invalid (fp32): no workspace
    assert L.lgs_last_error() == b""
    of = lambda **kw: L.tp_attn_out_fwd(1, 16, 64, kw.get("nq", 8), 8, 2, kw.get("rank", 0), 1, FAKE,
                                        kw.get("lda", 32), FAKE, 64, FAKE, 64, None)
    assert of(nq=7) == 1 and of(lda=24) == 1 and of(rank=5) == 1  # n_q % t, lda < q = 32, rank
    ob = L.tp_attn_out_bwd(1, 16, 64, 8, 8, 2, 0, 1, FAKE, 32, FAKE, 64, FAKE, 64, None, 32, FAKE, 64, None, 0,
                           None)
    assert ob == 1                          # dA_i required
    # dA's split-K workspace at the 70B shape: [4096, 1024] is 64 tiles, each
    # in two parts over K: two fp32 slots per tile, one counter per tile
    assert L.lgs_attn_out_bwd_workspace_bytes(1, 4096, 8192, 64, 128, 8, 1) == \
        (64 * 2 * 256 * 256 * 4 + 64 * 4 + 255) // 256 * 256
    assert L.lgs_attn_out_bwd_workspace_bytes(1, 16, 64, 8, 8, 2, 1) == 0
    qb = L.tp_attn_qkv_bwd(1, 16, 64, 8, 4, 8, 2, 0, 1, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 64, FAKE, 32, None)
    assert qb == 1                          # lddw < q + 2 kv


def test_sp_validation(L):
    rs = L.shard_reduce_scatter
    ag = L.shard_all_gather
    # (t, rank, s, b, h, in, out, parts, stride, out, stream)
    assert rs(4, 0, 10, 2, 8, 1, 1, FAKE, 160, FAKE, None) == 1    # s % t
    assert rs(4, 4, 8, 2, 8, 1, 1, FAKE, 128, FAKE, None) == 1     # rank
    assert rs(4, 0, 8, 2, 8, 1, 1, FAKE, 100, FAKE, None) == 1     # stride < s*b*h
    assert rs(4, 0, 8, 2, 8, 5, 1, FAKE, 128, FAKE, None) == 2     # dtype
    assert rs(4, 0, 8, 2, 8, 0, 1, FAKE + 2, 128, FAKE, None) == 2  # fp32 alignment
    assert rs(4, 0, 8, 2, 8, 1, 1, None, 128, FAKE, None) == 1
    assert rs(0, 0, 8, 2, 8, 1, 1, FAKE, 128, FAKE, None) == 1
    # (t, s, b, h, dtype, shards, stride, out, stream)
    assert ag(4, 10, 2, 8, 1, FAKE, 40, FAKE, None) == 1           # s % t
    assert ag(4, 8, 2, 8, 1, FAKE, 31, FAKE, None) == 1            # stride < (s/t)*b*h
    assert ag(4, 8, 2, 8, 7, FAKE, 32, FAKE, None) == 2
    assert ag(4, 8, 2, 8, 1, FAKE, 32, None, None) == 1
    assert ag(4, 8, 2, 8, 1, FAKE + 1, 32, FAKE, None) == 2
    ln = L.shard_reduce_scatter_layernorm

    def call(t=4, r=0, s=8, b=2, h=16, dt=1, parts=FAKE, stride=256, res=FAKE, keep=None, scale=1.0, g=FAKE,
             bb=FAKE, eps=1e-5, hs=FAKE, y=FAKE):
        return ln(t, r, s, b, h, dt, parts, stride, res, keep, scale, g, bb, eps, hs, y, None)
    assert call(s=10) == 1                      # s % t
    assert call(r=4) == 1                       # rank
    assert call(stride=255) == 1                # stride < s*b*h
    assert call(stride=260) == 2                # stride not a multiple of 8
    assert call(dt=0) == 2                      # fp32: bf16 only
    assert call(h=12) == 2                      # h % 8
    assert call(h=16392, stride=8 * 2 * 16392) == 2  # h above 16384
    assert call(eps=0.0) == 1 and call(eps=float("nan")) == 1 and call(scale=float("inf")) == 1
    assert call(res=None) == 1 and call(g=None) == 1 and call(y=None) == 1
    assert call(hs=FAKE + 8) == 2               # 16-byte alignment
    assert call(keep=FAKE + 4) == 2             # the mask's 8-byte alignment
    # the backward: (t, rank, s, b, h, dtype, hs, dy, dhs, keep, scale, gamma, eps, g, dz, dgamma, dbeta, ws, wsb)
    wsq = L.lgs_layernorm_bwd_workspace_bytes
    assert wsq(8, 1024, 8, 3072, 1) == 256 * 2 * 3072 * 4    # 1024 rows: 256 blocks of 4, two fp32 rows each
    assert wsq(4, 8, 2, 16, 1) == 256 * ((4 * 2 * 16 * 4 + 255) // 256)
    assert wsq(4, 8, 2, 12, 1) == 0 and wsq(4, 8, 2, 16, 0) == 0 and wsq(4, 10, 2, 16, 1) == 0
    bw = L.shard_layernorm_bwd

    def bcall(t=4, r=0, s=8, b=2, h=16, dt=1, dhs=None, keep=None, scale=1.0, eps=1e-5, g=FAKE, ws=FAKE,
              wsb=1 << 20):
        return bw(t, r, s, b, h, dt, FAKE, FAKE, dhs, keep, scale, FAKE, eps, g, FAKE, FAKE, FAKE, ws, wsb, None)
    assert bcall(s=10) == 1 and bcall(r=-1) == 1 and bcall(dt=0) == 2 and bcall(h=12) == 2
    assert bcall(eps=-1.0) == 1 and bcall(g=None) == 1
    assert bcall(ws=None) == 3 and bcall(wsb=16) == 3      # workspace missing or short
    assert bcall(dhs=FAKE + 2) == 2 and bcall(keep=FAKE + 1) == 2


def test_binding_raises_when_library_missing(tmp_path, monkeypatch):
    from logit_gemm_shard_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def test_testing_interface(L):
    from logit_gemm_shard_amd import binding
    shapes = binding.tile_shapes()
    assert (256, 256) in shapes and (128, 128) in shapes
    assert L.lgs_test_tile_shape(len(shapes), None, None) == -1
    # the picker weighs full rounds of 256 blocks against the cores' throughput:
    # 4096 x 3584 -> 224 blocks of 256x256 (one round) beats 256 of 256x224
    assert shapes[binding.pick_tile(4096, 3584)] == (256, 256)
    assert shapes[binding.pick_tile(8192, 1536)] == (256, 192)
    assert shapes[binding.pick_tile(8192, 6400)] == (256, 320)  # 640 blocks: 2.5 rounds
    assert L.lgs_test_gemm_bf16(0, 0, 1, 64, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, None) == 2
    assert L.lgs_test_gemm_bf16(9, 1, 1, 64, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, None) == 1
    assert L.lgs_test_gemm_bf16(0, 1, 1, 64, 60, 64, FAKE, 64, FAKE, 64, FAKE, 64, None) == 2
    # streaming CE partials: Vr % 8, leading dimension, required pointers, empty input
    assert L.lgs_test_xent_rows_bf16(4, 100, 0, FAKE, 104, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.lgs_test_xent_rows_bf16(4, 64, 0, FAKE, 32, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.lgs_test_xent_rows_bf16(4, 64, 0, FAKE, 64, None, FAKE, FAKE, FAKE, None) == 1
    assert L.lgs_test_xent_rows_bf16(4, 64, 0, FAKE + 2, 64, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.lgs_test_xent_rows_bf16(0, 64, 0, None, 64, None, None, None, None, None) == 0
    # matrix-core rate probe: block and wave counts, iteration bound, pointers, alignment
    assert L.lgs_test_mfma_rate(0, 4, 1, FAKE, FAKE, FAKE, None) == 1
    assert L.lgs_test_mfma_rate(65537, 4, 1, FAKE, FAKE, FAKE, None) == 1
    assert L.lgs_test_mfma_rate(1, 9, 1, FAKE, FAKE, FAKE, None) == 1
    assert L.lgs_test_mfma_rate(1, 4, (1 << 24) + 1, FAKE, FAKE, FAKE, None) == 1
    assert L.lgs_test_mfma_rate(1, 4, -1, FAKE, FAKE, FAKE, None) == 1
    assert L.lgs_test_mfma_rate(1, 4, 1, None, FAKE, FAKE, None) == 1
    assert L.lgs_test_mfma_rate(1, 4, 1, FAKE + 8, FAKE, FAKE, None) == 2


def test_binding_temporary_workspace_needs_a_recordable_stream():
    """A temporary workspace is recorded on the call's stream (so the caching
    allocator cannot reuse it under running kernels); a raw stream handle
    cannot be recorded, so the binding refuses to make one for it."""
    from logit_gemm_shard_amd import binding
    with pytest.raises(ValueError, match="raw handle"):
        binding._workspace(256, "cpu", None, stream=12345)
    assert binding._workspace(0, "cpu", None, stream=12345) == (None, 0)

"""ctypes binding of liblgs.so (include/lgs.h), same names as the C entry points.

Argument marshalling only: tensors become device pointers plus leading
dimensions, the stream is torch's current HIP stream, and a workspace tensor
is allocated through torch when the caller passes none.  Every step of the
computation runs in the library's kernels; there is no fallback: if the
library is not built, every call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblgs.so")

LGS_OK, LGS_ERR_INVALID_ARG, LGS_ERR_UNSUPPORTED, LGS_ERR_WORKSPACE, LGS_ERR_HIP = range(5)
LGS_F32, LGS_BF16 = 0, 1
LGS_GELU_ERF, LGS_GELU_TANH = 0, 1
LGS_REDUCE_SUM, LGS_REDUCE_XENT, LGS_REDUCE_XENT_LSE = 0, 1, 2

_ACT = {"erf": LGS_GELU_ERF, "tanh": LGS_GELU_TANH}
_DT = {torch.float32: LGS_F32, torch.bfloat16: LGS_BF16}

_lib = None

# (name, restype, argtypes) of every exported entry point, in header order.
_i, _i64, _p, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = [
    ("lgs_version", _i, []),
    ("lgs_status_string", ctypes.c_char_p, [_i]),
    ("lgs_last_error", ctypes.c_char_p, []),
    ("lgs_mlp_fwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i, _i]),
    ("lgs_mlp_bwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i]),
    ("lgs_swiglu_fwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i, _i]),
    ("lgs_swiglu_bwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i]),
    ("lgs_xent_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i]),
    ("lgs_xent_bwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i]),
    ("tp_mlp_fwd", _i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                        _p, _i64, _p, _i64, _p, _sz, _p]),
    ("tp_mlp_bwd", _i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                        _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _sz, _p]),
    ("tp_mlp_bwd_dgelu", _i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _sz, _p]),
    ("tp_mlp_bwd_dx", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _sz, _p]),
    ("tp_mlp_bwd_dw", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _sz,
                           _p]),
    ("tp_swiglu_fwd", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                           _p, _i64, _p, _i64, _p, _sz, _p]),
    ("tp_swiglu_bwd", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                           _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _sz, _p]),
    ("vocab_parallel_xent_fwd", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _p, _p,
                                     _p, _p, _p, _p, _sz, _p]),
    ("vocab_parallel_xent_fwd_noalloc", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _p,
                                             _p, _p, _p, _p, _p]),
    ("vocab_parallel_xent_bwd", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _p, _p,
                                     _p, _i64, _p, _i64, _p, _sz, _p]),
    ("shard_partial_sum", _i, [_i, _i, _i64, _i, _i, _p, _i64, _p, _p]),
    ("lgs_attn_qkv_fwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    ("tp_attn_qkv_fwd", _i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _sz,
                             _p]),
    ("tp_attn_qkv_bwd", _i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                             _p, _i64, _p]),
    ("tp_attn_out_fwd", _i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p]),
    ("lgs_attn_out_bwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i, _i, _i]),
    ("tp_attn_out_bwd", _i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p, _i64,
                             _p, _i64, _p, _sz, _p]),
    ("shard_reduce_scatter", _i, [_i, _i, _i, _i, _i, _i, _i, _p, _i64, _p, _p]),
    ("shard_all_gather", _i, [_i, _i, _i, _i, _i, _p, _i64, _p, _p]),
    ("shard_reduce_scatter_layernorm", _i,
     [_i, _i, _i, _i, _i, _i, _p, _i64, _p, _p, ctypes.c_float, _p, _p, ctypes.c_float, _p, _p, _p]),
    ("lgs_layernorm_bwd_workspace_bytes", _sz, [_i, _i, _i, _i, _i]),
    ("shard_layernorm_bwd", _i,
     [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, ctypes.c_float, _p, ctypes.c_float, _p, _p, _p, _p, _p, _sz, _p]),
    # include/lgs_testing.h
    ("lgs_test_num_tiles", _i, []),
    ("lgs_test_tile_shape", _i, [_i, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    ("lgs_test_pick_tile", _i, [_i, _i]),
    ("lgs_test_mlp_bwd_plan", _i, [_i, _i, _i, ctypes.POINTER(_i), ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    ("lgs_test_gemm_bf16", _i, [_i, _i, _i, _i, _i, _i, _p, _i64, _p, _i64, _p, _i64, _p]),
    ("lgs_test_xent_rows_bf16", _i, [_i, _i, _i, _p, _i64, _p, _p, _p, _p, _p]),
    ("lgs_test_mfma_rate", _i, [_i, _i, _i, _p, _p, _p, _p]),
    ("lgs_test_debug_build", _i, []),
    ("lgs_test_set_dry_run", _i, [_i]),
    ("lgs_test_debug_checks", ctypes.c_long, []),
    ("lgs_test_debug_span", _i, [_p, _sz, _p, _sz]),
]
LIB_DEBUG_PATH = os.path.join(_HERE, "liblgs_debug.so")


class LgsError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"lgs status {status}: {message}")
        self.status = status


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m logit_gemm_shard_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def version():
    return lib().lgs_version()


def _check(status):
    if status != LGS_OK:
        L = lib()
        raise LgsError(status, f"{L.lgs_status_string(status).decode()}: {L.lgs_last_error().decode()}")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _mat(x):
    """(pointer, leading dimension) of a row-major 2-D tensor view, or (None, 0)."""
    if x is None:
        return None, 0
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return x.data_ptr(), x.stride(0)


def _ptr(x):
    return None if x is None else x.data_ptr()


def _dtype(x):
    try:
        return _DT[x.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {x.dtype}") from None


def _workspace(nbytes, device, given, stream=None):
    """The caller's workspace, or a temporary one from torch's allocator.  A
    temporary one is allocated on the current stream and freed when the
    wrapper returns, while the call's kernels may still be running on
    `stream`: it is recorded on that stream so the allocator does not hand
    it out again before that work is done.  A raw stream handle cannot be
    recorded, so it needs a caller workspace."""
    if nbytes == 0:
        return None, 0
    if given is not None:
        return given.data_ptr(), given.numel() * given.element_size()
    if stream is not None and not isinstance(stream, torch.cuda.Stream):
        raise ValueError("pass workspace= when stream= is a raw handle: a temporary workspace "
                         "cannot be tied to that stream's work")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        ws.record_stream(stream)
    return ws, nbytes


def mlp_fwd_workspace_bytes(b, s, h, ffn, t, dtype, y_given):
    return lib().lgs_mlp_fwd_workspace_bytes(b, s, h, ffn, t, _DT[dtype], int(bool(y_given)))


def mlp_bwd_workspace_bytes(b, s, h, ffn, t, dtype):
    return lib().lgs_mlp_bwd_workspace_bytes(b, s, h, ffn, t, _DT[dtype])


def xent_workspace_bytes(b, s, h, vocab, t, dtype=torch.bfloat16):
    return lib().lgs_xent_workspace_bytes(b, s, h, vocab, t, _DT[dtype])


def tp_mlp_fwd(b, s, h, ffn, t, rank, X, A_i, B_i, Z_i, U_i=None, Y_i=None, act="erf",
               workspace=None, stream=None):
    """One rank's forward shard: U_i = X A_i, Y_i = GeLU(U_i), Z_i = Y_i B_i."""
    L = lib()
    dt = _dtype(X)
    need = L.lgs_mlp_fwd_workspace_bytes(b, s, h, ffn, t, dt, int(Y_i is not None))
    ws, ws_bytes = _workspace(need, X.device, workspace, stream)
    x, ldx = _mat(X)
    a, lda = _mat(A_i)
    bb, ldb = _mat(B_i)
    u, ldu = _mat(U_i)
    y, ldy = _mat(Y_i)
    z, ldz = _mat(Z_i)
    _check(L.tp_mlp_fwd(b, s, h, ffn, t, rank, dt, _ACT[act], x, ldx, a, lda, bb, ldb, u, ldu, y,
                        ldy, z, ldz, _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes,
                        _stream(stream)))
    return Z_i


def tp_mlp_bwd(b, s, h, ffn, t, rank, X, A_i, B_i, U_i, dZ, dX_i, dA_i, dB_i, act="erf",
               workspace=None, stream=None):
    """One rank's backward shard: dX_i (partial), dA_i, dB_i from X, U_i and dZ."""
    L = lib()
    dt = _dtype(X)
    need = L.lgs_mlp_bwd_workspace_bytes(b, s, h, ffn, t, dt)
    ws, ws_bytes = _workspace(need, X.device, workspace, stream)
    args = []
    for m in (X, A_i, B_i, U_i, dZ, dX_i, dA_i, dB_i):
        args.extend(_mat(m))
    _check(L.tp_mlp_bwd(b, s, h, ffn, t, rank, dt, _ACT[act], *args,
                        _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes, _stream(stream)))
    return dX_i, dA_i, dB_i


def swiglu_fwd_workspace_bytes(b, s, h, ffn, t, dtype, y_given):
    return lib().lgs_swiglu_fwd_workspace_bytes(b, s, h, ffn, t, _DT[dtype], int(bool(y_given)))


def swiglu_bwd_workspace_bytes(b, s, h, ffn, t, dtype):
    return lib().lgs_swiglu_bwd_workspace_bytes(b, s, h, ffn, t, _DT[dtype])


def tp_swiglu_fwd(b, s, h, ffn, t, rank, X, Wgu_i, Wd_i, Z_i, GU_i=None, Y_i=None,
                  workspace=None, stream=None):
    """One rank's SwiGLU forward shard: [G | U] = X [W_gate,i | W_up,i],
    Y_i = Swish(G) * U, Z_i = Y_i W_down,i."""
    L = lib()
    dt = _dtype(X)
    need = L.lgs_swiglu_fwd_workspace_bytes(b, s, h, ffn, t, dt, int(Y_i is not None))
    ws, ws_bytes = _workspace(need, X.device, workspace, stream)
    args = []
    for m in (X, Wgu_i, Wd_i, GU_i, Y_i, Z_i):
        args.extend(_mat(m))
    _check(L.tp_swiglu_fwd(b, s, h, ffn, t, rank, dt, *args,
                           _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes, _stream(stream)))
    return Z_i


def tp_swiglu_bwd(b, s, h, ffn, t, rank, X, Wgu_i, Wd_i, GU_i, dZ, dX_i, dWgu_i, dWd_i,
                  workspace=None, stream=None):
    """One rank's SwiGLU backward shard: dX_i (partial), dWgu_i, dWd_i from X,
    the saved [G | U] and dZ."""
    L = lib()
    dt = _dtype(X)
    need = L.lgs_swiglu_bwd_workspace_bytes(b, s, h, ffn, t, dt)
    ws, ws_bytes = _workspace(need, X.device, workspace, stream)
    args = []
    for m in (X, Wgu_i, Wd_i, GU_i, dZ, dX_i, dWgu_i, dWd_i):
        args.extend(_mat(m))
    _check(L.tp_swiglu_bwd(b, s, h, ffn, t, rank, dt, *args,
                           _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes, _stream(stream)))
    return dX_i, dWgu_i, dWd_i


def _ws_given(L, b, s, h, ffn, t, dt, workspace):
    need = L.lgs_mlp_bwd_workspace_bytes(b, s, h, ffn, t, dt)
    if workspace is None:
        raise ValueError("the three-part backward shares one caller-owned workspace")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), need


def tp_mlp_bwd_dgelu(b, s, h, ffn, t, rank, B_i, U_i, dZ, workspace, act="erf", stream=None):
    """dY = dZ B_i^T, dU = dY GeLU'(U_i) and Y = GeLU(U_i) into the workspace."""
    L = lib()
    dt = _dtype(dZ)
    ws, wsb, _ = _ws_given(L, b, s, h, ffn, t, dt, workspace)
    args = []
    for m in (B_i, U_i, dZ):
        args.extend(_mat(m))
    _check(L.tp_mlp_bwd_dgelu(b, s, h, ffn, t, rank, dt, _ACT[act], *args, ws, wsb, _stream(stream)))


def tp_mlp_bwd_dx(b, s, h, ffn, t, rank, A_i, dX_i, workspace, stream=None):
    """dX_i = dU A_i^T from the workspace (after tp_mlp_bwd_dgelu)."""
    L = lib()
    dt = _dtype(A_i)
    ws, wsb, _ = _ws_given(L, b, s, h, ffn, t, dt, workspace)
    a, lda = _mat(A_i)
    x, ldx = _mat(dX_i)
    _check(L.tp_mlp_bwd_dx(b, s, h, ffn, t, rank, dt, a, lda, x, ldx, ws, wsb, _stream(stream)))
    return dX_i


def tp_mlp_bwd_dw(b, s, h, ffn, t, rank, X, dZ, dA_i, dB_i, workspace, stream=None):
    """dB_i = Y^T dZ and dA_i = X^T dU from the workspace (after tp_mlp_bwd_dgelu)."""
    L = lib()
    dt = _dtype(X)
    ws, wsb, _ = _ws_given(L, b, s, h, ffn, t, dt, workspace)
    args = []
    for m in (X, dZ, dA_i, dB_i):
        args.extend(_mat(m))
    _check(L.tp_mlp_bwd_dw(b, s, h, ffn, t, rank, dt, *args, ws, wsb, _stream(stream)))
    return dA_i, dB_i


def vocab_parallel_xent_fwd(b, s, h, vocab, t, rank, H, E_r, targets, m_r, l_r, tgt_r,
                            argmax_r=None, loss=None, workspace=None, stream=None):
    """One rank's fused logit GEMM + CE partials over its vocabulary slice."""
    L = lib()
    dt = _dtype(H)
    need = L.lgs_xent_workspace_bytes(b, s, h, vocab, t, dt)
    ws, ws_bytes = _workspace(need, H.device, workspace, stream)
    hh, ldh = _mat(H)
    e, lde = _mat(E_r)
    _check(L.vocab_parallel_xent_fwd(b, s, h, vocab, t, rank, dt, hh, ldh, e, lde, _ptr(targets),
                                     _ptr(m_r), _ptr(l_r), _ptr(tgt_r), _ptr(argmax_r), _ptr(loss),
                                     _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes,
                                     _stream(stream)))
    return m_r, l_r, tgt_r


XENT_NOALLOC_SCRATCH_BYTES = 16 << 20  # LGS_XENT_NOALLOC_SCRATCH_BYTES


def vocab_parallel_xent_fwd_noalloc(b, s, h, vocab, t, rank, H, E_r, targets, m_r, l_r, tgt_r,
                                    argmax_r=None, loss=None, stream=None):
    """vocab_parallel_xent_fwd with the slab partials in the library's static
    device scratch: no workspace, nothing allocated (calls that overlap on one
    device race)."""
    L = lib()
    hh, ldh = _mat(H)
    e, lde = _mat(E_r)
    _check(L.vocab_parallel_xent_fwd_noalloc(b, s, h, vocab, t, rank, _dtype(H), hh, ldh, e, lde,
                                             _ptr(targets), _ptr(m_r), _ptr(l_r), _ptr(tgt_r),
                                             _ptr(argmax_r), _ptr(loss), _stream(stream)))
    return m_r, l_r, tgt_r


def xent_bwd_workspace_bytes(b, s, h, vocab, t, dtype=torch.bfloat16):
    return lib().lgs_xent_bwd_workspace_bytes(b, s, h, vocab, t, _DT[dtype])


def vocab_parallel_xent_bwd(b, s, h, vocab, t, rank, H, E_r, targets, lse, dH_r, dE_r, dloss=None,
                            workspace=None, stream=None):
    """One rank's CE backward: dH_r (partial) and dE_r from the merged lse."""
    L = lib()
    dt = _dtype(H)
    need = L.lgs_xent_bwd_workspace_bytes(b, s, h, vocab, t, dt)
    ws, ws_bytes = _workspace(need, H.device, workspace, stream)
    hh, ldh = _mat(H)
    e, lde = _mat(E_r)
    dh, lddh = _mat(dH_r)
    de, ldde = _mat(dE_r)
    _check(L.vocab_parallel_xent_bwd(b, s, h, vocab, t, rank, dt, hh, ldh, e, lde, _ptr(targets),
                                     _ptr(lse), _ptr(dloss), dh, lddh, de, ldde,
                                     _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes,
                                     _stream(stream)))
    return dH_r, dE_r


def shard_partial_sum(op, t, n, parts, part_stride, out, stream=None):
    """SUM: out = sum_r parts[r]; XENT: out = per-token loss from [t][3][n]
    partials; XENT_LSE ("xent_lse"): the per-token log-sum-exp alone."""
    L = lib()
    opc = {"sum": LGS_REDUCE_SUM, "xent": LGS_REDUCE_XENT,
           "xent_lse": LGS_REDUCE_XENT_LSE}[op] if isinstance(op, str) else op
    _check(L.shard_partial_sum(opc, t, n, _dtype(parts), _dtype(out), parts.data_ptr(), part_stride,
                               out.data_ptr(), _stream(stream)))
    return out


def attn_qkv_fwd_workspace_bytes(b, s, h, n_q, n_kv, d, t, dtype=torch.bfloat16):
    return lib().lgs_attn_qkv_fwd_workspace_bytes(b, s, h, n_q, n_kv, d, t, _DT[dtype])


def tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, rank, X, Wqkv_i, QKV_i, workspace=None, split=True,
                    stream=None):
    """QKV_i = X [W_Q^i | W_K^i | W_V^i] (rank's heads).  With split=False no
    workspace is passed (the product runs unsplit)."""
    L = lib()
    dt = _dtype(X)
    need = L.lgs_attn_qkv_fwd_workspace_bytes(b, s, h, n_q, n_kv, d, t, dt) if split else 0
    ws, ws_bytes = _workspace(need, X.device, workspace, stream)
    args = []
    for m in (X, Wqkv_i, QKV_i):
        args.extend(_mat(m))
    _check(L.tp_attn_qkv_fwd(b, s, h, n_q, n_kv, d, t, rank, dt, *args,
                             _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes, _stream(stream)))
    return QKV_i


def tp_attn_qkv_bwd(b, s, h, n_q, n_kv, d, t, rank, X, Wqkv_i, dQKV_i, dX_i, dWqkv_i, stream=None):
    """dX_i = dQKV_i Wqkv_i^T (a partial), dWqkv_i = X^T dQKV_i."""
    args = []
    for m in (X, Wqkv_i, dQKV_i, dX_i, dWqkv_i):
        args.extend(_mat(m))
    _check(lib().tp_attn_qkv_bwd(b, s, h, n_q, n_kv, d, t, rank, _dtype(X), *args, _stream(stream)))
    return dX_i, dWqkv_i


def tp_attn_out_fwd(b, s, h, n_q, d, t, rank, A_i, Wo_i, Z_i, stream=None):
    """The partial Z_i = A_i W_O^i."""
    args = []
    for m in (A_i, Wo_i, Z_i):
        args.extend(_mat(m))
    _check(lib().tp_attn_out_fwd(b, s, h, n_q, d, t, rank, _dtype(A_i), *args, _stream(stream)))
    return Z_i


def attn_out_bwd_workspace_bytes(b, s, h, n_q, d, t, dtype=torch.bfloat16):
    return lib().lgs_attn_out_bwd_workspace_bytes(b, s, h, n_q, d, t, _DT[dtype])


def tp_attn_out_bwd(b, s, h, n_q, d, t, rank, A_i, Wo_i, dZ, dA_i, dWo_i, workspace=None, split=True,
                    stream=None):
    """dA_i = dZ W_O^i^T, dWo_i = A_i^T dZ.  With split=False no workspace is
    passed (dA_i runs unsplit)."""
    L = lib()
    dt = _dtype(A_i)
    need = L.lgs_attn_out_bwd_workspace_bytes(b, s, h, n_q, d, t, dt) if split else 0
    ws, ws_bytes = _workspace(need, A_i.device, workspace, stream)
    args = []
    for m in (A_i, Wo_i, dZ, dA_i, dWo_i):
        args.extend(_mat(m))
    _check(L.tp_attn_out_bwd(b, s, h, n_q, d, t, rank, dt, *args,
                             _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes, _stream(stream)))
    return dA_i, dWo_i


def shard_reduce_scatter(t, rank, s, b, h, parts, part_stride, out, stream=None):
    """Rank's (s/t)*b rows of sum_i parts[i] (each part a dense [s*b, h])."""
    _check(lib().shard_reduce_scatter(t, rank, s, b, h, _dtype(parts), _dtype(out), parts.data_ptr(),
                                      part_stride, out.data_ptr(), _stream(stream)))
    return out


def shard_reduce_scatter_layernorm(t, rank, s, b, h, parts, part_stride, residual, gamma, beta, hs, y,
                                   keep=None, keep_scale=1.0, eps=1e-5, stream=None):
    """Rank's sequence-parallel region: hs = residual + dropout(rank's rows of
    sum_i parts[i]) and y = LayerNorm(hs) (bf16; keep a uint8 mask or None)."""
    _check(lib().shard_reduce_scatter_layernorm(t, rank, s, b, h, _dtype(parts), parts.data_ptr(), part_stride,
                                                residual.data_ptr(), None if keep is None else keep.data_ptr(),
                                                keep_scale, gamma.data_ptr(), beta.data_ptr(), eps, hs.data_ptr(),
                                                y.data_ptr(), _stream(stream)))
    return hs, y


def layernorm_bwd_workspace_bytes(t, s, b, h, dtype=torch.bfloat16):
    return lib().lgs_layernorm_bwd_workspace_bytes(t, s, b, h, _DT[dtype])


def shard_layernorm_bwd(t, rank, s, b, h, hs, dy, gamma, g, dz, dgamma, dbeta, dhs=None, keep=None,
                        keep_scale=1.0, eps=1e-5, workspace=None, stream=None):
    """Backward of the sequence-parallel region on the rank's rows: g (the
    gradient of hs and of the residual), dz (the masked g) and the rows'
    dgamma, dbeta (fp32)."""
    L = lib()
    dt = _dtype(hs)
    need = L.lgs_layernorm_bwd_workspace_bytes(t, s, b, h, dt)
    ws, ws_bytes = _workspace(need, hs.device, workspace, stream)
    _check(L.shard_layernorm_bwd(t, rank, s, b, h, dt, hs.data_ptr(), dy.data_ptr(),
                                 None if dhs is None else dhs.data_ptr(), None if keep is None else keep.data_ptr(),
                                 keep_scale, gamma.data_ptr(), eps, g.data_ptr(), dz.data_ptr(), dgamma.data_ptr(),
                                 dbeta.data_ptr(), _ptr(ws) if isinstance(ws, torch.Tensor) else ws, ws_bytes,
                                 _stream(stream)))
    return g, dz, dgamma, dbeta


def shard_all_gather(t, s, b, h, shards, shard_stride, out, stream=None):
    """The dense [s*b, h] tensor from t chunks of (s/t)*b rows, rank order."""
    if shards.dtype != out.dtype:
        raise ValueError("the all-gather copies: shards and out share a dtype")
    _check(lib().shard_all_gather(t, s, b, h, _dtype(out), shards.data_ptr(), shard_stride, out.data_ptr(),
                                  _stream(stream)))
    return out


def tile_shapes():
    """[(bm, bn)] of the GEMM core's block tiles, by tile id."""
    L = lib()
    out = []
    for t in range(L.lgs_test_num_tiles()):
        bm, bn = ctypes.c_int(), ctypes.c_int()
        L.lgs_test_tile_shape(t, ctypes.byref(bm), ctypes.byref(bn))
        out.append((bm.value, bn.value))
    return out


def pick_tile(M, N):
    return lib().lgs_test_pick_tile(M, N)


def mlp_bwd_plan(M, h, f):
    """(parts, tokens per part, tail) of the bf16 backward's weight
    gradients: (1, M, 0) when tp_mlp_bwd does not split them over the
    tokens; tail = 0 when it splits every dB and dA tile, else the number of
    (last) dA tiles it splits, dB then being unsplit."""
    parts, kchunk, tail = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    if lib().lgs_test_mlp_bwd_plan(M, h, f, ctypes.byref(parts), ctypes.byref(kchunk), ctypes.byref(tail)) != 0:
        raise ValueError("sizes must be positive")
    return parts.value, kchunk.value, tail.value


def gemm_bf16(A, B, C, a_kmajor=True, b_kmajor=False, tile=-1, stream=None):
    """C = A B through the GEMM core (testing interface).  A is [M, K] if
    a_kmajor else [K, M]; B is [K, N] if not b_kmajor else [N, K]."""
    a, lda = _mat(A)
    b, ldb = _mat(B)
    c, ldc = _mat(C)
    M, N = C.shape
    K = A.shape[1] if a_kmajor else A.shape[0]
    _check(lib().lgs_test_gemm_bf16(tile, int(a_kmajor), int(b_kmajor), M, N, K, a, lda, b, ldb, c,
                                    ldc, _stream(stream)))
    return C


def xent_rows_bf16(Z, targets, vocab_start, m, l, T, stream=None):
    """Slice partials (m, l, T) from materialised bf16 logits Z [M, Vr]
    (testing interface: the streaming form of the fused CE's reductions)."""
    z, ldz = _mat(Z)
    M, Vr = Z.shape
    _check(lib().lgs_test_xent_rows_bf16(M, Vr, vocab_start, z, ldz, targets.data_ptr(), m.data_ptr(),
                                         l.data_ptr(), T.data_ptr(), _stream(stream)))
    return m, l, T


def mfma_rate(blocks, waves, iters8, ops, out, clocks, stream=None):
    """The matrix cores' rate probe (testing interface): `blocks` workgroups of
    `waves` waves, 8 chains of 8 * iters8 MFMAs each on the operand pairs in
    ops (bf16 [16, 64, 8]); accumulators to out (float32, blocks * waves *
    8192), per-wave shader-clock and reference-tick counts to clocks (int64,
    2 * blocks * waves)."""
    if ops.dtype != torch.bfloat16 or ops.numel() != 16 * 64 * 8:
        raise ValueError("ops must be bf16 with 16 * 64 * 8 elements")
    if out.dtype != torch.float32 or out.numel() < blocks * waves * 8192:
        raise ValueError("out must be float32 with blocks * waves * 8192 elements")
    if clocks.dtype != torch.int64 or clocks.numel() < 2 * blocks * waves:
        raise ValueError("clocks must be int64 with 2 * blocks * waves elements")
    _check(lib().lgs_test_mfma_rate(blocks, waves, iters8, ops.data_ptr(), out.data_ptr(), clocks.data_ptr(),
                                    _stream(stream)))
    return out, clocks


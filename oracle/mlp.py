"""fp64 oracle: the GeLU MLP block split column-then-row over ``t`` ranks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Notation follows "Tensor Parallelism and Pipeline Parallelism: Mathematical
Foundations of Megatron-LM 1D Slicing, ..." (llms.blog), sections
"Column-Parallel Linear Layer" and "Row-Parallel Linear Layer", and the
lecture "Cutting a Model Into Pieces" (learn.kartikeya.me, lecture 3),
section "Megatron-LM: cutting inside the layer":

    U   = X A            X in R^{M x h},  A in R^{h x ffn}
    Y   = GeLU(U)        elementwise
    Z   = Y B            B in R^{ffn x h}

    A = [A_1 ... A_t]            (column blocks, A_i in R^{h x ffn/t})
    B = [B_1; ...; B_t]          (row blocks,    B_i in R^{ffn/t x h})
    Z_i = GeLU(X A_i) B_i,   Z = sum_i Z_i

Rows of X are tokens (the pages' (s, b, h) activation flattened to M = b*s
rows; every operation here is per token, so the order does not matter).
There is no bias: the pages' equations have none and their
ColumnParallelLinear defaults to ``bias=False``.

The backward pass is the chain rule through those equations, which is what
the conjugate operators f / g of the "Conjugate Communication Operators"
section imply: dZ reaches every rank unchanged (g* is the identity) and each
rank's dX_i is a partial that has to be summed (f* is an all-reduce).
"""

import numpy as np
from scipy.special import erf

_SQRT_2 = np.sqrt(2.0)
_SQRT_2PI = np.sqrt(2.0 * np.pi)
_TANH_C = np.sqrt(2.0 / np.pi)
_TANH_K = 0.044715

VARIANTS = ("erf", "tanh")


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def gelu(u, variant="erf"):
    """GeLU(u).

    ``erf``:  the exact form u * Phi(u) = u/2 * (1 + erf(u / sqrt 2)), Phi the
              standard normal CDF (the GeLU of Hendrycks & Gimpel, which the
              pages name as the nonlinearity between the two GEMMs).
    ``tanh``: the published approximation
              u/2 * (1 + tanh(sqrt(2/pi) * (u + 0.044715 u^3))).
    """
    u = _f64(u)
    if variant == "erf":
        return 0.5 * u * (1.0 + erf(u / _SQRT_2))
    if variant == "tanh":
        return 0.5 * u * (1.0 + np.tanh(_TANH_C * (u + _TANH_K * u ** 3)))
    raise ValueError(f"unknown GeLU variant {variant!r}")


def gelu_grad(u, variant="erf"):
    """d GeLU / du.

    ``erf``:  Phi(u) + u * phi(u), phi(u) = exp(-u^2/2) / sqrt(2 pi).
    ``tanh``: with a = sqrt(2/pi)(u + 0.044715 u^3), s = tanh(a):
              (1 + s)/2 + u/2 * (1 - s^2) * sqrt(2/pi) * (1 + 3*0.044715 u^2).
    """
    u = _f64(u)
    if variant == "erf":
        return 0.5 * (1.0 + erf(u / _SQRT_2)) + u * np.exp(-0.5 * u * u) / _SQRT_2PI
    if variant == "tanh":
        s = np.tanh(_TANH_C * (u + _TANH_K * u ** 3))
        return 0.5 * (1.0 + s) + 0.5 * u * (1.0 - s * s) * _TANH_C * (1.0 + 3.0 * _TANH_K * u * u)
    raise ValueError(f"unknown GeLU variant {variant!r}")


def column_shard(A, t, i):
    """A_i: the i-th of t column blocks of A (h x ffn/t)."""
    A = _f64(A)
    ffn = A.shape[1]
    if ffn % t:
        raise ValueError("ffn must divide by t")
    f = ffn // t
    return A[:, i * f:(i + 1) * f]


def row_shard(B, t, i):
    """B_i: the i-th of t row blocks of B (ffn/t x h)."""
    B = _f64(B)
    ffn = B.shape[0]
    if ffn % t:
        raise ValueError("ffn must divide by t")
    f = ffn // t
    return B[i * f:(i + 1) * f, :]


def mlp_forward(X, A, B, variant="erf"):
    """The unsplit block: U = X A, Y = GeLU(U), Z = Y B."""
    X, A, B = _f64(X), _f64(A), _f64(B)
    U = X @ A
    Y = gelu(U, variant)
    Z = Y @ B
    return U, Y, Z


def shard_forward(X, A_i, B_i, variant="erf"):
    """One rank's shard: U_i = X A_i, Y_i = GeLU(U_i), Z_i = Y_i B_i (a partial)."""
    X, A_i, B_i = _f64(X), _f64(A_i), _f64(B_i)
    U_i = X @ A_i
    Y_i = gelu(U_i, variant)
    Z_i = Y_i @ B_i
    return U_i, Y_i, Z_i


def shard_backward(X, A_i, B_i, U_i, dZ, variant="erf"):
    """One rank's backward, given the saved X and pre-GeLU U_i and the
    incoming dZ (identical on every rank).

        dY_i = dZ B_i^T
        dU_i = dY_i * GeLU'(U_i)          (elementwise)
        Y_i  = GeLU(U_i)                  (recomputed from the saved U_i)
        dB_i = Y_i^T dZ
        dA_i = X^T dU_i
        dX_i = dU_i A_i^T                 (a partial: dX = sum_i dX_i)
    """
    X, A_i, B_i, U_i, dZ = _f64(X), _f64(A_i), _f64(B_i), _f64(U_i), _f64(dZ)
    dY_i = dZ @ B_i.T
    dU_i = dY_i * gelu_grad(U_i, variant)
    Y_i = gelu(U_i, variant)
    dB_i = Y_i.T @ dZ
    dA_i = X.T @ dU_i
    dX_i = dU_i @ A_i.T
    return {"dY": dY_i, "dU": dU_i, "Y": Y_i, "dA": dA_i, "dB": dB_i, "dX": dX_i}


def mlp_backward(X, A, B, dZ, variant="erf"):
    """Backward of the unsplit block (the t = 1 case of ``shard_backward``)."""
    X, A = _f64(X), _f64(A)
    U = X @ A
    return shard_backward(X, A, B, U, dZ, variant)


def partial_sum(parts):
    """Sum of t partials in ascending rank order: the all-reduce of the
    forward g (row-parallel exit) and of the backward f* (column-parallel
    entry), computed on one device."""
    parts = [_f64(p) for p in parts]
    out = np.zeros_like(parts[0])
    for p in parts:
        out = out + p
    return out

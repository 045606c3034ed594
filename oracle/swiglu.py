"""fp64 oracle: the SwiGLU MLP block split column-then-row over ``t`` ranks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The block of Llama-3 as the mohashari.github.io page on tensor parallelism for
70B models states it, section "The MLP Block": three linear layers, gate,
up and down,

    MLP(X) = (Swish(X W_gate) * (X W_up)) W_down        (* elementwise)

with W_gate and W_up split by columns and W_down by rows across the TP group,
so that rank i computes

    G_i = X W_gate,i,   U_i = X W_up,i,   Y_i = Swish(G_i) * U_i,
    Z_i = Y_i W_down,i,                    Z = sum_i Z_i.

Reading: Swish is the plain Swish of the SiLU form, Swish(g) = g * sigmoid(g)
(the page gives no beta; beta = 1 is the form Llama uses), no biases.  Shard
layout: rank i's gate and up blocks are the column blocks of the two weights;
the library takes them side by side as one [h, 2 f_i] matrix
[W_gate,i | W_up,i].  The backward is the chain rule through the equations;
as in the GeLU block, dZ reaches every rank unchanged and dX_i is a partial.
"""

import numpy as np

from .mlp import column_shard, row_shard  # noqa: F401  (same splits as the GeLU block)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(g):
    """1 / (1 + exp(-g)), evaluated without overflow for either sign."""
    g = _f64(g)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def swish(g):
    """Swish(g) = g * sigmoid(g)."""
    g = _f64(g)
    return g * sigmoid(g)


def swish_grad(g):
    """d Swish / dg = sigmoid(g) + g * sigmoid(g) * (1 - sigmoid(g))."""
    g = _f64(g)
    s = sigmoid(g)
    return s + g * s * (1.0 - s)


def swiglu_forward(X, Wg, Wu, Wd):
    """The unsplit block: G = X Wg, U = X Wu, Y = Swish(G) * U, Z = Y Wd."""
    X, Wg, Wu, Wd = _f64(X), _f64(Wg), _f64(Wu), _f64(Wd)
    G = X @ Wg
    U = X @ Wu
    Y = swish(G) * U
    return G, U, Y, Y @ Wd


def shard_forward(X, Wg_i, Wu_i, Wd_i):
    """One rank's shard: G_i, U_i, Y_i and the partial Z_i."""
    return swiglu_forward(X, Wg_i, Wu_i, Wd_i)


def shard_backward(X, Wg_i, Wu_i, Wd_i, G_i, U_i, dZ):
    """One rank's backward, given the saved X, the pre-activations G_i, U_i
    and the incoming dZ:

        dY_i  = dZ Wd_i^T
        dG_i  = dY_i * U_i * Swish'(G_i)
        dU_i  = dY_i * Swish(G_i)
        Y_i   = Swish(G_i) * U_i               (recomputed)
        dWd_i = Y_i^T dZ
        dWg_i = X^T dG_i,   dWu_i = X^T dU_i
        dX_i  = dG_i Wg_i^T + dU_i Wu_i^T      (a partial: dX = sum_i dX_i)
    """
    X, Wg_i, Wu_i, Wd_i = _f64(X), _f64(Wg_i), _f64(Wu_i), _f64(Wd_i)
    G_i, U_i, dZ = _f64(G_i), _f64(U_i), _f64(dZ)
    dY = dZ @ Wd_i.T
    dG = dY * U_i * swish_grad(G_i)
    dU = dY * swish(G_i)
    Y = swish(G_i) * U_i
    return {"dY": dY, "dG": dG, "dU": dU, "Y": Y, "dWd": Y.T @ dZ, "dWg": X.T @ dG,
            "dWu": X.T @ dU, "dX": dG @ Wg_i.T + dU @ Wu_i.T}


def swiglu_backward(X, Wg, Wu, Wd, dZ):
    """Backward of the unsplit block (the t = 1 case of ``shard_backward``)."""
    X, Wg, Wu = _f64(X), _f64(Wg), _f64(Wu)
    return shard_backward(X, Wg, Wu, Wd, X @ Wg, X @ Wu, dZ)

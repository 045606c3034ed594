"""fp64 oracle: the sequence-parallel exit and entry around the row-parallel GEMM.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Tensor Parallelism and Pipeline Parallelism: Mathematical Foundations of
Megatron-LM ..." (llms.blog), section "Sequence Parallelism", "Splitting
All-Reduce into Reduce-Scatter and All-Gather": the row-parallel exit's
all-reduce becomes a reduce-scatter that sums the t partials and leaves each
rank the (s/t, b, h) chunk of the result along the sequence; LayerNorm,
dropout and residual run on that chunk; an all-gather rebuilds the (s, b, h)
tensor before the next column-parallel GEMM.

Layout reading: activations are the pages' (s, b, h) tensor flattened with s
outermost, so row k = s_idx * b + b_idx of an [s*b, h] matrix, and rank r's
chunk is the contiguous rows [r*(s/t)*b, (r+1)*(s/t)*b).  s must divide by t.
"""

import numpy as np

from .mlp import partial_sum


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def chunk_rows(s, b, t, r):
    """[start, stop) of rank r's rows of the flattened (s, b) token axis."""
    if s % t:
        raise ValueError("the sequence length must divide by t")
    n = (s // t) * b
    return r * n, (r + 1) * n


def reduce_scatter(parts, s, b, t, r):
    """Rank r's chunk of sum_i parts[i], each part [s*b, h]."""
    a, z = chunk_rows(s, b, t, r)
    return partial_sum([_f64(p)[a:z] for p in parts])


def all_gather(shards, s, b, t):
    """The [s*b, h] tensor from the t ranks' chunks, rank order along s."""
    shards = [_f64(x) for x in shards]
    if len(shards) != t or any(x.shape[0] != (s // t) * b for x in shards):
        raise ValueError("expected t chunks of (s/t)*b rows")
    return np.concatenate(shards, axis=0)


def comm_volume(kind, t, n):
    """Elements each rank sends in a ring collective over a tensor of n
    elements: (t-1)/t n for a reduce-scatter or an all-gather, twice that for
    the all-reduce they compose (the section's volume identity)."""
    one = (t - 1) / t * n
    return {"reduce_scatter": one, "all_gather": one, "all_reduce": 2 * one}[kind]


def layernorm(x, gamma, beta, eps=1e-5):
    """Per token row of x [n, h]: (x - mean) / sqrt(var + eps) * gamma + beta,
    with the mean and the (biased, 1/h) variance taken over the h features
    and gamma, beta [h] per feature.  The section says only that LayerNorm
    works on each token independently along h; this is the usual definition."""
    x = _f64(x)
    mean = x.mean(axis=1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * _f64(gamma)[None, :] + _f64(beta)[None, :]


def exit_region(parts, s, b, t, r, residual, gamma, beta, eps=1e-5, keep=None, keep_scale=1.0):
    """Rank r's sequence-parallel region after the row-parallel exit, on its
    (s/t, b, h) chunk (the section's "Normalized Execution": LayerNorm,
    residual additions and dropout run locally on the chunk):

      z   = reduce_scatter(parts)                   rank r's rows of sum_i Z_i
      d   = z * keep * keep_scale  (keep given)     dropout with a given keep mask
            z                      (keep None)      (no dropout)
      hs  = residual + d                            the residual stream's chunk
      y   = layernorm(hs, gamma, beta, eps)         the next sub-layer's input

    Readings: dropout acts on the block's output before the residual add and
    LayerNorm follows the add (the next sub-layer's norm, as in Megatron's
    pre-norm blocks); the keep mask is an input (the pages give no random
    number generator), keep_scale normally 1 / (1 - p).  Returns (hs, y)."""
    z = reduce_scatter(parts, s, b, t, r)
    d = z if keep is None else z * (np.asarray(keep) != 0) * float(keep_scale)
    hs = _f64(residual) + d
    return hs, layernorm(hs, gamma, beta, eps)


def layernorm_backward(x, gamma, dy, eps=1e-5):
    """Gradients of y = layernorm(x, gamma, beta, eps) for the upstream dy
    (the chain rule through the per-row definition above):

      xhat  = (x - mean) / sqrt(var + eps),  dxhat = dy * gamma
      dx    = (dxhat - mean_h(dxhat) - xhat * mean_h(dxhat * xhat)) / sqrt(var + eps)
      dgamma = sum over rows of dy * xhat,   dbeta = sum over rows of dy

    Returns (dx, dgamma, dbeta)."""
    x, dy = _f64(x), _f64(dy)
    mean = x.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mean) ** 2).mean(axis=1, keepdims=True) + eps)
    xhat = (x - mean) * rstd
    dxhat = dy * _f64(gamma)[None, :]
    dx = (dxhat - dxhat.mean(axis=1, keepdims=True) - xhat * (dxhat * xhat).mean(axis=1, keepdims=True)) * rstd
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def exit_region_backward(hs, gamma, dy, dhs=None, eps=1e-5, keep=None, keep_scale=1.0):
    """Backward of exit_region on rank r's chunk, from the gradient dy of its
    LayerNorm output y and the gradient dhs that later layers send back along
    the residual stream (None: none):

      g      = dhs + dx of LayerNorm at hs     the gradient of hs, which is also
                                               the residual input's gradient
      dz     = g * keep * keep_scale  (or g)   the gradient of the rank's rows of
                                               sum_i Z_i (the all-gather's input
                                               in the backward)
      dgamma, dbeta                            the rank's sums over its rows (a
                                               partial: the ranks' sums add up)

    Returns {"g", "dz", "dgamma", "dbeta"}."""
    dx, dgamma, dbeta = layernorm_backward(hs, gamma, dy, eps)
    g = dx if dhs is None else _f64(dhs) + dx
    dz = g if keep is None else g * (np.asarray(keep) != 0) * float(keep_scale)
    return {"g": g, "dz": dz, "dgamma": dgamma, "dbeta": dbeta}

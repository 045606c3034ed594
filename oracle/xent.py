"""fp64 oracle: softmax cross-entropy over a vocabulary split across ranks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"LIT-022: Megatron-LM: Training Multi-Billion Parameter Language Models Using
Model Parallelism" (dmarx.github.io anthology), "Key takeaways": the parallel
logit GEMM is fused into the cross-entropy so that ranks exchange O(b*s)
numbers instead of all-gathering the b*s*v logits; the vocabulary is padded
(50,257 -> 51,200) so each rank's slice is a multiple of 128.

Plain definitions used here:

* logits  z = H E^T,  H in R^{M x h} (hidden rows, one per token),
  E in R^{V x h} (the output embedding, one row per vocabulary entry).
* per-token loss (natural log, no mean, no smoothing):
      loss_k = ln sum_j exp(z_kj) - z_{k, y_k}
* rank r owns the contiguous vocabulary rows [r*V/t, (r+1)*V/t).  Its
  per-token partials are the local max m_r, the sum of exponentials taken
  relative to that local max l_r, and the target logit T_r (exactly +0.0 when
  the target is not in the slice).  The merge is the log-sum-exp identity
      M* = max_r m_r,  L* = sum_r l_r exp(m_r - M*),
      loss = M* + ln L* - sum_r T_r
  which equals the full-logit loss in exact arithmetic.  (The pages state only
  the O(b*s) exchange; the partials and this merge are the plain reading.)

The backward is the plain derivative of the summed per-token losses (the page
states only the forward).  With upstream weights w_k (dloss, 1 by default),
p_kj = exp(z_kj - lse_k), lse_k = ln sum_j exp(z_kj):

      G = (p - onehot(y)) * w[:, None],   dH = G E,   dE = G^T H.

Split by vocabulary, rank r needs only the merged lse_k = M* + ln L* (one
more O(b*s) quantity from the same exchange): G_r = (exp(z_r - lse) -
onehot_r) * w, its dH_r = G_r E_r is a partial (dH = sum_r dH_r) and its
dE_r = G_r^T H is rank r's rows of dE.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def naive_loss(H, E, y, chunk=1024):
    """Full-logit cross-entropy per token, computed chunk by chunk of tokens
    (a memory bound only; each token's loss is independent), with the row
    max subtracted before exponentiating."""
    H, E = _f64(H), _f64(E)
    y = np.asarray(y, dtype=np.int64)
    M = H.shape[0]
    out = np.empty(M, dtype=np.float64)
    for s in range(0, M, chunk):
        z = H[s:s + chunk] @ E.T
        mx = z.max(axis=1)
        lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
        out[s:s + chunk] = lse - z[np.arange(z.shape[0]), y[s:s + chunk]]
    return out


def vocab_slice(V, t, r):
    """[start, stop) of rank r's contiguous slice of a V-row vocabulary."""
    if V % t:
        raise ValueError("vocabulary size must divide by t")
    n = V // t
    return r * n, (r + 1) * n


def shard_partials(H, E_r, y, vocab_start):
    """Rank partials for the slice E_r = E[vocab_start : vocab_start + V_r].

    Returns (m_r, l_r, T_r, argmax_r):
      m_r      = max_j z_kj over the slice
      l_r      = sum_j exp(z_kj - m_r)
      T_r      = z_{k, y_k - vocab_start} if the target is in the slice, else +0.0
      argmax_r = global vocabulary id of the slice's largest logit (lowest id
                 among exact ties)
    """
    return slice_partials(_f64(H) @ _f64(E_r).T, y, vocab_start)


def slice_partials(z, y, vocab_start):
    """The same partials from a slice's logits z [M, V_r] directly."""
    z = _f64(z)
    y = np.asarray(y, dtype=np.int64)
    Vr = z.shape[1]
    m = z.max(axis=1)
    l = np.exp(z - m[:, None]).sum(axis=1)
    local = y - vocab_start
    own = (local >= 0) & (local < Vr)
    T = np.zeros(z.shape[0], dtype=np.float64)
    rows = np.nonzero(own)[0]
    T[rows] = z[rows, local[rows]]
    am = vocab_start + np.argmax(z, axis=1)  # numpy returns the first maximum
    return m, l, T, am


def merge(m, l, T):
    """Per-token loss from the t ranks' partials, arrays of shape [t, M]."""
    m, l, T = _f64(m), _f64(l), _f64(T)
    Mx = m.max(axis=0)
    L = (l * np.exp(m - Mx[None, :])).sum(axis=0)
    return Mx + np.log(L) - T.sum(axis=0)


def merge_argmax(m, am):
    """Global argmax from per-rank maxima m [t, M] and ids am [t, M]: the
    rank holding the largest maximum wins; on equal maxima the lower rank
    (which owns the lower ids) wins."""
    m = _f64(m)
    am = np.asarray(am)
    r = np.argmax(m, axis=0)
    return am[r, np.arange(m.shape[1])]


def vocab_parallel_loss(H, E, y, t):
    """The fused form end to end: every rank's partials, then the merge."""
    V = _f64(E).shape[0]
    parts = [shard_partials(H, E[a:b], y, a) for a, b in (vocab_slice(V, t, r) for r in range(t))]
    m = np.stack([p[0] for p in parts])
    l = np.stack([p[1] for p in parts])
    T = np.stack([p[2] for p in parts])
    return merge(m, l, T)


def merge_lse(m, l):
    """Per-token log-sum-exp over the whole vocabulary from the ranks'
    partials m, l [t, M]: M* + ln L*."""
    m, l = _f64(m), _f64(l)
    Mx = m.max(axis=0)
    return Mx + np.log((l * np.exp(m - Mx[None, :])).sum(axis=0))


def _weights(dloss, M):
    return np.ones(M) if dloss is None else _f64(dloss)


def xent_backward(H, E, y, dloss=None):
    """Gradient of sum_k dloss_k * loss_k with respect to H and E (the whole
    vocabulary): returns {"G", "dH", "dE"}."""
    H, E = _f64(H), _f64(E)
    y = np.asarray(y, dtype=np.int64)
    z = H @ E.T
    mx = z.max(axis=1)
    p = np.exp(z - mx[:, None])
    p /= p.sum(axis=1)[:, None]
    G = p
    G[np.arange(z.shape[0]), y] -= 1.0
    G *= _weights(dloss, z.shape[0])[:, None]
    return {"G": G, "dH": G @ E, "dE": G.T @ H}


def shard_backward(H, E_r, y, vocab_start, lse, dloss=None):
    """Rank r's share for the slice E_r = E[vocab_start : vocab_start + V_r],
    given the merged per-token lse: returns {"G", "dH", "dE"} with
    G_r = (exp(z_r - lse) - onehot_r) * dloss, dH_r = G_r E_r (a partial),
    dE_r = G_r^T H (rank r's rows of dE)."""
    H, E_r = _f64(H), _f64(E_r)
    y = np.asarray(y, dtype=np.int64)
    z = H @ E_r.T
    G = np.exp(z - _f64(lse)[:, None])
    local = y - vocab_start
    rows = np.nonzero((local >= 0) & (local < z.shape[1]))[0]
    G[rows, local[rows]] -= 1.0
    G *= _weights(dloss, z.shape[0])[:, None]
    return {"G": G, "dH": G @ E_r, "dE": G.T @ H}

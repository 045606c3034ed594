"""fp64 oracle: the attention block's projections split across ``t`` ranks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Tensor Parallelism and Pipeline Parallelism: Mathematical Foundations of
Megatron-LM ..." (llms.blog), section "Self-Attention Layer Decomposition",
and the mohashari.github.io 70B page, "The Multi-Head Attention Block": the
Q, K and V projections are split by columns so each rank holds whole heads
(h/t of them; with grouped-query attention, n_q/t query heads and n_kv/t
key/value heads, e.g. 8 and 1 for Llama-3-70B at t = 8), each rank runs
attention on its own heads, and the output projection W_O is split by rows
so rank i's product is a partial that one all-reduce sums:

    Q_i = X W_Q^i,  K_i = X W_K^i,  V_i = X W_V^i
    Head_{i,k} = Softmax(Q_{i,k} K_{i,k}^T / sqrt(d)) V_{i,k}
    Z_i = [Head_{i,1} ... Head_{i,n}] W_O^i,    Z = sum_i Z_i

Layout readings: head k of Q occupies columns [k d, (k+1) d) of W_Q (and of
Q), likewise for K and V; rank i's query heads are [i n_q/t, (i+1) n_q/t) and
its KV heads [i n_kv/t, (i+1) n_kv/t); a query head k uses KV head
k // (n_q / n_kv).  The library takes rank i's three column blocks side by
side as one [h, (n_q/t + 2 n_kv/t) d] matrix [W_Q^i | W_K^i | W_V^i]; W_O^i
is rows [i (n_q/t) d, (i+1) (n_q/t) d) of W_O.  No biases, no mask (the
section's formula has none).  The attention core here exists only to check
the split end to end; the library computes the projections.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, i):
    """[W_Q^i | W_K^i | W_V^i]: rank i's heads' columns side by side."""
    if n_q % t or n_kv % t or n_q % n_kv:
        raise ValueError("heads must divide by t, and query heads by KV heads")
    q, kv = n_q // t * d, n_kv // t * d
    Wq, Wk, Wv = _f64(Wq), _f64(Wk), _f64(Wv)
    return np.concatenate([Wq[:, i * q:(i + 1) * q], Wk[:, i * kv:(i + 1) * kv], Wv[:, i * kv:(i + 1) * kv]],
                          axis=1)


def out_shard(Wo, n_q, d, t, i):
    """W_O^i: the rows that multiply rank i's query heads' outputs."""
    q = n_q // t * d
    return _f64(Wo)[i * q:(i + 1) * q]


def qkv_forward(X, Wqkv_i):
    """[Q_i | K_i | V_i] = X [W_Q^i | W_K^i | W_V^i]."""
    return _f64(X) @ _f64(Wqkv_i)


def out_forward(A_i, Wo_i):
    """The partial Z_i = A_i W_O^i, A_i the rank's heads' outputs side by side."""
    return _f64(A_i) @ _f64(Wo_i)


def qkv_backward(X, Wqkv_i, dQKV_i):
    """dX_i = dQKV_i Wqkv_i^T (a partial), dWqkv_i = X^T dQKV_i."""
    X, W, dY = _f64(X), _f64(Wqkv_i), _f64(dQKV_i)
    return {"dX": dY @ W.T, "dW": X.T @ dY}


def out_backward(A_i, Wo_i, dZ):
    """dA_i = dZ W_O^i^T, dWo_i = A_i^T dZ (dZ reaches every rank unchanged)."""
    A, W, dZ = _f64(A_i), _f64(Wo_i), _f64(dZ)
    return {"dA": dZ @ W.T, "dW": A.T @ dZ}


def attention_core(QKV, n_q, n_kv, d):
    """Softmax(Q_k K_g^T / sqrt(d)) V_g per query head k (g = its KV head),
    outputs side by side [M, n_q d].  QKV holds [Q | K | V] for n_q query and
    n_kv KV heads; rows are the positions of one sequence."""
    QKV = _f64(QKV)
    Q, K, V = QKV[:, :n_q * d], QKV[:, n_q * d:(n_q + n_kv) * d], QKV[:, (n_q + n_kv) * d:]
    out = np.empty((QKV.shape[0], n_q * d))
    group = n_q // n_kv
    for k in range(n_q):
        g = k // group
        q, kk, v = Q[:, k * d:(k + 1) * d], K[:, g * d:(g + 1) * d], V[:, g * d:(g + 1) * d]
        a = q @ kk.T / np.sqrt(d)
        a = np.exp(a - a.max(axis=1)[:, None])
        a /= a.sum(axis=1)[:, None]
        out[:, k * d:(k + 1) * d] = a @ v
    return out


def block_forward(X, Wq, Wk, Wv, Wo, n_q, n_kv, d):
    """The unsplit attention block: all heads, then W_O."""
    X = _f64(X)
    QKV = np.concatenate([X @ _f64(Wq), X @ _f64(Wk), X @ _f64(Wv)], axis=1)
    return attention_core(QKV, n_q, n_kv, d) @ _f64(Wo)

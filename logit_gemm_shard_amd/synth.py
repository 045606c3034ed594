"""Seeded synthetic inputs, shared by the tests, the benchmark and the smoke run.

This module only draws random numbers: it holds none of the method's
arithmetic.  Every draw uses a CPU ``torch.Generator`` seeded per workload, in
a fixed order, in float32, scaled to the stated standard deviation and cast
once to the workload's dtype (round-to-nearest-even for bfloat16).  Both the
HIP path and the fp64 oracle then read those same rounded values.
"""

import math

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name):
    return _DT[name]


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed_or_gen, dtype="f32"):
    """std * N(0, 1) draws of ``shape`` from a seeded CPU generator."""
    g = seed_or_gen if isinstance(seed_or_gen, torch.Generator) else _gen(seed_or_gen)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(_DT[dtype])


def residual_std(n_blocks, base=0.02):
    """Standard deviation of a weight placed just before a residual."""
    return base / math.sqrt(2.0 * n_blocks)


def mlp_weights(w, dtype=None):
    """X [M, h], A [h, ffn], B [ffn, h] for an MLP workload (draw order X, A, B)."""
    dt = dtype or w.dtype
    g = _gen(w.seed)
    X = normal((w.M, w.h), 1.0, g, dt)
    A = normal((w.h, w.ffn), 0.02, g, dt)
    B = normal((w.ffn, w.h), residual_std(w.n_blocks), g, dt)
    return X, A, B


def swiglu_weights(w, dtype=None):
    """X [M, h], W_gate [h, ffn], W_up [h, ffn], W_down [ffn, h] for a SwiGLU
    workload (draw order X, W_gate, W_up, W_down; W_down is the weight before
    the residual)."""
    dt = dtype or w.dtype
    g = _gen(w.seed)
    X = normal((w.M, w.h), 1.0, g, dt)
    Wg = normal((w.h, w.ffn), 0.02, g, dt)
    Wu = normal((w.h, w.ffn), 0.02, g, dt)
    Wd = normal((w.ffn, w.h), residual_std(w.n_blocks), g, dt)
    return X, Wg, Wu, Wd


def gate_up_shard(Wg, Wu, t, r):
    """Rank r's column blocks of W_gate and W_up side by side, [h, 2 ffn/t]
    (a copy in the layout the library takes; no arithmetic)."""
    f = Wg.shape[1] // t
    return torch.cat([Wg[:, r * f:(r + 1) * f], Wu[:, r * f:(r + 1) * f]], dim=1).contiguous()


def attn_weights(w, dtype=None):
    """X [M, h], W_Q [h, n_q d], W_K, W_V [h, n_kv d], W_O [n_q d, h] for an
    attention workload (draw order X, W_Q, W_K, W_V, W_O; W_O is the weight
    before the residual)."""
    dt = dtype or w.dtype
    g = _gen(w.seed)
    X = normal((w.M, w.h), 1.0, g, dt)
    Wq = normal((w.h, w.n_heads * w.head_dim), 0.02, g, dt)
    Wk = normal((w.h, w.n_kv_heads * w.head_dim), 0.02, g, dt)
    Wv = normal((w.h, w.n_kv_heads * w.head_dim), 0.02, g, dt)
    Wo = normal((w.n_heads * w.head_dim, w.h), residual_std(w.n_blocks), g, dt)
    return X, Wq, Wk, Wv, Wo


def qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, r):
    """Rank r's heads' columns of W_Q, W_K, W_V side by side (a copy in the
    layout the library takes; no arithmetic)."""
    q, kv = n_q // t * d, n_kv // t * d
    return torch.cat([Wq[:, r * q:(r + 1) * q], Wk[:, r * kv:(r + 1) * kv], Wv[:, r * kv:(r + 1) * kv]],
                     dim=1).contiguous()


def mlp_grad(w, dtype=None):
    """The incoming gradient dZ [M, h] of a backward workload."""
    return normal((w.M, w.h), w.dz_std, _gen(w.dz_seed), dtype or w.dtype)


def xent_inputs(w, dtype=None):
    """H [M, h], E [vocab, h] and int32 targets [M] uniform over the whole
    padded vocabulary (draw order H, E, targets)."""
    dt = dtype or w.dtype
    g = _gen(w.seed)
    H = normal((w.M, w.h), 1.0, g, dt)
    E = normal((w.vocab, w.h), 0.02, g, dt)
    y = torch.randint(0, w.vocab, (w.M,), generator=g, dtype=torch.int64).to(torch.int32)
    return H, E, y


def small(seed, *shapes, std=1.0, dtype="f32"):
    """Independent std*N(0,1) tensors of the given shapes from one seed (tests)."""
    g = _gen(seed)
    return [normal(s, std, g, dtype) for s in shapes]

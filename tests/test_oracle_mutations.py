"""Plant plausible mistakes in the oracle (on the CPU) and show that the pins
catch each one: a dropped term, a wrong sign, a wrong index or slice, a
transposed operand, a missing max subtraction.  A mutation that no pin
caught would mean the pins leave that part of the oracle unchecked."""

import numpy as np
import pytest
from scipy.special import erf

import oracle
import oracle_pins as pins

mlp, xent, sw = oracle.mlp, oracle.xent, oracle.swiglu
_orig_gelu, _orig_grad = mlp.gelu, mlp.gelu_grad


def _caught(checks, module):
    for c in checks:
        try:
            c(module)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


def _gelu_no_half(u, variant="erf"):
    u = np.asarray(u, dtype=np.float64)
    return u * (1.0 + erf(u / np.sqrt(2.0))) if variant == "erf" else _orig_gelu(u, variant)


def _gelu_no_sqrt2(u, variant="erf"):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + erf(u)) if variant == "erf" else _orig_gelu(u, variant)


def _gelu_tanh_no_cubic(u, variant="erf"):
    u = np.asarray(u, dtype=np.float64)
    if variant == "tanh":
        return 0.5 * u * (1.0 + np.tanh(np.sqrt(2 / np.pi) * u))
    return _orig_gelu(u, variant)


def _grad_dropped_term(u, variant="erf"):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * (1.0 + erf(u / np.sqrt(2.0))) if variant == "erf" else _orig_grad(u, variant)


def _grad_wrong_sign(u, variant="erf"):
    u = np.asarray(u, dtype=np.float64)
    if variant == "erf":
        return 0.5 * (1.0 + erf(u / np.sqrt(2.0))) - u * np.exp(-0.5 * u * u) / np.sqrt(2 * np.pi)
    return _orig_grad(u, variant)


def _column_shard_off_by_one(A, t, i):
    A = np.asarray(A, dtype=np.float64)
    f = A.shape[1] // t
    j = (i + 1) % t
    return A[:, j * f:(j + 1) * f]


def _row_shard_uses_columns(B, t, i):
    B = np.asarray(B, dtype=np.float64)
    f = B.shape[0] // t
    return B[i * f:(i + 1) * f, :][:, ::-1]


def _backward_missing_gelu_grad(X, A_i, B_i, U_i, dZ, variant="erf"):
    g = _REAL_BWD(X, A_i, B_i, U_i, dZ, variant)
    X = np.asarray(X, dtype=np.float64)
    g["dA"] = X.T @ g["dY"]
    return g


def _backward_dx_no_transpose(X, A_i, B_i, U_i, dZ, variant="erf"):
    g = _REAL_BWD(X, A_i, B_i, U_i, dZ, variant)
    A_i = np.asarray(A_i, dtype=np.float64)
    if A_i.shape[0] == A_i.shape[1]:
        g["dX"] = g["dU"] @ A_i
    else:
        g["dX"] = g["dU"][:, :A_i.shape[0]] @ A_i[:, :A_i.shape[0]]
    return g


def _backward_db_uses_u(X, A_i, B_i, U_i, dZ, variant="erf"):
    g = _REAL_BWD(X, A_i, B_i, U_i, dZ, variant)
    g["dB"] = np.asarray(U_i, dtype=np.float64).T @ np.asarray(dZ, dtype=np.float64)
    return g


def _partial_sum_skips_first(parts):
    parts = [np.asarray(p, dtype=np.float64) for p in parts]
    out = np.zeros_like(parts[0])
    for p in parts[1:]:
        out = out + p
    return out if len(parts) > 1 else parts[0]


_REAL_BWD = mlp.shard_backward

MLP_MUTANTS = {
    "gelu_no_half": ("gelu", _gelu_no_half),
    "gelu_no_sqrt2": ("gelu", _gelu_no_sqrt2),
    "gelu_tanh_no_cubic": ("gelu", _gelu_tanh_no_cubic),
    "grad_dropped_term": ("gelu_grad", _grad_dropped_term),
    "grad_wrong_sign": ("gelu_grad", _grad_wrong_sign),
    "column_shard_wrong_block": ("column_shard", _column_shard_off_by_one),
    "row_shard_scrambled": ("row_shard", _row_shard_uses_columns),
    "bwd_missing_gelu_grad": ("shard_backward", _backward_missing_gelu_grad),
    "bwd_dx_no_transpose": ("shard_backward", _backward_dx_no_transpose),
    "bwd_db_uses_preact": ("shard_backward", _backward_db_uses_u),
    "partial_sum_skips_rank0": ("partial_sum", _partial_sum_skips_first),
}


@pytest.mark.parametrize("name", sorted(MLP_MUTANTS))
def test_mlp_mutant_is_caught(name, monkeypatch):
    attr, fn = MLP_MUTANTS[name]
    monkeypatch.setattr(mlp, attr, fn)  # module-level, so the oracle's own callers see it too
    assert _caught(pins.MLP_CHECKS, mlp), f"no pin caught the planted mistake {name}"


def _naive_no_max(H, E, y, chunk=1024):
    H, E = np.asarray(H, dtype=np.float64), np.asarray(E, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        z = H @ E.T
        return np.log(np.exp(z).sum(axis=1)) - z[np.arange(z.shape[0]), np.asarray(y)]


def _naive_log2(H, E, y, chunk=1024):
    H, E = np.asarray(H, dtype=np.float64), np.asarray(E, dtype=np.float64)
    z = H @ E.T
    mx = z.max(axis=1)
    return mx + np.log2(np.exp(z - mx[:, None]).sum(axis=1)) - z[np.arange(z.shape[0]), np.asarray(y)]


_REAL_PARTIALS = xent.shard_partials


def _partials_global_target(H, E_r, y, vocab_start):
    m, l, T, am = _REAL_PARTIALS(H, E_r, y, vocab_start)
    z = np.asarray(H, dtype=np.float64) @ np.asarray(E_r, dtype=np.float64).T
    y = np.asarray(y)
    own = y < z.shape[1]
    T = np.where(own, z[np.arange(z.shape[0]), np.minimum(y, z.shape[1] - 1)], 0.0)
    return m, l, T, am


def _partials_local_argmax(H, E_r, y, vocab_start):
    m, l, T, am = _REAL_PARTIALS(H, E_r, y, vocab_start)
    return m, l, T, am - vocab_start


def _partials_last_tie(H, E_r, y, vocab_start):
    m, l, T, am = _REAL_PARTIALS(H, E_r, y, vocab_start)
    z = np.asarray(H, dtype=np.float64) @ np.asarray(E_r, dtype=np.float64).T
    am = vocab_start + z.shape[1] - 1 - np.argmax(z[:, ::-1], axis=1)
    return m, l, T, am


def _merge_wrong_sign(m, l, T):
    m, l, T = (np.asarray(a, dtype=np.float64) for a in (m, l, T))
    Mx = m.max(axis=0)
    return Mx + np.log((l * np.exp(Mx[None, :] - m)).sum(axis=0)) - T.sum(axis=0)


def _merge_drops_max(m, l, T):
    m, l, T = (np.asarray(a, dtype=np.float64) for a in (m, l, T))
    Mx = m.max(axis=0)
    return np.log((l * np.exp(m - Mx[None, :])).sum(axis=0)) - T.sum(axis=0)


def _merge_argmax_last_rank(m, am):
    m = np.asarray(m, dtype=np.float64)
    r = m.shape[0] - 1 - np.argmax(m[::-1], axis=0)
    return np.asarray(am)[r, np.arange(m.shape[1])]


XENT_MUTANTS = {
    "naive_no_max_subtraction": ("naive_loss", _naive_no_max),
    "naive_log2": ("naive_loss", _naive_log2),
    "partials_global_target_index": ("shard_partials", _partials_global_target),
    "partials_local_argmax_id": ("shard_partials", _partials_local_argmax),
    "partials_last_tie": ("shard_partials", _partials_last_tie),
    "merge_wrong_sign": ("merge", _merge_wrong_sign),
    "merge_drops_max": ("merge", _merge_drops_max),
    "merge_argmax_last_rank": ("merge_argmax", _merge_argmax_last_rank),
}


@pytest.mark.parametrize("name", sorted(XENT_MUTANTS))
def test_xent_mutant_is_caught(name, monkeypatch):
    attr, fn = XENT_MUTANTS[name]
    monkeypatch.setattr(xent, attr, fn)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        assert _caught(pins.XENT_CHECKS, xent), f"no pin caught the planted mistake {name}"


# ----------------------------------------------------------------- SwiGLU

_REAL_SIGMOID, _REAL_SWISH, _REAL_SWISH_GRAD = sw.sigmoid, sw.swish, sw.swish_grad
_REAL_SW_BWD = sw.shard_backward


def _sigmoid_flipped(g):
    return _REAL_SIGMOID(-np.asarray(g, dtype=np.float64))


def _swish_is_sigmoid(g):
    return _REAL_SIGMOID(g)


def _swish_grad_dropped_term(g):
    return _REAL_SIGMOID(g)


def _swish_grad_wrong_sign(g):
    g = np.asarray(g, dtype=np.float64)
    s = _REAL_SIGMOID(g)
    return s - g * s * (1.0 - s)


def _swish_grad_missing_one_minus(g):
    g = np.asarray(g, dtype=np.float64)
    s = _REAL_SIGMOID(g)
    return s + g * s


def _sw_forward_gate_on_up(X, Wg, Wu, Wd):
    X, Wg, Wu, Wd = (np.asarray(a, dtype=np.float64) for a in (X, Wg, Wu, Wd))
    G, U = X @ Wg, X @ Wu
    Y = G * _REAL_SWISH(U)
    return G, U, Y, Y @ Wd


def _sw_bwd_dg_missing_u(X, Wg, Wu, Wd, G, U, dZ):
    g = _REAL_SW_BWD(X, Wg, Wu, Wd, G, U, dZ)
    g["dG"] = g["dY"] * sw.swish_grad(np.asarray(G, dtype=np.float64))
    g["dWg"] = np.asarray(X, dtype=np.float64).T @ g["dG"]
    g["dX"] = g["dG"] @ np.asarray(Wg, dtype=np.float64).T + g["dU"] @ np.asarray(Wu, dtype=np.float64).T
    return g


def _sw_bwd_du_uses_g(X, Wg, Wu, Wd, G, U, dZ):
    g = _REAL_SW_BWD(X, Wg, Wu, Wd, G, U, dZ)
    g["dU"] = g["dY"] * np.asarray(G, dtype=np.float64)
    g["dWu"] = np.asarray(X, dtype=np.float64).T @ g["dU"]
    return g


def _sw_bwd_swapped_weight_grads(X, Wg, Wu, Wd, G, U, dZ):
    g = _REAL_SW_BWD(X, Wg, Wu, Wd, G, U, dZ)
    g["dWg"], g["dWu"] = g["dWu"], g["dWg"]
    return g


def _sw_bwd_dx_drops_up(X, Wg, Wu, Wd, G, U, dZ):
    g = _REAL_SW_BWD(X, Wg, Wu, Wd, G, U, dZ)
    g["dX"] = g["dG"] @ np.asarray(Wg, dtype=np.float64).T
    return g


def _sw_bwd_dwd_uses_g_times_u(X, Wg, Wu, Wd, G, U, dZ):
    g = _REAL_SW_BWD(X, Wg, Wu, Wd, G, U, dZ)
    Y = np.asarray(G, dtype=np.float64) * np.asarray(U, dtype=np.float64)
    g["Y"], g["dWd"] = Y, Y.T @ np.asarray(dZ, dtype=np.float64)
    return g


def _sw_bwd_dx_wrong_operand(X, Wg, Wu, Wd, G, U, dZ):
    g = _REAL_SW_BWD(X, Wg, Wu, Wd, G, U, dZ)
    g["dX"] = g["dU"] @ np.asarray(Wg, dtype=np.float64).T + g["dG"] @ np.asarray(Wu, dtype=np.float64).T
    return g


SWIGLU_MUTANTS = {
    "sigmoid_flipped": ("sigmoid", _sigmoid_flipped),
    "swish_is_sigmoid": ("swish", _swish_is_sigmoid),
    "swish_grad_dropped_term": ("swish_grad", _swish_grad_dropped_term),
    "swish_grad_wrong_sign": ("swish_grad", _swish_grad_wrong_sign),
    "swish_grad_missing_one_minus": ("swish_grad", _swish_grad_missing_one_minus),
    "forward_gate_on_up": ("swiglu_forward", _sw_forward_gate_on_up),
    "bwd_dg_missing_up": ("shard_backward", _sw_bwd_dg_missing_u),
    "bwd_du_uses_preact": ("shard_backward", _sw_bwd_du_uses_g),
    "bwd_swapped_weight_grads": ("shard_backward", _sw_bwd_swapped_weight_grads),
    "bwd_dx_drops_up": ("shard_backward", _sw_bwd_dx_drops_up),
    "bwd_dwd_ungated": ("shard_backward", _sw_bwd_dwd_uses_g_times_u),
    "bwd_dx_crossed_operands": ("shard_backward", _sw_bwd_dx_wrong_operand),
    "column_shard_wrong_block": ("column_shard", _column_shard_off_by_one),
}


@pytest.mark.parametrize("name", sorted(SWIGLU_MUTANTS))
def test_swiglu_mutant_is_caught(name, monkeypatch):
    attr, fn = SWIGLU_MUTANTS[name]
    monkeypatch.setattr(sw, attr, fn)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        assert _caught(pins.SWIGLU_CHECKS, sw), f"no pin caught the planted mistake {name}"


# ------------------------------------------------------------ CE backward

_REAL_XBWD, _REAL_XSHARD, _REAL_LSE = xent.xent_backward, xent.shard_backward, xent.merge_lse


def _xbwd_no_onehot(H, E, y, dloss=None):
    g = _REAL_XBWD(H, E, y, dloss)
    w = np.ones(len(y)) if dloss is None else np.asarray(dloss, dtype=np.float64)
    G = g["G"].copy()
    G[np.arange(len(y)), np.asarray(y)] += w  # the one-hot dropped
    H, E = np.asarray(H, dtype=np.float64), np.asarray(E, dtype=np.float64)
    return {"G": G, "dH": G @ E, "dE": G.T @ H}


def _xbwd_unweighted(H, E, y, dloss=None):
    return _REAL_XBWD(H, E, y, None)


def _xbwd_de_uses_e(H, E, y, dloss=None):
    g = _REAL_XBWD(H, E, y, dloss)
    E = np.asarray(E, dtype=np.float64)
    g["dE"] = g["G"].T @ (g["G"] @ E) if g["G"].shape[1] == E.shape[0] else g["dE"] * 2
    return g


def _xbwd_softmax_wrong_axis(H, E, y, dloss=None):
    H, E = np.asarray(H, dtype=np.float64), np.asarray(E, dtype=np.float64)
    z = H @ E.T
    p = np.exp(z - z.max(axis=0)[None, :])
    p /= p.sum(axis=0)[None, :]
    p[np.arange(z.shape[0]), np.asarray(y)] -= 1.0
    p *= (np.ones(z.shape[0]) if dloss is None else np.asarray(dloss, dtype=np.float64))[:, None]
    return {"G": p, "dH": p @ E, "dE": p.T @ H}


def _xshard_global_target(H, E_r, y, vocab_start, lse, dloss=None):
    return _REAL_XSHARD(H, E_r, y, 0, lse, dloss)  # target column not shifted into the slice


def _xshard_local_lse(H, E_r, y, vocab_start, lse, dloss=None):
    z = np.asarray(H, dtype=np.float64) @ np.asarray(E_r, dtype=np.float64).T
    mx = z.max(axis=1)
    own = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))  # the slice's own lse, not the merged one
    return _REAL_XSHARD(H, E_r, y, vocab_start, own, dloss)


def _merge_lse_drops_max(m, l):
    m, l = np.asarray(m, dtype=np.float64), np.asarray(l, dtype=np.float64)
    return np.log((l * np.exp(m - m.max(axis=0)[None, :])).sum(axis=0))


XENT_BWD_MUTANTS = {
    "bwd_no_onehot": ("xent_backward", _xbwd_no_onehot),
    "bwd_ignores_dloss": ("xent_backward", _xbwd_unweighted),
    "bwd_de_wrong_operand": ("xent_backward", _xbwd_de_uses_e),
    "bwd_softmax_over_tokens": ("xent_backward", _xbwd_softmax_wrong_axis),
    "shard_target_not_shifted": ("shard_backward", _xshard_global_target),
    "shard_uses_local_lse": ("shard_backward", _xshard_local_lse),
    "merge_lse_drops_max": ("merge_lse", _merge_lse_drops_max),
}


@pytest.mark.parametrize("name", sorted(XENT_BWD_MUTANTS))
def test_xent_backward_mutant_is_caught(name, monkeypatch):
    attr, fn = XENT_BWD_MUTANTS[name]
    monkeypatch.setattr(xent, attr, fn)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        assert _caught(pins.XENT_BWD_CHECKS, xent), f"no pin caught the planted mistake {name}"


# ------------------------------------------------------ sequence parallelism

sp = oracle.sp
_REAL_CHUNK = sp.chunk_rows


def _chunk_b_major(s, b, t, r):
    # chunks taken along the flattened axis as if it were (b, s): wrong rows
    a, z = _REAL_CHUNK(s, b, t, r)
    return (a + b) % (s * b), (a + b) % (s * b) + (z - a)


def _rs_skips_last(parts, s, b, t, r):
    a, z = sp.chunk_rows(s, b, t, r)
    out = np.zeros_like(np.asarray(parts[0], dtype=np.float64)[a:z])
    for p in parts[:-1] if len(parts) > 1 else parts:
        out = out + np.asarray(p, dtype=np.float64)[a:z]
    return out


def _ag_reversed(shards, s, b, t):
    return np.concatenate([np.asarray(x, dtype=np.float64) for x in shards[::-1]], axis=0)


def _volume_no_half(kind, t, n):
    one = (t - 1) * n
    return {"reduce_scatter": one, "all_gather": one, "all_reduce": one}[kind]


_REAL_LN, _REAL_EXIT = sp.layernorm, sp.exit_region


def _ln_no_eps(x, gamma, beta, eps=1e-5):
    return _REAL_LN(x, gamma, beta, 0.0)


def _ln_unbiased(x, gamma, beta, eps=1e-5):
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=1, keepdims=True)
    var = ((x - mean) ** 2).sum(axis=1, keepdims=True) / (x.shape[1] - 1)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def _ln_stats_over_tokens(x, gamma, beta, eps=1e-5):
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=0, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=0, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def _ln_gamma_beta_swapped(x, gamma, beta, eps=1e-5):
    return _REAL_LN(x, beta, gamma, eps)


def _exit_no_dropout_scale(parts, s, b, t, r, residual, gamma, beta, eps=1e-5, keep=None, keep_scale=1.0):
    return _REAL_EXIT(parts, s, b, t, r, residual, gamma, beta, eps, keep, 1.0)


def _exit_no_residual(parts, s, b, t, r, residual, gamma, beta, eps=1e-5, keep=None, keep_scale=1.0):
    return _REAL_EXIT(parts, s, b, t, r, np.zeros_like(np.asarray(residual, dtype=np.float64)), gamma, beta, eps,
                      keep, keep_scale)


def _exit_norm_before_add(parts, s, b, t, r, residual, gamma, beta, eps=1e-5, keep=None, keep_scale=1.0):
    z = sp.reduce_scatter(parts, s, b, t, r)
    d = z if keep is None else z * (np.asarray(keep) != 0) * keep_scale
    return residual + d, _REAL_LN(d, gamma, beta, eps) + residual


_REAL_LN_BWD, _REAL_EXIT_BWD = sp.layernorm_backward, sp.exit_region_backward


def _lnb_core(x, gamma, dy, eps, drop_mean=False, drop_proj=False, dgamma_plain=False):
    x, dy = np.asarray(x, dtype=np.float64), np.asarray(dy, dtype=np.float64)
    mean = x.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mean) ** 2).mean(axis=1, keepdims=True) + eps)
    xhat = (x - mean) * rstd
    dxh = dy * gamma
    dx = dxh
    if not drop_mean:
        dx = dx - dxh.mean(axis=1, keepdims=True)
    if not drop_proj:
        dx = dx - xhat * (dxh * xhat).mean(axis=1, keepdims=True)
    return dx * rstd, (dy if dgamma_plain else dy * xhat).sum(axis=0), dy.sum(axis=0)


def _lnb_no_mean(x, gamma, dy, eps=1e-5):
    return _lnb_core(x, gamma, dy, eps, drop_mean=True)


def _lnb_no_projection(x, gamma, dy, eps=1e-5):
    return _lnb_core(x, gamma, dy, eps, drop_proj=True)


def _lnb_dgamma_without_xhat(x, gamma, dy, eps=1e-5):
    return _lnb_core(x, gamma, dy, eps, dgamma_plain=True)


def _exitb_dz_unmasked(hs, gamma, dy, dhs=None, eps=1e-5, keep=None, keep_scale=1.0):
    return _REAL_EXIT_BWD(hs, gamma, dy, dhs, eps, None, keep_scale)


def _exitb_no_residual_grad(hs, gamma, dy, dhs=None, eps=1e-5, keep=None, keep_scale=1.0):
    return _REAL_EXIT_BWD(hs, gamma, dy, None, eps, keep, keep_scale)


SP_MUTANTS = {
    "lnb_no_mean_term": ("layernorm_backward", _lnb_no_mean),
    "lnb_no_projection_term": ("layernorm_backward", _lnb_no_projection),
    "lnb_dgamma_without_xhat": ("layernorm_backward", _lnb_dgamma_without_xhat),
    "exitb_dz_unmasked": ("exit_region_backward", _exitb_dz_unmasked),
    "exitb_residual_grad_dropped": ("exit_region_backward", _exitb_no_residual_grad),
    "ln_no_eps": ("layernorm", _ln_no_eps),
    "ln_unbiased_variance": ("layernorm", _ln_unbiased),
    "ln_stats_over_tokens": ("layernorm", _ln_stats_over_tokens),
    "ln_gamma_beta_swapped": ("layernorm", _ln_gamma_beta_swapped),
    "exit_dropout_unscaled": ("exit_region", _exit_no_dropout_scale),
    "exit_residual_dropped": ("exit_region", _exit_no_residual),
    "exit_norm_before_add": ("exit_region", _exit_norm_before_add),
    "chunk_wrong_rows": ("chunk_rows", _chunk_b_major),
    "rs_skips_last_rank": ("reduce_scatter", _rs_skips_last),
    "ag_reversed_order": ("all_gather", _ag_reversed),
    "volume_wrong": ("comm_volume", _volume_no_half),
}


@pytest.mark.parametrize("name", sorted(SP_MUTANTS))
def test_sp_mutant_is_caught(name, monkeypatch):
    attr, fn = SP_MUTANTS[name]
    monkeypatch.setattr(sp, attr, fn)
    assert _caught(pins.SP_CHECKS, sp), f"no pin caught the planted mistake {name}"


# ---------------------------------------------------- attention projections

at = oracle.attn
_REAL_QKV_SHARD, _REAL_OUT_SHARD, _REAL_CORE = at.qkv_shard, at.out_shard, at.attention_core
_REAL_QKV_BWD, _REAL_OUT_BWD = at.qkv_backward, at.out_backward


def _qkv_shard_k_from_q(Wq, Wk, Wv, n_q, n_kv, d, t, i):
    return _REAL_QKV_SHARD(Wq, Wq[:, :Wk.shape[1]], Wv, n_q, n_kv, d, t, i)


def _qkv_shard_kv_not_split(Wq, Wk, Wv, n_q, n_kv, d, t, i):
    return _REAL_QKV_SHARD(Wq, Wk, Wv, n_q, n_kv, d, t, 0) if i else _REAL_QKV_SHARD(Wq, Wk, Wv, n_q, n_kv, d, t, i)


def _out_shard_next_rank(Wo, n_q, d, t, i):
    return _REAL_OUT_SHARD(Wo, n_q, d, t, (i + 1) % t)


def _core_kv_interleaved(QKV, n_q, n_kv, d):
    # query head k reading KV head k % n_kv instead of k // (n_q / n_kv)
    QKV = np.asarray(QKV, dtype=np.float64)
    Q, K, V = QKV[:, :n_q * d], QKV[:, n_q * d:(n_q + n_kv) * d], QKV[:, (n_q + n_kv) * d:]
    out = np.empty((QKV.shape[0], n_q * d))
    for k in range(n_q):
        g = k % n_kv
        a = Q[:, k * d:(k + 1) * d] @ K[:, g * d:(g + 1) * d].T / np.sqrt(d)
        a = np.exp(a - a.max(axis=1)[:, None])
        a /= a.sum(axis=1)[:, None]
        out[:, k * d:(k + 1) * d] = a @ V[:, g * d:(g + 1) * d]
    return out


def _core_no_scale(QKV, n_q, n_kv, d):
    return _REAL_CORE(np.asarray(QKV, dtype=np.float64) * np.concatenate(
        [np.full(n_q * d, np.sqrt(np.sqrt(d))), np.full(n_kv * d, np.sqrt(np.sqrt(d))), np.ones(n_kv * d)]),
        n_q, n_kv, d)


def _qkv_bwd_dx_scaled(X, W, dY):
    g = _REAL_QKV_BWD(X, W, dY)
    g["dX"] = g["dX"] * (1 + 1e-3)  # a stray factor
    return g


def _qkv_bwd_dw_of_dx(X, W, dY):
    g = _REAL_QKV_BWD(X, W, dY)
    g["dW"] = np.asarray(dY, dtype=np.float64).T @ np.asarray(X, dtype=np.float64)  # transposed product
    return g


def _out_bwd_dw_swapped(A, Wo, dZ):
    g = _REAL_OUT_BWD(A, Wo, dZ)
    g["dW"] = np.asarray(A, dtype=np.float64).T @ np.asarray(dZ, dtype=np.float64)[::-1]
    return g


ATTN_MUTANTS = {
    "qkv_shard_k_from_q": ("qkv_shard", _qkv_shard_k_from_q),
    "qkv_shard_kv_not_split": ("qkv_shard", _qkv_shard_kv_not_split),
    "out_shard_next_rank": ("out_shard", _out_shard_next_rank),
    "core_kv_interleaved": ("attention_core", _core_kv_interleaved),
    "core_no_scale": ("attention_core", _core_no_scale),
    "qkv_bwd_dx_scaled": ("qkv_backward", _qkv_bwd_dx_scaled),
    "qkv_bwd_dw_transposed": ("qkv_backward", _qkv_bwd_dw_of_dx),
    "out_bwd_dw_rows_swapped": ("out_backward", _out_bwd_dw_swapped),
}


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attn_mutant_is_caught(name, monkeypatch):
    attr, fn = ATTN_MUTANTS[name]
    monkeypatch.setattr(at, attr, fn)
    assert _caught(pins.ATTN_CHECKS, at), f"no pin caught the planted mistake {name}"

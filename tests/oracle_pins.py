"""Checks that pin the fp64 oracle to things other than itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with:
brute-force pure-Python loops, printed normal-table values, hand-worked
examples (``tests/golden/``), central finite differences, or identities that
the pages state (the split sum, the elementwise commutation of the
nonlinearity, fused == full-logit cross-entropy).

They take the oracle modules as arguments so that ``test_oracle_mutations.py``
can plant mistakes in the oracle (on the CPU) and show that some check fails.
"""

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / den


def read_rows(name):
    """Parse a golden file: {key: [row, row, ...]} of float lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append([float(v) for v in vals])
    return out


# ----------------------------------------------------------------- brute force

def bf_matmul(P, Q):
    n, k = len(P), len(P[0])
    m = len(Q[0])
    assert len(Q) == k
    return [[sum(P[i][kk] * Q[kk][j] for kk in range(k)) for j in range(m)] for i in range(n)]


def bf_gelu(u):
    return 0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0)))


def bf_mlp(X, A, B):
    """The unsplit block by nested loops (exact GeLU through math.erf)."""
    U = bf_matmul(X, A)
    Y = [[bf_gelu(v) for v in row] for row in U]
    return U, Y, bf_matmul(Y, B)


def bf_xent(H, E, y):
    """Per-token full-vocabulary cross-entropy by nested loops."""
    out = []
    for k, hrow in enumerate(H):
        z = [sum(hrow[c] * erow[c] for c in range(len(hrow))) for erow in E]
        mx = max(z)
        s = sum(math.exp(v - mx) for v in z)
        out.append(mx + math.log(s) - z[y[k]])
    return out


# ------------------------------------------------------------------ MLP checks

def check_gelu_table(mlp):
    pts = []
    with open(os.path.join(GOLDEN, "gelu_normal_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                u, p = line.split()
                pts.append((float(u), float(p)))
    for u, phi in pts:
        got = float(mlp.gelu(np.array([u]), "erf")[0])
        assert abs(got - u * phi) <= 1e-15 * max(1.0, abs(u)), (u, got, u * phi)
    # GeLU'(0) = Phi(0) = 1/2, and GeLU'(u) -> 1 / 0 far out
    assert abs(float(mlp.gelu_grad(np.array([0.0]), "erf")[0]) - 0.5) < 1e-15
    assert abs(float(mlp.gelu_grad(np.array([12.0]), "erf")[0]) - 1.0) < 1e-12
    assert abs(float(mlp.gelu_grad(np.array([-12.0]), "erf")[0])) < 1e-12


def check_gelu_shape(mlp):
    """Odd-part identity GeLU(u) - GeLU(-u) = u (both variants), asymptotes,
    and the tanh form within its known distance of the exact form."""
    u = np.linspace(-8, 8, 4001)
    for v in ("erf", "tanh"):
        g = mlp.gelu(u, v)
        assert np.abs(g - mlp.gelu(-u, v) - u).max() < 1e-13, v
        assert abs(float(mlp.gelu(np.array([40.0]), v)[0]) - 40.0) < 1e-12, v
        assert abs(float(mlp.gelu(np.array([-40.0]), v)[0])) < 1e-12, v
        assert float(mlp.gelu(np.array([0.0]), v)[0]) == 0.0, v
    exact = np.array([bf_gelu(x) for x in u])
    assert np.abs(mlp.gelu(u, "erf") - exact).max() < 1e-14
    dev = np.abs(mlp.gelu(u, "tanh") - exact).max()
    assert 1e-4 < dev < 5e-4, dev  # the tanh approximation's max error is about 4.7e-4


def check_gelu_grad_fd(mlp):
    u = np.linspace(-6, 6, 1201)
    eps = 1e-6
    for v in ("erf", "tanh"):
        fd = (mlp.gelu(u + eps, v) - mlp.gelu(u - eps, v)) / (2 * eps)
        assert np.abs(mlp.gelu_grad(u, v) - fd).max() < 1e-8, v


def check_mlp_hand_example(mlp):
    g = read_rows("mlp_hand_example.txt")
    X, A, B = (np.array(g[k]) for k in ("X", "A", "B"))
    U, Y, Z = mlp.mlp_forward(X, A, B, "erf")
    assert np.array_equal(U, np.array(g["U"]))
    assert _rel(Y, g["Y"]) < 1e-15
    assert _rel(Z, g["Z"]) < 1e-15
    Z1 = mlp.shard_forward(X, mlp.column_shard(A, 2, 0), mlp.row_shard(B, 2, 0), "erf")[2]
    Z2 = mlp.shard_forward(X, mlp.column_shard(A, 2, 1), mlp.row_shard(B, 2, 1), "erf")[2]
    assert _rel(Z1, g["Z1"]) < 1e-15 and _rel(Z2, g["Z2"]) < 1e-15
    assert _rel(mlp.partial_sum([Z1, Z2]), g["Z"]) < 1e-15


def check_mlp_brute_force(mlp):
    for seed, (M, h, ffn, t) in enumerate([(3, 5, 8, 2), (4, 3, 6, 3), (2, 7, 4, 1), (5, 4, 12, 4)]):
        r = _rng(100 + seed)
        X, A, B = r.normal(size=(M, h)), r.normal(size=(h, ffn)), r.normal(size=(ffn, h))
        bU, bY, bZ = bf_mlp(X.tolist(), A.tolist(), B.tolist())
        U, Y, Z = mlp.mlp_forward(X, A, B, "erf")
        assert _rel(U, bU) < 1e-13 and _rel(Y, bY) < 1e-13 and _rel(Z, bZ) < 1e-13
        f = ffn // t
        for i in range(t):
            Ai = [row[i * f:(i + 1) * f] for row in A.tolist()]
            Bi = B.tolist()[i * f:(i + 1) * f]
            cU, cY, cZ = bf_mlp(X.tolist(), Ai, Bi)
            U_i, Y_i, Z_i = mlp.shard_forward(X, mlp.column_shard(A, t, i), mlp.row_shard(B, t, i), "erf")
            assert _rel(U_i, cU) < 1e-13 and _rel(Y_i, cY) < 1e-13 and _rel(Z_i, cZ) < 1e-13


def check_split_identity(mlp):
    """Z = sum_i GeLU(X A_i) B_i, sigma commutes with the column split, and
    t = 1 is the unsplit layer."""
    r = _rng(7)
    M, h, ffn = 16, 24, 64
    X, A, B = r.normal(size=(M, h)), r.normal(size=(h, ffn)) * 0.3, r.normal(size=(ffn, h)) * 0.3
    U, Y, Z = mlp.mlp_forward(X, A, B, "erf")
    for t in (1, 2, 8):
        parts, Ys = [], []
        for i in range(t):
            U_i, Y_i, Z_i = mlp.shard_forward(X, mlp.column_shard(A, t, i), mlp.row_shard(B, t, i), "erf")
            parts.append(Z_i)
            Ys.append(Y_i)
        assert _rel(mlp.partial_sum(parts), Z) < 1e-12, t
        assert _rel(np.concatenate(Ys, axis=1), Y) < 1e-15, t
        if t == 1:
            assert _rel(parts[0], Z) < 1e-15


def check_partial_sum_exact(mlp):
    r = _rng(11)
    parts = [r.integers(-1000, 1000, size=(7, 9)).astype(np.float64) for _ in range(5)]
    want = np.zeros((7, 9))
    for p in parts:
        for a in range(7):
            for b in range(9):
                want[a, b] += p[a, b]
    assert np.array_equal(mlp.partial_sum(parts), want)


def _loss(mlp, X, A_i, B_i, dZ, v):
    return float((mlp.shard_forward(X, A_i, B_i, v)[2] * dZ).sum())


def check_backward_fd(mlp):
    """Every entry of dX_i, dA_i, dB_i equals a central difference of
    L = <dZ, Z_i(X, A_i, B_i)>, on tiny shapes."""
    eps = 1e-6
    for v in ("erf", "tanh"):
        r = _rng(21)
        M, h, f = 3, 4, 5
        X, A_i, B_i, dZ = (r.normal(size=s) for s in ((M, h), (h, f), (f, h), (M, h)))
        U_i = X @ A_i
        g = mlp.shard_backward(X, A_i, B_i, U_i, dZ, v)
        for name, P in (("dX", X), ("dA", A_i), ("dB", B_i)):
            fd = np.zeros_like(P)
            for idx in np.ndindex(P.shape):
                old = P[idx]
                P[idx] = old + eps
                lp = _loss(mlp, X, A_i, B_i, dZ, v)
                P[idx] = old - eps
                lm = _loss(mlp, X, A_i, B_i, dZ, v)
                P[idx] = old
                fd[idx] = (lp - lm) / (2 * eps)
            assert _rel(g[name], fd) < 1e-6, (v, name, _rel(g[name], fd))
        assert _rel(g["Y"], mlp.gelu(U_i, v)) < 1e-15


def check_backward_directional(mlp):
    """At a moderate size: <dP, dir> equals the central difference of L along
    a random direction, for P in X, A_i, B_i (a check over every entry at once)."""
    r = _rng(31)
    M, h, f = 48, 40, 56
    X, A_i, B_i = r.normal(size=(M, h)), r.normal(size=(h, f)) * 0.2, r.normal(size=(f, h)) * 0.2
    dZ = r.normal(size=(M, h))
    g = mlp.shard_backward(X, A_i, B_i, X @ A_i, dZ, "erf")
    eps = 1e-5
    for name in ("dX", "dA", "dB"):
        D = r.normal(size={"dX": X, "dA": A_i, "dB": B_i}[name].shape)
        args_p = [X, A_i, B_i]
        args_m = [X, A_i, B_i]
        k = {"dX": 0, "dA": 1, "dB": 2}[name]
        args_p = args_p[:k] + [args_p[k] + eps * D] + args_p[k + 1:]
        args_m = args_m[:k] + [args_m[k] - eps * D] + args_m[k + 1:]
        fd = (_loss(mlp, *args_p, dZ, "erf") - _loss(mlp, *args_m, dZ, "erf")) / (2 * eps)
        an = float((g[name] * D).sum())
        assert abs(an - fd) <= 1e-7 * max(1.0, abs(fd)), (name, an, fd)


def check_backward_shards(mlp):
    """Concatenated dA_i / dB_i equal the unsplit layer's dA / dB, and the
    sum of the partials dX_i equals the unsplit dX (the f* all-reduce)."""
    r = _rng(41)
    M, h, ffn, t = 20, 16, 48, 4
    X, A, B, dZ = r.normal(size=(M, h)), r.normal(size=(h, ffn)) * 0.3, r.normal(size=(ffn, h)) * 0.3, r.normal(size=(M, h))
    full = mlp.mlp_backward(X, A, B, dZ, "erf")
    dAs, dBs, dXs = [], [], []
    for i in range(t):
        A_i, B_i = mlp.column_shard(A, t, i), mlp.row_shard(B, t, i)
        g = mlp.shard_backward(X, A_i, B_i, X @ A_i, dZ, "erf")
        dAs.append(g["dA"])
        dBs.append(g["dB"])
        dXs.append(g["dX"])
    assert _rel(np.concatenate(dAs, axis=1), full["dA"]) < 1e-13
    assert _rel(np.concatenate(dBs, axis=0), full["dB"]) < 1e-13
    assert _rel(mlp.partial_sum(dXs), full["dX"]) < 1e-12


# --------------------------------------------------------------- SwiGLU checks

def bf_swish(g):
    return g / (1.0 + math.exp(-g)) if g >= 0 else g * math.exp(g) / (1.0 + math.exp(g))


def bf_swiglu(X, Wg, Wu, Wd):
    """The unsplit gated block by nested loops."""
    G, U = bf_matmul(X, Wg), bf_matmul(X, Wu)
    Y = [[bf_swish(g) * u for g, u in zip(gr, ur)] for gr, ur in zip(G, U)]
    return G, U, Y, bf_matmul(Y, Wd)


def check_swish_closed_forms(sw):
    """sigmoid(ln k) = k / (k + 1) gives Swish and its slope in closed form at
    g = ln k; Swish(0) = 0, Swish'(0) = 1/2; the odd-part identity
    Swish(g) - Swish(-g) = g (from sigmoid(g) + sigmoid(-g) = 1); Swish
    approaches g far right and 0 far left, its slope 1 and 0."""
    for k in (0.25, 0.5, 1.0, 3.0, 9.0, 1e6):
        g = math.log(k)
        s = k / (k + 1.0)
        assert abs(float(sw.swish(np.array([g]))[0]) - g * s) <= 1e-15 * max(1.0, abs(g)), k
        assert abs(float(sw.swish_grad(np.array([g]))[0]) - (s + g * s / (k + 1.0))) <= 1e-15 * max(1.0, abs(g)), k
    assert float(sw.swish(np.array([0.0]))[0]) == 0.0
    assert abs(float(sw.swish_grad(np.array([0.0]))[0]) - 0.5) < 1e-16
    g = np.linspace(-30, 30, 6001)
    assert np.abs(sw.swish(g) - sw.swish(-g) - g).max() < 1e-13
    assert np.abs(sw.sigmoid(g) + sw.sigmoid(-g) - 1.0).max() < 1e-15
    assert abs(float(sw.swish(np.array([50.0]))[0]) - 50.0) < 1e-12
    assert abs(float(sw.swish(np.array([-50.0]))[0])) < 1e-18
    assert abs(float(sw.swish_grad(np.array([50.0]))[0]) - 1.0) < 1e-12
    assert abs(float(sw.swish_grad(np.array([-50.0]))[0])) < 1e-18
    # no overflow at the far ends of fp64
    with np.errstate(over="raise", invalid="raise"):
        ends = sw.swish(np.array([-800.0, 800.0]))
    assert abs(ends[0]) < 1e-300 and ends[1] == 800.0
    assert np.abs(sw.swish(g) - np.array([bf_swish(x) for x in g])).max() < 1e-13


def check_swish_grad_fd(sw):
    g = np.linspace(-12, 12, 2401)
    eps = 1e-6
    fd = (sw.swish(g + eps) - sw.swish(g - eps)) / (2 * eps)
    assert np.abs(sw.swish_grad(g) - fd).max() < 1e-8


def check_swiglu_brute_force(sw):
    for seed, (M, h, ffn, t) in enumerate([(3, 5, 8, 2), (4, 3, 6, 3), (2, 7, 4, 1), (5, 4, 12, 4)]):
        r = _rng(200 + seed)
        X, Wg, Wu, Wd = (r.normal(size=s) for s in ((M, h), (h, ffn), (h, ffn), (ffn, h)))
        bG, bU, bY, bZ = bf_swiglu(X.tolist(), Wg.tolist(), Wu.tolist(), Wd.tolist())
        G, U, Y, Z = sw.swiglu_forward(X, Wg, Wu, Wd)
        for a, b in ((G, bG), (U, bU), (Y, bY), (Z, bZ)):
            assert _rel(a, b) < 1e-13
        f = ffn // t
        for i in range(t):
            cols = slice(i * f, (i + 1) * f)
            cG, cU, cY, cZ = bf_swiglu(X.tolist(), Wg[:, cols].tolist(), Wu[:, cols].tolist(),
                                       Wd[cols, :].tolist())
            G_i, U_i, Y_i, Z_i = sw.shard_forward(X, sw.column_shard(Wg, t, i), sw.column_shard(Wu, t, i),
                                                  sw.row_shard(Wd, t, i))
            for a, b in ((G_i, cG), (U_i, cU), (Y_i, cY), (Z_i, cZ)):
                assert _rel(a, b) < 1e-13


def check_swiglu_split_identity(sw):
    """Z = sum_i Z_i, the gate product commutes with the column split, and
    t = 1 is the unsplit block."""
    r = _rng(8)
    M, h, ffn = 16, 24, 64
    X = r.normal(size=(M, h))
    Wg, Wu, Wd = r.normal(size=(h, ffn)) * 0.3, r.normal(size=(h, ffn)) * 0.3, r.normal(size=(ffn, h)) * 0.3
    Z = sw.swiglu_forward(X, Wg, Wu, Wd)[3]
    Y = sw.swiglu_forward(X, Wg, Wu, Wd)[2]
    for t in (1, 2, 8):
        outs = [sw.shard_forward(X, sw.column_shard(Wg, t, i), sw.column_shard(Wu, t, i), sw.row_shard(Wd, t, i))
                for i in range(t)]
        assert _rel(sum(o[3] for o in outs), Z) < 1e-12, t
        assert _rel(np.concatenate([o[2] for o in outs], axis=1), Y) < 1e-15, t


def check_swiglu_gate_limits(sw):
    """Special cases that reduce the block to plainer ones: an up projection
    that yields all ones (a constant input column) leaves a Swish MLP; a gate
    far in the positive range makes Swish the identity, leaving the bilinear
    product (X Wg) * (X Wu); a gate far negative shuts the block off."""
    r = _rng(9)
    M, h, f = 6, 5, 7
    X = r.normal(size=(M, h))
    X[:, -1] = 1.0
    Wg, Wd = r.normal(size=(h, f)), r.normal(size=(f, h))
    Wu = np.zeros((h, f))
    Wu[-1, :] = 1.0
    G, U, Y, Z = sw.swiglu_forward(X, Wg, Wu, Wd)
    assert np.array_equal(U, np.ones((M, f)))
    gg = (X @ Wg).tolist()
    assert _rel(Y, [[bf_swish(v) for v in row] for row in gg]) < 1e-15
    Wg2 = np.zeros((h, f))
    Wg2[-1, :] = 60.0  # G = 60 everywhere, Swish(60) = 60 to fp64 precision
    Wu2 = r.normal(size=(h, f))
    Y2 = sw.swiglu_forward(X, Wg2, Wu2, Wd)[2]
    assert _rel(Y2, 60.0 * (X @ Wu2)) < 1e-15
    Y3 = sw.swiglu_forward(X, -Wg2, Wu2, Wd)[2]
    assert np.abs(Y3).max() < 1e-20 * np.abs(X @ Wu2).max()


def _sw_loss(sw, X, Wg, Wu, Wd, dZ):
    return float((sw.shard_forward(X, Wg, Wu, Wd)[3] * dZ).sum())


def check_swiglu_backward_fd(sw):
    """Every entry of dX_i, dWg_i, dWu_i, dWd_i equals a central difference of
    L = <dZ, Z_i(X, Wg_i, Wu_i, Wd_i)>, on tiny shapes."""
    eps = 1e-6
    r = _rng(22)
    M, h, f = 3, 4, 5
    X, Wg, Wu, Wd, dZ = (r.normal(size=s) for s in ((M, h), (h, f), (h, f), (f, h), (M, h)))
    g = sw.shard_backward(X, Wg, Wu, Wd, X @ Wg, X @ Wu, dZ)
    for name, P in (("dX", X), ("dWg", Wg), ("dWu", Wu), ("dWd", Wd)):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + eps
            lp = _sw_loss(sw, X, Wg, Wu, Wd, dZ)
            P[idx] = old - eps
            lm = _sw_loss(sw, X, Wg, Wu, Wd, dZ)
            P[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        assert _rel(g[name], fd) < 1e-6, (name, _rel(g[name], fd))
    G, U = X @ Wg, X @ Wu
    assert _rel(g["Y"], [[bf_swish(a) * b for a, b in zip(ga, ua)] for ga, ua in zip(G.tolist(), U.tolist())]) < 1e-15
    # the two pre-activation gradients are the derivative of L through Y_i
    for name, P in (("dG", G), ("dU", U)):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + eps
            Yp = [[bf_swish(a) * b for a, b in zip(ga, ua)] for ga, ua in zip(G.tolist(), U.tolist())]
            P[idx] = old - eps
            Ym = [[bf_swish(a) * b for a, b in zip(ga, ua)] for ga, ua in zip(G.tolist(), U.tolist())]
            P[idx] = old
            fd[idx] = float(((np.array(Yp) - np.array(Ym)) @ Wd * dZ).sum()) / (2 * eps)
        assert _rel(g[name], fd) < 1e-6, (name, _rel(g[name], fd))


def check_swiglu_backward_directional(sw):
    """At a moderate size: <dP, D> equals the central difference of L along a
    random direction D, for every operand P."""
    r = _rng(32)
    M, h, f = 48, 40, 56
    X = r.normal(size=(M, h))
    Wg, Wu, Wd = r.normal(size=(h, f)) * 0.2, r.normal(size=(h, f)) * 0.2, r.normal(size=(f, h)) * 0.2
    dZ = r.normal(size=(M, h))
    g = sw.shard_backward(X, Wg, Wu, Wd, X @ Wg, X @ Wu, dZ)
    eps = 1e-5
    for k, name in enumerate(("dX", "dWg", "dWu", "dWd")):
        args = [X, Wg, Wu, Wd]
        D = r.normal(size=args[k].shape)
        ap = args[:k] + [args[k] + eps * D] + args[k + 1:]
        am = args[:k] + [args[k] - eps * D] + args[k + 1:]
        fd = (_sw_loss(sw, *ap, dZ) - _sw_loss(sw, *am, dZ)) / (2 * eps)
        an = float((g[name] * D).sum())
        assert abs(an - fd) <= 1e-7 * max(1.0, abs(fd)), (name, an, fd)


def check_swiglu_backward_shards(sw):
    """Concatenated weight gradients of the t shards equal the unsplit
    block's, and the sum of the partials dX_i equals the unsplit dX."""
    r = _rng(42)
    M, h, ffn, t = 20, 16, 48, 4
    X, dZ = r.normal(size=(M, h)), r.normal(size=(M, h))
    Wg, Wu, Wd = r.normal(size=(h, ffn)) * 0.3, r.normal(size=(h, ffn)) * 0.3, r.normal(size=(ffn, h)) * 0.3
    full = sw.swiglu_backward(X, Wg, Wu, Wd, dZ)
    parts = []
    for i in range(t):
        Wg_i, Wu_i, Wd_i = sw.column_shard(Wg, t, i), sw.column_shard(Wu, t, i), sw.row_shard(Wd, t, i)
        parts.append(sw.shard_backward(X, Wg_i, Wu_i, Wd_i, X @ Wg_i, X @ Wu_i, dZ))
    for name, ax in (("dWg", 1), ("dWu", 1), ("dWd", 0), ("dG", 1), ("dU", 1)):
        assert _rel(np.concatenate([p[name] for p in parts], axis=ax), full[name]) < 1e-13, name
    assert _rel(sum(p["dX"] for p in parts), full["dX"]) < 1e-12


# ------------------------------------------------------------------- CE checks

def check_xent_hand_example(xent):
    g = read_rows("xent_hand_example.txt")
    H, E = np.array(g["H"]), np.array(g["E"])
    y = np.array(g["targets"][0], dtype=np.int64)
    want = np.array(g["loss"][0])
    assert _rel(xent.naive_loss(H.repeat(4, 0), E, y), want) < 1e-15
    assert _rel(xent.vocab_parallel_loss(H.repeat(4, 0), E, y, 2), want) < 1e-15
    H4 = H.repeat(4, 0)
    m0, l0, T0, a0 = xent.shard_partials(H4, E[0:2], y, 0)
    m1, l1, T1, a1 = xent.shard_partials(H4, E[2:4], y, 2)
    assert np.all(np.abs(m0 - g["m0"][0][0]) < 1e-16) and np.all(np.abs(l0 - g["l0"][0][0]) < 1e-15)
    assert np.all(np.abs(m1 - g["m1"][0][0]) < 1e-16) and np.all(np.abs(l1 - g["l1"][0][0]) < 1e-15)
    # targets 0, 1 are rank 0's, targets 2, 3 rank 1's; the other rank's T is +0.0
    z = E[:, 0]
    assert list(T0) == [z[0], z[1], 0.0, 0.0] and list(T1) == [0.0, 0.0, z[2], z[3]]
    assert np.all(a0 == int(g["argmax0"][0][0])) and np.all(a1 == int(g["argmax1"][0][0]))
    am = xent.merge_argmax(np.stack([m0, m1]), np.stack([a0, a1]))
    assert np.all(am == int(g["argmax"][0][0]))


def check_xent_brute_force(xent):
    r = _rng(51)
    M, h, V, t = 6, 5, 16, 4
    H, E = r.normal(size=(M, h)), r.normal(size=(V, h))
    y = r.integers(0, V, size=M)
    want = bf_xent(H.tolist(), E.tolist(), y.tolist())
    assert _rel(xent.naive_loss(H, E, y, chunk=4), want) < 1e-13
    assert _rel(xent.vocab_parallel_loss(H, E, y, t), want) < 1e-13
    # per-rank partials by loops
    n = V // t
    for rank in range(t):
        m, l, T, am = xent.shard_partials(H, E[rank * n:(rank + 1) * n], y, rank * n)
        for k in range(M):
            z = [sum(H[k, c] * E[j, c] for c in range(h)) for j in range(rank * n, (rank + 1) * n)]
            mx = max(z)
            assert abs(m[k] - mx) < 1e-13
            assert abs(l[k] - sum(math.exp(v - mx) for v in z)) < 1e-12
            if rank * n <= y[k] < (rank + 1) * n:
                assert abs(T[k] - z[y[k] - rank * n]) < 1e-13
            else:
                assert T[k] == 0.0 and not math.copysign(1.0, T[k]) < 0
            assert am[k] == rank * n + z.index(mx)


def check_xent_fused_equals_naive(xent):
    r = _rng(61)
    M, h, V = 64, 32, 1024
    H, E = r.normal(size=(M, h)), r.normal(size=(V, h)) * 0.5
    y = r.integers(0, V, size=M)
    base = xent.naive_loss(H, E, y, chunk=17)
    for t in (1, 2, 8, 16):
        assert _rel(xent.vocab_parallel_loss(H, E, y, t), base) < 1e-12, t
    # the merge does not depend on the rank order
    parts = [xent.shard_partials(H, E[a:a + 128], y, a) for a in range(0, V, 128)]
    m, l, T = (np.stack([p[j] for p in parts]) for j in range(3))
    perm = r.permutation(len(parts))
    assert np.abs(xent.merge(m[perm], l[perm], T[perm]) - xent.merge(m, l, T)).max() < 1e-13
    # t = 1: the partials give the loss directly
    m1, l1, T1, _ = xent.shard_partials(H, E, y, 0)
    assert _rel(m1 + np.log(l1) - T1, base) < 1e-13


def check_xent_uniform(xent):
    """E = 0: every logit is 0, so the loss is ln V, each rank's max is 0 and
    its sum-exp is its slice size."""
    V, t = 51200, 8
    H = _rng(71).normal(size=(3, 8))
    E = np.zeros((V, 8))
    y = np.array([0, 25600, 51199])
    loss = xent.vocab_parallel_loss(H, E, y, t)
    assert np.abs(loss - math.log(51200)).max() < 1e-12
    assert abs(math.log(51200) - 10.843494811027599) < 1e-15
    m, l, T, am = xent.shard_partials(H, E[:6400], y, 0)
    assert np.all(m == 0.0) and np.all(l == 6400.0) and np.all(T == 0.0)
    assert np.all(am == 0)  # all tied: the lowest id


def check_xent_shift(xent):
    """A large common shift of every logit of a token leaves its loss
    unchanged (the max subtraction; a plain exp would overflow)."""
    r = _rng(81)
    M, h, V = 8, 6, 64
    H, E = r.normal(size=(M, h)), r.normal(size=(V, h))
    y = r.integers(0, V, size=M)
    base = xent.naive_loss(H, E, y)
    H2 = np.concatenate([H, np.full((M, 1), 1000.0)], axis=1)
    E2 = np.concatenate([E, np.ones((V, 1))], axis=1)
    for fn in (lambda: xent.naive_loss(H2, E2, y), lambda: xent.vocab_parallel_loss(H2, E2, y, 4)):
        got = fn()
        assert np.all(np.isfinite(got))
        assert np.abs(got - base).max() < 1e-9


def check_xent_argmax_ties(xent):
    """Exact ties resolve to the lowest global id, within and across ranks."""
    H = np.array([[1.0, 0.0], [0.0, 1.0]])
    E = np.array([[0.0, 0.0], [2.0, 1.0], [1.0, 3.0], [2.0, 3.0], [0.0, 0.0], [2.0, 0.0]])
    # token 0 logits: 0 2 1 2 0 2 -> max 2 at ids 1, 3, 5 -> 1
    # token 1 logits: 0 1 3 3 0 0 -> max 3 at ids 2, 3 -> 2
    parts = [xent.shard_partials(H, E[a:a + 2], np.array([0, 0]), a) for a in (0, 2, 4)]
    m = np.stack([p[0] for p in parts])
    am = np.stack([p[3] for p in parts])
    assert list(xent.merge_argmax(m, am)) == [1, 2]


# ---------------------------------------------------------- CE backward checks

def _bf_weighted_loss(H, E, y, w):
    return sum(wk * lk for wk, lk in zip(w, bf_xent(H.tolist(), E.tolist(), list(y))))


def check_xent_backward_fd(xent):
    """Every entry of dH and dE equals a central difference of
    L = sum_k w_k loss_k(H, E), the loss evaluated by brute-force loops."""
    r = _rng(51)
    M, h, V = 3, 4, 7
    H, E = r.normal(size=(M, h)), r.normal(size=(V, h))
    y = np.array([2, 0, 6])
    w = np.array([0.5, -1.25, 2.0])
    g = xent.xent_backward(H, E, y, w)
    eps = 1e-6
    for name, P in (("dH", H), ("dE", E)):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + eps
            lp = _bf_weighted_loss(H, E, y, w)
            P[idx] = old - eps
            lm = _bf_weighted_loss(H, E, y, w)
            P[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        assert _rel(g[name], fd) < 1e-7, (name, _rel(g[name], fd))
    # G is the derivative with respect to the logits themselves
    z = H @ E.T
    fd = np.zeros_like(z)
    for k in range(M):
        for j in range(V):
            zp, zm = z[k].copy(), z[k].copy()
            zp[j] += eps
            zm[j] -= eps
            lse = lambda v: max(v) + math.log(sum(math.exp(x - max(v)) for x in v))
            fd[k, j] = w[k] * ((lse(zp) - zp[y[k]]) - (lse(zm) - zm[y[k]])) / (2 * eps)
    assert _rel(g["G"], fd) < 1e-7


def check_xent_backward_default_weights(xent):
    """dloss omitted means weight 1 per token; each row of G then sums to 0
    (softmax sums to 1, the one-hot to 1), and G's target entries are p - 1."""
    r = _rng(52)
    H, E = r.normal(size=(9, 5)), r.normal(size=(13, 5))
    y = r.integers(0, 13, size=9)
    g1 = xent.xent_backward(H, E, y)
    gw = xent.xent_backward(H, E, y, np.ones(9))
    assert np.array_equal(g1["G"], gw["G"])
    assert np.abs(g1["G"].sum(axis=1)).max() < 1e-14
    assert np.all(g1["G"][np.arange(9), y] < 0) and np.all(g1["G"][np.arange(9), y] > -1)
    off = np.ones_like(g1["G"], dtype=bool)
    off[np.arange(9), y] = False
    assert np.all(g1["G"][off] > 0)


def check_xent_backward_zero_embedding(xent):
    """E = 0: every logit is 0, so G = 1/V - onehot, dH = 0, and
    dE_j = sum_k w_k (1/V - [y_k = j]) H_k, for the unsplit form and the
    shards with lse = ln V."""
    r = _rng(53)
    M, h, V, t = 6, 4, 12, 3
    H, E = r.normal(size=(M, h)), np.zeros((V, h))
    y = np.array([0, 5, 5, 11, 3, 7])
    w = r.uniform(0.5, 2.0, size=M)
    want_G = np.full((M, V), 1.0 / V)
    want_G[np.arange(M), y] -= 1.0
    want_G *= w[:, None]
    want_dE = np.zeros((V, h))
    for k in range(M):
        for j in range(V):
            want_dE[j] += w[k] * ((1.0 / V) - (1.0 if y[k] == j else 0.0)) * H[k]
    g = xent.xent_backward(H, E, y, w)
    assert _rel(g["G"], want_G) < 1e-15 and np.abs(g["dH"]).max() == 0.0
    assert _rel(g["dE"], want_dE) < 1e-14
    Vr = V // t
    lse = np.full(M, math.log(V))
    for rk in range(t):
        gs = xent.shard_backward(H, E[rk * Vr:(rk + 1) * Vr], y, rk * Vr, lse, w)
        assert _rel(gs["G"], want_G[:, rk * Vr:(rk + 1) * Vr]) < 1e-15
        assert _rel(gs["dE"], want_dE[rk * Vr:(rk + 1) * Vr]) < 1e-14


def check_xent_merge_lse(xent):
    """The merged lse of the ranks' partials equals ln sum_j exp(z_kj) by
    brute-force loops, and is unchanged by a constant shift of a token's
    logits (up to that shift) and by the order of the ranks."""
    r = _rng(54)
    M, h, V, t = 5, 6, 20, 4
    H, E = r.normal(size=(M, h)) * 3, r.normal(size=(V, h))
    Vr = V // t
    parts = [xent.shard_partials(H, E[k * Vr:(k + 1) * Vr], np.zeros(M, dtype=np.int64), k * Vr)
             for k in range(t)]
    m, l = np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])
    lse = xent.merge_lse(m, l)
    z = (H @ E.T).tolist()
    want = [math.log(sum(math.exp(v) for v in row)) for row in z]
    assert _rel(lse, want) < 1e-14
    perm = [2, 0, 3, 1]
    assert _rel(xent.merge_lse(m[perm], l[perm]), lse) < 1e-15
    assert _rel(xent.merge_lse(m + 1000.0, l), lse + 1000.0) < 1e-15


def check_xent_backward_shards(xent):
    """Sum over ranks of dH_r equals the unsplit dH, the ranks' dE_r stacked
    equal dE, and their G_r side by side equal G, with lse merged from the
    ranks' own partials."""
    r = _rng(55)
    M, h, V, t = 24, 16, 8 * 40, 8
    H, E = r.normal(size=(M, h)), r.normal(size=(V, h)) * 0.5
    y = r.integers(0, V, size=M)
    w = r.normal(size=M)
    full = xent.xent_backward(H, E, y, w)
    Vr = V // t
    parts = [xent.shard_partials(H, E[k * Vr:(k + 1) * Vr], y, k * Vr) for k in range(t)]
    lse = xent.merge_lse(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    sh = [xent.shard_backward(H, E[k * Vr:(k + 1) * Vr], y, k * Vr, lse, w) for k in range(t)]
    assert _rel(sum(g["dH"] for g in sh), full["dH"]) < 1e-12
    assert _rel(np.concatenate([g["dE"] for g in sh], axis=0), full["dE"]) < 1e-12
    assert _rel(np.concatenate([g["G"] for g in sh], axis=1), full["G"]) < 1e-12


# ---------------------------------------------------------------- SP checks

def check_sp_reduce_scatter_brute(sp):
    """Each rank's chunk equals the element-by-element sum of the parts over
    its rows, by loops over the (s, b) index pairs that land in the chunk."""
    r_ = _rng(61)
    s, b, h, t = 8, 3, 5, 4
    parts = [r_.integers(-50, 50, size=(s * b, h)).astype(np.float64) for _ in range(t)]
    for r in range(t):
        got = sp.reduce_scatter(parts, s, b, t, r)
        want = []
        for si in range(r * s // t, (r + 1) * s // t):
            for bi in range(b):
                k = si * b + bi
                want.append([sum(p[k, c] for p in parts) for c in range(h)])
        assert np.array_equal(got, np.array(want)), r


def check_sp_identity(sp):
    """All-gather of every rank's reduce-scatter = the all-reduce (the sum of
    the partials), exactly; and the chunks tile the token axis in rank order."""
    r_ = _rng(62)
    s, b, h = 16, 2, 7
    for t in (1, 2, 4, 8):
        parts = [r_.normal(size=(s * b, h)) for _ in range(t)]
        chunks = [sp.reduce_scatter(parts, s, b, t, r) for r in range(t)]
        full = sp.all_gather(chunks, s, b, t)
        want = parts[0].copy()
        for p in parts[1:]:
            want = want + p
        assert np.array_equal(full, want), t
        bounds = [sp.chunk_rows(s, b, t, r) for r in range(t)]
        assert bounds[0][0] == 0 and bounds[-1][1] == s * b
        assert all(bounds[i][1] == bounds[i + 1][0] for i in range(t - 1))


def check_sp_volume(sp):
    """The section's identity: (t-1)/t M + (t-1)/t M = 2 (t-1)/t M, and at
    t = 8 each rank sends 7/8 of the tensor per half."""
    for t in (2, 4, 8):
        n = 8 * 1024 * 3072
        rs, ag, ar = (sp.comm_volume(k, t, n) for k in ("reduce_scatter", "all_gather", "all_reduce"))
        assert rs + ag == ar == 2 * (t - 1) * n / t
    assert sp.comm_volume("all_gather", 8, 8) == 7.0


def _ln_row_loops(row, gamma, beta, eps):
    n = len(row)
    mean = math.fsum(row) / n
    var = math.fsum((v - mean) ** 2 for v in row) / n
    inv = 1.0 / math.sqrt(var + eps)
    return [(v - mean) * inv * g + bb for v, g, bb in zip(row, gamma, beta)]


def check_sp_layernorm_brute(sp):
    """LayerNorm against loops per row (math.fsum means, the biased
    variance, eps inside the square root, per-feature gamma and beta)."""
    r_ = _rng(63)
    x = r_.normal(size=(4, 7)) * 3 + 1
    g, b = r_.normal(size=7), r_.normal(size=7)
    for eps in (1e-5, 0.5):
        want = np.array([_ln_row_loops(list(row), g, b, eps) for row in x])
        assert _rel(sp.layernorm(x, g, b, eps), want) < 1e-13, eps


def check_sp_layernorm_closed_forms(sp):
    """A constant row normalises to beta exactly; with gamma = 1, beta = 0 a
    row comes out with mean 0 and variance var / (var + eps); with eps = 0 the
    result does not change when the row is scaled by a > 0 and shifted."""
    r_ = _rng(64)
    h = 9
    g, b = r_.normal(size=h), r_.normal(size=h)
    c = np.full((2, h), 3.25)
    assert np.array_equal(sp.layernorm(c, g, b, 1e-5), np.stack([b, b]))
    x = r_.normal(size=(5, h)) * 0.01
    y = sp.layernorm(x, np.ones(h), np.zeros(h), 1e-5)
    v = x.var(axis=1)
    assert np.abs(y.mean(axis=1)).max() < 1e-12
    assert _rel(y.var(axis=1), v / (v + 1e-5)) < 1e-10
    assert _rel(sp.layernorm(2.5 * x - 7.0, g, b, 0.0), sp.layernorm(x, g, b, 0.0)) < 1e-9


def check_sp_layernorm_library(sp):
    """The library routine (torch.nn.functional.layer_norm in float64 on the
    CPU) as a special case."""
    import torch
    r_ = _rng(65)
    x, g, b = r_.normal(size=(6, 40)), r_.normal(size=40), r_.normal(size=40)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), torch.from_numpy(b),
                                          1e-5).numpy()
    assert _rel(sp.layernorm(x, g, b, 1e-5), want) < 1e-12


def check_sp_exit_region_brute(sp):
    """Rank r's region by loops: every element of its chunk summed over the
    ranks' partials, masked and scaled, added to the residual, then each row
    normalised by the loop LayerNorm."""
    r_ = _rng(66)
    s, b, h, t = 6, 2, 5, 3
    parts = [r_.normal(size=(s * b, h)) for _ in range(t)]
    n = (s // t) * b
    res = r_.normal(size=(n, h))
    keep = (r_.random(size=(n, h)) > 0.3).astype(np.uint8)
    g, bb = r_.normal(size=h), r_.normal(size=h)
    for r in range(t):
        hs, y = sp.exit_region(parts, s, b, t, r, res, g, bb, 1e-5, keep, 1 / 0.7)
        for j in range(n):
            k = r * n + j
            row = [res[j, c] + math.fsum(p[k, c] for p in parts) * (1 / 0.7 if keep[j, c] else 0.0)
                   for c in range(h)]
            assert _rel(hs[j], row) < 1e-13, (r, j)
            assert _rel(y[j], _ln_row_loops(row, g, bb, 1e-5)) < 1e-12, (r, j)


def check_sp_exit_region_split_identity(sp):
    """The ranks' chunks, gathered in rank order, equal the region computed on
    the whole tensor after the all-reduce (LayerNorm works per token, so the
    split along the sequence changes nothing); a mask of zeros leaves the
    residual alone, and no mask is dropout off."""
    r_ = _rng(67)
    s, b, h = 8, 3, 6
    for t in (1, 2, 4):
        parts = [r_.normal(size=(s * b, h)) for _ in range(t)]
        res = r_.normal(size=(s * b, h))
        keep = (r_.random(size=(s * b, h)) > 0.1).astype(np.uint8)
        g, bb = r_.normal(size=h), r_.normal(size=h)
        n = (s // t) * b
        out = [sp.exit_region(parts, s, b, t, r, res[r * n:(r + 1) * n], g, bb, 1e-5, keep[r * n:(r + 1) * n],
                              1 / 0.9) for r in range(t)]
        z = sum(parts)
        full_h = res + z * keep / 0.9
        assert _rel(np.concatenate([o[0] for o in out]), full_h) < 1e-13
        assert _rel(np.concatenate([o[1] for o in out]), sp.layernorm(full_h, g, bb, 1e-5)) < 1e-12
        hs0, _ = sp.exit_region(parts, s, b, t, 0, res[:n], g, bb, 1e-5, np.zeros((n, h), np.uint8), 2.0)
        assert np.array_equal(hs0, res[:n])
        hs1, _ = sp.exit_region(parts, s, b, t, 0, res[:n], g, bb)
        assert _rel(hs1, res[:n] + z[:n]) < 1e-13


def _fd(f, x, i, step=1e-6):
    xp, xm = x.copy(), x.copy()
    xp.flat[i] += step
    xm.flat[i] -= step
    return (f(xp) - f(xm)) / (2 * step)


def check_sp_layernorm_backward_fd(sp):
    """dx, dgamma, dbeta of LayerNorm against central finite differences of
    L = sum(w * layernorm(x, gamma, beta)), every element."""
    r_ = _rng(68)
    x, g, b, w = r_.normal(size=(3, 6)), r_.normal(size=6), r_.normal(size=6), r_.normal(size=(3, 6))
    eps = 1e-3
    dx, dg, db = sp.layernorm_backward(x, g, w, eps)
    for i in range(x.size):
        assert abs(_fd(lambda v: (w * sp.layernorm(v, g, b, eps)).sum(), x, i) - dx.flat[i]) < 1e-7, i
    for i in range(6):
        assert abs(_fd(lambda v: (w * sp.layernorm(x, v, b, eps)).sum(), g, i) - dg[i]) < 1e-7, i
        assert abs(_fd(lambda v: (w * sp.layernorm(x, g, v, eps)).sum(), b, i) - db[i]) < 1e-7, i


def check_sp_layernorm_backward_closed_forms(sp):
    """A row's dx sums to zero (the output ignores a shift of the row); with
    eps = 0 it is also orthogonal to the normalised row (the output ignores a
    scaling); dbeta is the column sum of dy."""
    r_ = _rng(69)
    x, g, dy = r_.normal(size=(5, 11)), r_.normal(size=11), r_.normal(size=(5, 11))
    dx, _, db = sp.layernorm_backward(x, g, dy, 1e-5)
    assert np.abs(dx.sum(axis=1)).max() < 1e-12
    assert np.array_equal(db, dy.sum(axis=0))
    dx0, _, _ = sp.layernorm_backward(x, g, dy, 0.0)
    xc = x - x.mean(axis=1, keepdims=True)
    assert np.abs((dx0 * xc).sum(axis=1)).max() < 1e-12


def check_sp_region_backward_fd(sp):
    """The region's backward against finite differences of
    L = sum(w1 * y) + sum(w2 * hs) through exit_region: g is dL/d(residual),
    dz is dL/d(part_i) on the rank's rows for every i, dgamma and dbeta."""
    r_ = _rng(70)
    s, b, h, t, r = 4, 1, 5, 2, 1
    n = (s // t) * b
    parts = [r_.normal(size=(s * b, h)) for _ in range(t)]
    res, g, bb = r_.normal(size=(n, h)), r_.normal(size=h), r_.normal(size=h)
    keep = (r_.random(size=(n, h)) > 0.3).astype(np.uint8)
    w1, w2 = r_.normal(size=(n, h)), r_.normal(size=(n, h))
    eps, sc = 1e-3, 1.5

    def loss(P=parts, R=res, G=g, B=bb):
        hs_, y_ = sp.exit_region(P, s, b, t, r, R, G, B, eps, keep, sc)
        return (w1 * y_).sum() + (w2 * hs_).sum()
    hs, _ = sp.exit_region(parts, s, b, t, r, res, g, bb, eps, keep, sc)
    out = sp.exit_region_backward(hs, g, w1, w2, eps, keep, sc)
    for i in range(res.size):
        assert abs(_fd(lambda v: loss(R=v), res, i) - out["g"].flat[i]) < 1e-6, i
    a = r * n * h
    for k in range(t):
        for i in range(n * h):
            def lk(v, k=k):
                P = [p.copy() for p in parts]
                P[k] = v
                return loss(P=P)
            assert abs(_fd(lk, parts[k], a + i) - out["dz"].flat[i]) < 1e-6, (k, i)
    for i in range(h):
        assert abs(_fd(lambda v: loss(G=v), g, i) - out["dgamma"][i]) < 1e-6, i
        assert abs(_fd(lambda v: loss(B=v), bb, i) - out["dbeta"][i]) < 1e-6, i


def check_sp_region_backward_split(sp):
    """The ranks' dgamma and dbeta add up to those of the whole tensor, and
    their g and dz chunks, gathered, equal the whole tensor's."""
    r_ = _rng(71)
    s, b, h, t = 8, 2, 7, 4
    hs, dy, dhs = r_.normal(size=(s * b, h)), r_.normal(size=(s * b, h)), r_.normal(size=(s * b, h))
    keep = (r_.random(size=(s * b, h)) > 0.2).astype(np.uint8)
    g = r_.normal(size=h)
    full = sp.exit_region_backward(hs, g, dy, dhs, 1e-5, keep, 1.25)
    n = (s // t) * b
    ch = [sp.exit_region_backward(hs[k * n:(k + 1) * n], g, dy[k * n:(k + 1) * n], dhs[k * n:(k + 1) * n], 1e-5,
                                  keep[k * n:(k + 1) * n], 1.25) for k in range(t)]
    assert _rel(sum(c["dgamma"] for c in ch), full["dgamma"]) < 1e-12
    assert _rel(sum(c["dbeta"] for c in ch), full["dbeta"]) < 1e-12
    assert _rel(np.concatenate([c["g"] for c in ch]), full["g"]) < 1e-13
    assert _rel(np.concatenate([c["dz"] for c in ch]), full["dz"]) < 1e-13


SP_CHECKS = [check_sp_reduce_scatter_brute, check_sp_identity, check_sp_volume, check_sp_layernorm_brute,
             check_sp_layernorm_closed_forms, check_sp_layernorm_library, check_sp_exit_region_brute,
             check_sp_exit_region_split_identity, check_sp_layernorm_backward_fd,
             check_sp_layernorm_backward_closed_forms, check_sp_region_backward_fd, check_sp_region_backward_split]


# ------------------------------------------------------ attention projections

def check_attn_core_brute(at):
    """The attention core against loops: every query head's softmax row by
    math.exp, the scores scaled by 1/sqrt(d), query head k reading KV head
    k // (n_q / n_kv)."""
    r_ = _rng(71)
    M, n_q, n_kv, d = 4, 4, 2, 3
    QKV = r_.normal(size=(M, (n_q + 2 * n_kv) * d))
    got = at.attention_core(QKV, n_q, n_kv, d)
    for k in range(n_q):
        g = k // (n_q // n_kv)
        for i in range(M):
            q = QKV[i, k * d:(k + 1) * d]
            sc = [sum(q[c] * QKV[j, (n_q + g) * d + c] for c in range(d)) / math.sqrt(d) for j in range(M)]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            tot = sum(e)
            for c in range(d):
                want = sum(e[j] / tot * QKV[j, (n_q + n_kv + g) * d + c] for j in range(M))
                assert abs(got[i, k * d + c] - want) < 1e-13


def check_attn_projections_brute(at):
    """The rank's fused weight holds its heads' columns (by explicit head
    index loops), and the projections are plain products (brute force)."""
    r_ = _rng(72)
    M, h, n_q, n_kv, d, t = 3, 5, 4, 2, 2, 2
    Wq, Wk, Wv = r_.normal(size=(h, n_q * d)), r_.normal(size=(h, n_kv * d)), r_.normal(size=(h, n_kv * d))
    Wo = r_.normal(size=(n_q * d, h))
    X = r_.normal(size=(M, h))
    for i in range(t):
        W = at.qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, i)
        cols = []
        for k in range(i * n_q // t, (i + 1) * n_q // t):
            cols += [Wq[:, k * d + c] for c in range(d)]
        for src in (Wk, Wv):
            for k in range(i * n_kv // t, (i + 1) * n_kv // t):
                cols += [src[:, k * d + c] for c in range(d)]
        assert np.array_equal(W, np.stack(cols, axis=1))
        assert _rel(at.qkv_forward(X, W), bf_matmul(X.tolist(), W.tolist())) < 1e-14
        Wo_i = at.out_shard(Wo, n_q, d, t, i)
        rows = [Wo[k * d + c] for k in range(i * n_q // t, (i + 1) * n_q // t) for c in range(d)]
        assert np.array_equal(Wo_i, np.stack(rows, axis=0))
        A = r_.normal(size=(M, n_q // t * d))
        assert _rel(at.out_forward(A, Wo_i), bf_matmul(A.tolist(), Wo_i.tolist())) < 1e-14


def check_attn_split_identity(at):
    """Each rank's heads attended on their own, then its W_O rows: the sum of
    the partials equals the unsplit block, for t = 1, 2, 4 with grouped KV
    heads."""
    r_ = _rng(73)
    M, h, n_q, n_kv, d = 6, 16, 8, 4, 4
    X = r_.normal(size=(M, h))
    Wq, Wk, Wv = (r_.normal(size=(h, n * d)) * 0.3 for n in (n_q, n_kv, n_kv))
    Wo = r_.normal(size=(n_q * d, h)) * 0.3
    full = at.block_forward(X, Wq, Wk, Wv, Wo, n_q, n_kv, d)
    for t in (1, 2, 4):
        parts = []
        for i in range(t):
            qkv = at.qkv_forward(X, at.qkv_shard(Wq, Wk, Wv, n_q, n_kv, d, t, i))
            heads = at.attention_core(qkv, n_q // t, n_kv // t, d)
            parts.append(at.out_forward(heads, at.out_shard(Wo, n_q, d, t, i)))
        assert _rel(sum(parts), full) < 1e-13, t


def check_attn_backward_fd(at):
    """Gradients of L = <dY, X Wqkv> and L = <dZ, A Wo> by central
    differences, every entry."""
    r_ = _rng(74)
    X, W, dY = r_.normal(size=(3, 4)), r_.normal(size=(4, 5)), r_.normal(size=(3, 5))
    g = at.qkv_backward(X, W, dY)
    A, Wo, dZ = r_.normal(size=(3, 2)), r_.normal(size=(2, 4)), r_.normal(size=(3, 4))
    go = at.out_backward(A, Wo, dZ)
    eps = 1e-6
    for name, P, fwd, args, dd in (("dX", X, at.qkv_forward, (X, W), g["dX"]),
                                   ("dW", W, at.qkv_forward, (X, W), g["dW"]),
                                   ("dA", A, at.out_forward, (A, Wo), go["dA"]),
                                   ("dWo", Wo, at.out_forward, (A, Wo), go["dW"])):
        up = dY if fwd is at.qkv_forward else dZ
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + eps
            lp = float((fwd(*args) * up).sum())
            P[idx] = old - eps
            lm = float((fwd(*args) * up).sum())
            P[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        assert _rel(dd, fd) < 1e-8, name


ATTN_CHECKS = [check_attn_core_brute, check_attn_projections_brute, check_attn_split_identity,
               check_attn_backward_fd]


MLP_CHECKS = [check_gelu_table, check_gelu_shape, check_gelu_grad_fd, check_mlp_hand_example,
              check_mlp_brute_force, check_split_identity, check_partial_sum_exact,
              check_backward_fd, check_backward_directional, check_backward_shards]
SWIGLU_CHECKS = [check_swish_closed_forms, check_swish_grad_fd, check_swiglu_brute_force,
                 check_swiglu_split_identity, check_swiglu_gate_limits, check_swiglu_backward_fd,
                 check_swiglu_backward_directional, check_swiglu_backward_shards]
XENT_CHECKS = [check_xent_hand_example, check_xent_brute_force, check_xent_fused_equals_naive,
               check_xent_uniform, check_xent_shift, check_xent_argmax_ties]
XENT_BWD_CHECKS = [check_xent_backward_fd, check_xent_backward_default_weights,
                   check_xent_backward_zero_embedding, check_xent_merge_lse, check_xent_backward_shards]

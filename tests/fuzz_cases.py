"""Seeded random shapes for the randomized parity tests (test_gpu_fuzz.py)
and the debug build's bounds checks (test_debug_build.py).  Plain Python and
numpy only: importing this module draws the same cases every time."""

import numpy as np

_rng = np.random.default_rng(20261202)


def _w8(lo, hi):
    """A width in [lo, hi], a multiple of 8 (16-byte bf16 rows)."""
    return 8 * int(_rng.integers(lo // 8, hi // 8 + 1))


def _tokens():
    """(b, s): mostly ragged counts, some single tokens and exact multiples of 256."""
    kind = _rng.integers(0, 6)
    if kind == 0:
        return 1, 1
    if kind == 1:
        return 1, 256 * int(_rng.integers(1, 5))
    return int(_rng.integers(1, 4)), int(_rng.integers(1, 450))


# (b, s, h, ffn, t, rank, act)
MLP_CASES = []
for _ in range(12):
    t = int(_rng.choice([1, 2, 3, 4, 8]))
    b, s = _tokens()
    MLP_CASES.append((b, s, _w8(8, 1100), t * _w8(8, 1100 // t if t > 1 else 1100), t,
                      int(_rng.integers(0, t)), str(_rng.choice(["erf", "tanh"]))))

# (b, s, h, vocab, t)
XENT_CASES = []
for _ in range(10):
    t = int(_rng.choice([1, 2, 3, 4, 8]))
    b, s = _tokens()
    XENT_CASES.append((b, s, _w8(8, 384), t * _w8(8, 2000), t))

# (b, s, h, ffn, t, rank)
SWIGLU_CASES = []
for _ in range(6):
    t = int(_rng.choice([1, 2, 4, 8]))
    b, s = _tokens()
    SWIGLU_CASES.append((b, s, _w8(8, 800), t * _w8(8, 800 // t if t > 1 else 800), t, int(_rng.integers(0, t))))

# (b, s, h, n_q, n_kv, d, t, rank): heads divisible by t, n_q a multiple of n_kv
ATTN_CASES = []
for _ in range(6):
    t = int(_rng.choice([1, 2, 4, 8]))
    n_kv = t * int(_rng.integers(1, 3))
    n_q = n_kv * int(_rng.choice([1, 2, 4]))
    b, s = _tokens()
    ATTN_CASES.append((b, s, _w8(8, 1400), n_q, n_kv, _w8(8, 136), t, int(_rng.integers(0, t))))

# (t, n, bf16 output)
SUM_CASES = [(int(_rng.integers(1, 13)), int(_rng.integers(1, 70000)), bool(_rng.integers(0, 2)))
             for _ in range(8)]

# (t, s, b, h, rank, masked): the fused sequence-parallel region
SPLN_CASES = []
for _ in range(6):
    t = int(_rng.choice([1, 2, 4, 8]))
    SPLN_CASES.append((t, t * int(_rng.integers(1, 40)), int(_rng.integers(1, 5)), _w8(8, 16384),
                       int(_rng.integers(0, t)), bool(_rng.integers(0, 2))))

# A second batch, drawn after every case above so those stay the same: wider
# MLP blocks (multi-tile in every dimension, up to 2100) and CE slices with a
# larger hidden size, to reach the 256-wide tiles and several rounds of blocks.
for _ in range(6):
    t = int(_rng.choice([1, 2, 4, 8]))
    b, s = int(_rng.integers(1, 3)), int(_rng.integers(300, 1100))
    MLP_CASES.append((b, s, _w8(520, 2100), t * _w8(136, max(136, 2100 // t)), t,
                      int(_rng.integers(0, t)), str(_rng.choice(["erf", "tanh"]))))
for _ in range(4):
    t = int(_rng.choice([2, 4, 8]))
    b, s = int(_rng.integers(1, 3)), int(_rng.integers(200, 700))
    XENT_CASES.append((b, s, _w8(264, 1040), t * _w8(520, 3000), t))
for _ in range(3):
    t = int(_rng.choice([2, 4, 8]))
    b, s = int(_rng.integers(1, 3)), int(_rng.integers(300, 900))
    SWIGLU_CASES.append((b, s, _w8(520, 1600), t * _w8(136, max(136, 1600 // t)), t, int(_rng.integers(0, t))))
for _ in range(3):
    t = int(_rng.choice([2, 4, 8]))
    n_kv = t * int(_rng.integers(1, 3))
    n_q = n_kv * int(_rng.choice([2, 4]))
    b, s = int(_rng.integers(1, 3)), int(_rng.integers(300, 900))
    ATTN_CASES.append((b, s, _w8(1040, 2100), n_q, n_kv, _w8(64, 136), t, int(_rng.integers(0, t))))
for _ in range(2):
    t = int(_rng.choice([4, 8]))
    SPLN_CASES.append((t, t * int(_rng.integers(100, 300)), int(_rng.integers(1, 5)), _w8(1024, 8192),
                       int(_rng.integers(0, t)), bool(_rng.integers(0, 2))))

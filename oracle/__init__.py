"""Plain fp64 CPU oracle for one tensor-parallel rank's transformer-block shard.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library under ``logit_gemm_shard_amd/`` and imports
nothing from it; both sides only ever see the same seeded input arrays.

Everything here is the plain definition of what the method computes, written
in numpy float64 (BLAS matmul and scipy's ``erf`` are the only library
primitives), with no blocking, fusion or reordering beyond what the pages'
equations state:

* ``oracle.mlp``  -- the GeLU MLP split column-then-row across ``t`` ranks
  (forward, backward and the sum of partials).
* ``oracle.swiglu`` -- the SwiGLU (gated) MLP block with the same split.
* ``oracle.attn`` -- the attention block's QKV column-parallel and W_O
  row-parallel projections (and a plain attention core to check the split).
* ``oracle.sp`` -- the sequence-parallel reduce-scatter exit and all-gather
  entry that replace the row-parallel all-reduce.
* ``oracle.xent`` -- full-logit softmax cross-entropy and its vocab-parallel
  form (per-rank max / sum-exp / target logit, then the merge), and its
  backward (unsplit, and per rank from the merged log-sum-exp).

Every function is pinned by ``tests/test_oracle_*.py`` against things other
than itself: brute-force loops, closed forms, printed normal-table values,
finite differences and algebraic identities.  No function here is "parity
unpinned".
"""

from . import attn, mlp, sp, swiglu, xent  # noqa: F401

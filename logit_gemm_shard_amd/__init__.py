"""logit_gemm_shard_amd: one tensor-parallel rank's transformer-block shard
(GeLU MLP forward/backward, fused vocab-parallel cross-entropy, sum of
partials) as hand-written HIP kernels for gfx950, behind the C ABI of
``include/lgs.h``.

The kernels live in ``liblgs.so`` (built by ``python -m
logit_gemm_shard_amd.build``); ``binding`` exposes the same entry points to
Python with torch tensors.  Importing this package does not load the library:
the first call does, and raises if it is missing.
"""

from .binding import (  # noqa: F401
    LgsError,
    lib,
    mlp_bwd_workspace_bytes,
    mlp_fwd_workspace_bytes,
    shard_partial_sum,
    tp_mlp_bwd,
    tp_mlp_fwd,
    version,
    vocab_parallel_xent_fwd,
    xent_workspace_bytes,
)

"""Helpers for the GPU parity tests: device handling, conversions, the
tolerance metric, and a progress line before every GPU step."""

import sys

import numpy as np
import torch

# max |gpu - ref| / max |ref| per output tensor
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda", 0)


def step(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def f64(x):
    """torch tensor (any device / dtype) or array -> numpy float64."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float32).double().numpy() if x.dtype != torch.float64 \
            else x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def rel_err(got, ref):
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def assert_close(name, got, ref, dtype):
    e = rel_err(got, ref)
    tol = TOL[dtype]
    print(f"    {name}: max|err|/max|ref| = {e:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(f64(got))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: {e:.3e} > {tol}"


def round_like(x64, dtype):
    """fp64 numpy -> torch CPU tensor in dtype (round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x64)).to(dtype)

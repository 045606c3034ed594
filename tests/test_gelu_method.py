"""The erf used by the device GeLU / GeLU' epilogues: Abramowitz & Stegun,
Handbook of Mathematical Functions, formula 7.1.26, with its published
coefficients and error bound |e(z)| <= 1.5e-7 (z >= 0), checked against the
C library's erf.  The device code evaluates the same rational-times-exp form
in fp32; its end-to-end error is checked on the GPU by
test_gpu_parity.py::test_gelu_epilogue_error_bound."""

import math

import numpy as np

P = 0.3275911
A = (0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429)


def as_erf(z, dtype=np.float64):
    z = np.asarray(z, dtype=dtype)
    t = dtype(1.0) / (dtype(1.0) + dtype(P) * z)
    p = dtype(A[4])
    for a in A[3::-1]:
        p = p * t + dtype(a)
    return dtype(1.0) - (p * t) * np.exp(-z * z)


def test_published_error_bound():
    z = np.linspace(0.0, 8.0, 400001)
    ref = np.array([math.erf(v) for v in z])
    assert np.abs(as_erf(z) - ref).max() <= 1.5e-7


def test_fp32_evaluation_stays_near_the_bound():
    # in fp32 the final 1 - P*exp(-z^2) cancels near z = 0 (P*exp -> 1), which
    # adds up to ~4e-7 of rounding to the method's 1.5e-7
    z = np.linspace(0.0, 8.0, 200001).astype(np.float32)
    ref = np.array([math.erf(float(v)) for v in z])
    with np.errstate(over="ignore"):
        err = np.abs(as_erf(z, np.float32).astype(np.float64) - ref).max()
    assert err <= 6e-7, err


def test_phi_from_the_formula_matches_the_normal_table():
    # Phi(u) = 1 - erfc-tail for u >= 0, reflected for u < 0, as the device code does
    for u, phi in [(-2.0, 0.022750131948179195), (-1.0, 0.15865525393145707), (0.0, 0.5),
                   (1.0, 0.8413447460685429), (2.0, 0.9772498680518208), (3.0, 0.9986501019683699)]:
        tail = 0.5 * (1.0 - as_erf(abs(u) / math.sqrt(2.0)))
        got = 1.0 - tail if u >= 0 else tail
        assert abs(got - phi) <= 1e-7

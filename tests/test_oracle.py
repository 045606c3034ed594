"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("check", pins.MLP_CHECKS, ids=lambda f: f.__name__)
def test_mlp_oracle(check):
    check(oracle.mlp)


@pytest.mark.parametrize("check", pins.XENT_CHECKS, ids=lambda f: f.__name__)
def test_xent_oracle(check):
    check(oracle.xent)


@pytest.mark.parametrize("check", pins.SWIGLU_CHECKS, ids=lambda f: f.__name__)
def test_swiglu_oracle(check):
    check(oracle.swiglu)


@pytest.mark.parametrize("check", pins.XENT_BWD_CHECKS, ids=lambda f: f.__name__)
def test_xent_backward_oracle(check):
    check(oracle.xent)


@pytest.mark.parametrize("check", pins.SP_CHECKS, ids=lambda f: f.__name__)
def test_sp_oracle(check):
    check(oracle.sp)


@pytest.mark.parametrize("check", pins.ATTN_CHECKS, ids=lambda f: f.__name__)
def test_attn_oracle(check):
    check(oracle.attn)

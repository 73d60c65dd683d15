import os, sys
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
"""The fp64 oracle against closed forms, identity cases, brute force and invariants."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("choose", ["first", "boundary", "last", "random"])
def test_identity_gather_variants(dtype, choose):
    P.check_identity_gather(dtype, choose)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_brute_variants(dtype):
    P.check_brute_decode(dtype, seed=31)
    P.check_brute_append(dtype, seed=32, causal=True)
    P.check_brute_append(dtype, seed=33, causal=False)
    P.check_count(dtype)

"""The CPU oracle against what the definitions and the mathematics fix
(fixtures, library routines, brute force, closed forms, invariants)."""
import pytest

import oracle
import oracle_checks as oc


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle.load()


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(lib, check):
    check(lib)

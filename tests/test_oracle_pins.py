"""The fp64 oracle pinned to facts fixed outside it (brute force, closed
forms, library routines, invariants). CPU only."""

import pytest

import centroid_checks
import oracle
import oracle_checks


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS + centroid_checks.CENTROID_CHECKS,
                         ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)

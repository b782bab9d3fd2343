"""The fp64 oracle against the pages' worked numbers, closed forms, invariants and
independent library routines (CPU only)."""

import pytest

import oracle.fa_oracle as orc
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(orc)

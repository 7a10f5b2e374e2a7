"""The CPU oracle against its pins (closed forms, invariants, library special
cases, hand-derived examples, brute force).  CPU only."""

import pytest

import oracle.paged_attention as oracle_mod
from tests.oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(check):
    check(oracle_mod)

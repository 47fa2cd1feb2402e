"""The oracle against its pins (closed forms, brute force, library routines, invariants,
and the pages' worked routing arithmetic)."""
import pytest

import oracle.moe_oracle as O
from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(O)

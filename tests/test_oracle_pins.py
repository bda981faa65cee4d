"""The CPU oracle against its pins (values worked by hand from the pages'
equations, closed forms, invariants, brute force, library routines)."""
import pytest

import pins
from oracle import quest_oracle as O


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(O)

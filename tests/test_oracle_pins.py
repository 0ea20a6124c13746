"""The float64 oracle against brute force, torch float64, closed forms,
hand-derived and page-printed values (CPU only)."""
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)

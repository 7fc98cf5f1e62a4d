"""Oracle pins (CPU only): see oracle_pins.py for what each check ties the
oracle to."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()

"""The CPU oracle against its pins (closed forms, brute force, library routines,
values printed on the pages).  See tests/oracle_pins.py for what each pins."""

import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)

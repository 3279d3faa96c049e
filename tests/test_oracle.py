"""CPU oracle against its pins (hand examples, library routines, closed forms,
invariants).  See ``oracle_pins.py`` for what each check fixes."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_mod, check):
    check()

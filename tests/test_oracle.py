"""The CPU oracle against its pins (library routines, closed forms, brute
force, invariants, the stored column table). CPU only."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)

"""The oracle against the pages' printed facts, closed forms, library routines
and invariants (CPU only)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()

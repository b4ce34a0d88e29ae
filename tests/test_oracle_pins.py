"""The oracle against facts other than itself (CPU only; see oracle_pins.py)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    import oracle.oracle as O
    check(O.lib())

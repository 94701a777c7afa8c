"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("name,check", P.ALL_CHECKS, ids=[n for n, _ in P.ALL_CHECKS])
def test_pin(name, check):
    check()

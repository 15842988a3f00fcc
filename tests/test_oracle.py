"""The float64 oracle against its pins (CPU only)."""
import pytest

import oracle as O
import pins


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check(O)

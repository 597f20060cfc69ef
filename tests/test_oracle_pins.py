"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)

"""The CPU oracle against pins that do not come from the oracle itself."""
import pytest

import oracle
from tests import _pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    fails = pin(o)
    assert not fails, "\n".join(fails)

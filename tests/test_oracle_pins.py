"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def test_default_build_has_no_planted_mistake(o):
    assert o.mutant == 0


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)

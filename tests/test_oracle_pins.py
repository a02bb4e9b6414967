"""The CPU oracle pinned to page figures, closed forms, library routines and brute force."""
import pytest

import pins
from oracle import moe_oracle as O


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)


def test_page_accesses():
    pins.pin_page_accesses()

"""The fp64 oracle against the pages' printed values, closed forms, invariants and
library routines (see pins.py)."""
import pytest

import pins
from oracle import oracle as o


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(o)

"""The fp64 oracle against its pins (closed forms, library routines, the
independent chunked form, the pages' printed sizes).  CPU only."""
import pytest

import oracle_pins
from oracle import gdn_oracle


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(gdn_oracle)

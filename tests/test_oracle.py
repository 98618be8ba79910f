"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle.sfa as orc
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(orc)


def test_mask_rejects_bad_arguments():
    with pytest.raises(ValueError):
        orc.mask("both", 2, 3)
    with pytest.raises(ValueError):
        orc.mask("cross_window", 2, 3, 0)

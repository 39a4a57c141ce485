"""The oracle's grouped and indexed contractions against their pins (no GPU)."""
import pytest

import pins_grouped


@pytest.mark.parametrize("pin", pins_grouped.GROUPED_PINS, ids=lambda f: f.__name__)
def test_grouped_pin(orc, pin):
    pin(orc)

"""The oracle's multi-step epilogue against its pins (no GPU)."""
import pytest

import pins_epilogue


@pytest.mark.parametrize("pin", pins_epilogue.EPILOGUE_PINS, ids=lambda f: f.__name__)
def test_epilogue_pin(orc, pin):
    pin(orc)

"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.FAST_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_toy_shapes_match_pages():
    pins.pin_toy_shapes()


def test_rne_exhaustive_all_binary32_words(orc):
    """binary32 -> binary16 RNE for all 2^32 words against torch's conversion."""
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        words = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        pins.check_rne_words(orc, words)


def test_bf16_rne_exhaustive_all_binary32_words(orc):
    """binary32 -> bfloat16 RNE for all 2^32 words against torch's conversion."""
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        words = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        pins.check_bf16_rne_words(orc, words)

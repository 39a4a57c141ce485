"""The CPU oracle against its pins (no GPU)."""
import concurrent.futures

import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.FAST_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_toy_shapes_match_pages():
    pins.pin_toy_shapes()


def _all_binary32_words(check):
    """Run check(words) over all 2^32 binary32 words in chunks of 2^24, on 8
    threads (the oracle's ctypes calls and torch's conversions release the GIL)."""
    chunk = 1 << 24

    def one(start):
        check(np.arange(chunk, dtype=np.uint32) + np.uint32(start))

    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        list(ex.map(one, range(0, 1 << 32, chunk)))


def test_rne_exhaustive_all_binary32_words(orc):
    """binary32 -> binary16 RNE for all 2^32 words against torch's conversion."""
    _all_binary32_words(lambda words: pins.check_rne_words(orc, words))


def test_bf16_rne_exhaustive_all_binary32_words(orc):
    """binary32 -> bfloat16 RNE for all 2^32 words against torch's conversion."""
    _all_binary32_words(lambda words: pins.check_bf16_rne_words(orc, words))

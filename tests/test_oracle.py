"""The CPU oracle against its pins (closed forms, brute force, textbook
attention, the pages' worked count and invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_threads_reported(oracle_lib):
    assert oracle_lib.threads() >= 1

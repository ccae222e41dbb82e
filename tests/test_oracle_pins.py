"""The CPU oracle against its pins (brute force, closed forms, invariants, the pages)."""

import pytest

import oracle.paged_attention as pa
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(pa)


@pytest.mark.parametrize("pin", oracle_pins.FP8_PINS, ids=lambda f: f.__name__)
def test_fp8_oracle_pin(pin):
    import oracle.fp8_cache as o8
    pin(o8)

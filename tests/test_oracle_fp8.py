"""The FP8 part of the oracle against torch's fp8 conversions, scipy's Hadamard matrix and the
mathematics of the rotation and of the rounding bound (no GPU)."""

import pytest

import oracle_pins_fp8 as pins


@pytest.mark.parametrize("check", pins.FP8_CHECKS, ids=lambda c: c.__name__)
def test_fp8_pin(check):
    check()

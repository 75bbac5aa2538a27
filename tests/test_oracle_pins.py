"""The fp64 oracle against what the pages and the mathematics fix (no GPU)."""

import pytest

import oracle_pins as pins


@pytest.mark.parametrize("check", pins.FORWARD_CHECKS, ids=lambda c: c.__name__)
def test_forward_pin(check):
    check()


@pytest.mark.parametrize("check", pins.BACKWARD_CHECKS, ids=lambda c: c.__name__)
def test_backward_pin(check):
    check()

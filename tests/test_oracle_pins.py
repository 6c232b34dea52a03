"""The CPU oracle against its pins (closed forms, invariants, hand-derived
golden values and plain-Python brute force). Runs on the CPU."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle.svdq_ref)


@pytest.mark.parametrize("check", pins.SLOW_CHECKS, ids=lambda f: f.__name__)
def test_slow_pin(check):
    check(oracle.svdq_ref)

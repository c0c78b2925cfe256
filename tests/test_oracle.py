"""The CPU oracle against its pins (closed forms, fsum, brute force, semantics)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("name,pin", PINS, ids=[n for n, _ in PINS])
def test_oracle_pin(name, pin):
    pin(oracle.default())


def test_tolerance_rule():
    assert oracle.sum_within_tolerance(1.0, 1.0, 0.0)
    assert oracle.sum_within_tolerance(1.0 + 1e-6, 1.0, 0.0)
    assert not oracle.sum_within_tolerance(1.0 + 3e-6, 1.0, 0.0)
    assert oracle.sum_within_tolerance(100.0 + 9e-3, 100.0, 1000.0)
    assert not oracle.sum_within_tolerance(100.0 + 2e-2, 100.0, 1000.0)
    assert oracle.sum_within_tolerance(float("nan"), float("nan"), 0.0)
    assert not oracle.sum_within_tolerance(0.0, float("nan"), 0.0)
    assert oracle.sum_within_tolerance(float("inf"), float("inf"), 0.0)
    assert not oracle.sum_within_tolerance(float("-inf"), float("inf"), 0.0)
    assert oracle.max_equal(-0.0, 0.0)

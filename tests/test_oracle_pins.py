"""The oracle pinned to the pages' printed values, brute force and closed forms."""
import os
import tempfile

import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    assert pin() is None


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13])
def test_pins_reject_planted_mistakes(mutant):
    """Each deliberately broken oracle build fails at least one pin."""
    with tempfile.TemporaryDirectory() as d:
        path = oracle.build(force=True, mutant=mutant, out=os.path.join(d, f"mut{mutant}.so"))
        with oracle.use_library(path):
            failures = pins.failing_pins(tiny_count=60)
    assert failures, f"mutant {mutant} passed every pin"

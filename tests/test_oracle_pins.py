"""The CPU oracle against its pins (closed forms, dense mixture, invariants)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_golden_tiny_regression():
    """The oracle still reproduces the committed record of the tiny workload."""
    import json
    import os

    import numpy as np

    from tests.golden import make_golden

    with open(make_golden.OUT) as f:
        gold = json.load(f)
    now = make_golden.record()
    assert now["input_hash"] == gold["input_hash"]
    assert now["ids"] == gold["ids"] and now["counts"] == gold["counts"] and now["perm"] == gold["perm"]
    np.testing.assert_allclose(now["w"], gold["w"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(now["y_row0_first8"], gold["y_row0_first8"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(now["y_row_l2"], gold["y_row_l2"], rtol=1e-13)

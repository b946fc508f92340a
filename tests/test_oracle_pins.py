"""Run every pin of the fp64 oracle (see tests/oracle_pins.py)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle.load())


def test_oracle_rejects_bad_arguments():
    import numpy as np
    q = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        oracle.forward("decay", q, q, q)          # decay needs a log-gate
    with pytest.raises(ValueError):
        oracle.forward("gated_delta", q, q, q)    # delta rule needs beta

"""The fp64 oracle against facts that do not come from it (CPU only).

See ``oracle_pins.py`` for what each pin checks and where it comes from.
"""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_rejects_bad_arguments(lib):
    import numpy as np
    with pytest.raises(ValueError):
        oracle.ks_matmul((0, 1, 1, 1), np.zeros(0), np.zeros((1, 0)), lib=lib)
    with pytest.raises(ValueError):   # chain widths do not match
        oracle.ks_chain_matmul([(1, 2, 2, 1), (1, 2, 3, 1)],
                               [np.zeros(4), np.zeros(6)], np.zeros((1, 2)), lib=lib)


def test_empty_batch(lib):
    import numpy as np
    Y = oracle.ks_matmul((2, 3, 4, 5), np.ones(120), np.zeros((0, 40)), lib=lib)
    assert Y.shape == (0, 30)

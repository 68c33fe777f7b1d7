"""The oracle pinned against facts outside itself (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle._lib()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_rejects_bad_arguments(lib):
    import numpy as np
    A = np.zeros(16, dtype=np.uint16)
    with pytest.raises(ValueError):
        lib.gemm(4, 4, 4, "bf16", A, 3, A, 4)          # lda < K
    with pytest.raises(ValueError):
        lib.gemm_points(4, 4, 4, "bf16", A, 4, A, 4, np.array([[0, 4, 0]]))  # i out of range

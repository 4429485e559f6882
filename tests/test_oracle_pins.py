"""The oracle against facts outside itself (CPU only)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


def test_invalid_arguments_rejected(o):
    import numpy as np
    A = np.ones((2, 3), np.float32)
    B = np.ones((3, 4), np.float32)
    with pytest.raises(ValueError):
        o.gemm_rows("f32", A, B, 1, 5)          # rows past M
    with pytest.raises(ValueError):
        o.gemm_points("f32", A, B, [0, 2], [0, 0])  # row 2 out of range
    with pytest.raises(TypeError):
        o.gemm("bf16", A, B)                    # float32 passed as 16-bit

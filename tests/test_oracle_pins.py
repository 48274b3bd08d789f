"""The CPU reference against its pins (no GPU needed)."""

import numpy as np
import pytest

from oracle import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.oracle_sgemm)


def test_thread_count_does_not_change_bits():
    from dense_fp32_matrix_row_amd import inputs
    A, B, C = inputs.make_abc(37, 45, 53, 5)
    one = oracle.oracle_sgemm(A, B, C, 0.5, 3.0, threads=1)
    many = oracle.oracle_sgemm(A, B, C, 0.5, 3.0, threads=8)
    assert one.threads == 1 and many.threads == 8
    assert np.array_equal(one.ref, many.ref)
    assert np.array_equal(one.sumabs, many.sumabs)


def test_argument_errors():
    z = np.zeros(16, np.float32)
    with pytest.raises(ValueError, match="argument 1"):
        oracle.oracle_sgemm(z, z, z, 1.0, 0.0, M=-1, N=2, K=2)
    with pytest.raises(ValueError, match="argument 6"):
        oracle.oracle_sgemm(z, z, z, 1.0, 0.0, M=2, N=2, K=3, lda=2)
    with pytest.raises(ValueError, match="argument 8"):
        oracle.oracle_sgemm(z, z, z, 1.0, 0.0, M=2, N=3, K=2, ldb=2)


@pytest.mark.parametrize("pin", oracle_pins.CHECKER_PINS, ids=lambda f: f.__name__)
def test_checker_metric(pin):
    """The normalised-error checker on hand-made cases with exact ratios."""
    pin(oracle.normalised_error)

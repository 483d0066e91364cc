"""The oracle against its pins (brute force, closed forms, invariants)."""
import numpy as np
import pytest

import oracle
from oracle import sdpa as oracle_sdpa
from tests import oracle_pins



@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle_sdpa)


def test_softmax_rows_sum_to_one():
    """Rows of the attention matrix are probability distributions; causal rows
    put zero weight above the diagonal."""
    r = np.random.default_rng(30)
    q, k = r.standard_normal((6, 4)), r.standard_normal((6, 4))
    for causal in (False, True):
        P = oracle.attention_weights(q, k, 0.9, causal)
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-15
        if causal:
            assert np.all(np.triu(P, 1) == 0)


def test_empty_rejected():
    with pytest.raises(ValueError):
        oracle.sdpa_fwd(np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 3, 4)),
                        np.zeros((1, 1, 3, 4)), 1.0)
    with pytest.raises(ValueError):
        oracle.sdpa_fwd(np.zeros((1, 1, 3, 4)), np.zeros((1, 1, 0, 4)),
                        np.zeros((1, 1, 0, 4)), 1.0)


def test_varlen_zero_length_sequence_writes_nothing():
    r = np.random.default_rng(31)
    cu = np.array([0, 2, 2, 5], dtype=np.int32)
    q, k, v = (r.standard_normal((5, 1, 3)) for _ in range(3))
    O, L = oracle.sdpa_fwd_varlen(q, k, v, cu, 0.5)
    assert O.shape == (5, 1, 3) and np.all(np.isfinite(O)) and np.all(np.isfinite(L))


def test_large_scores_no_overflow():
    """Scores far outside exp's range: the max shift keeps the result finite
    and equal to the selection limit."""
    q = np.array([[[[1000.0, 0.0]]]])
    k = np.array([[[[1.0, 0.0], [0.5, 0.0], [-1.0, 0.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]]]])
    O, L = oracle.sdpa_fwd(q, k, v, 1.0)
    assert np.allclose(O[0, 0, 0], [1.0, 2.0], atol=0, rtol=0)
    assert abs(L[0, 0, 0] - 1000.0) < 1e-9

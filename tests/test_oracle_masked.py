"""Pins of the attention-mask oracle (oracle/masked.py), independent of its
formula.

* All-true boolean masks and zero biases give the dense oracle.
* A bias constant along each row changes nothing in O and shifts lse by the
  constant (softmax is shift invariant).
* A bias of log w_ij weights key j by w_ij: O_i = sum_j w e^s v / sum_j w e^s
  (closed form, written out with the weights).
* -inf biases equal the boolean mask; a boolean mask matches the pure-Python
  brute force with its own visibility callback.
* Fully masked rows give zeros and -inf; broadcasting over batch and heads
  equals the repeated mask.
* Planted mistakes (mask transposed, bias not scaled with the scores' units,
  bias applied after the softmax) each fail a pin.
"""
import numpy as np
import pytest

from oracle import brute
from oracle import masked as M
from oracle import sdpa as dense


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_all_true_and_zero_bias_are_dense(causal):
    q, k, v = _rand((2, 3, 9, 4), 1), _rand((2, 3, 11, 4), 2), _rand((2, 3, 11, 4), 3)
    want = dense.sdpa_fwd(q, k, v, 0.6, causal)
    for mask, kind in ((np.ones((1, 1, 9, 11), np.uint8), "bool"),
                       (np.zeros((2, 3, 9, 11)), "add")):
        got = M.sdpa_fwd_masked(q, k, v, mask, kind, 0.6, causal)
        np.testing.assert_allclose(got[0], want[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(got[1], want[1], rtol=1e-13)


def test_row_constant_bias_shifts_lse_only():
    q, k, v = _rand((6, 4), 4), _rand((8, 4), 5), _rand((8, 4), 6)
    c = _rand((6, 1), 7) * 5
    o0, l0 = M.attend_biased(q, k, v, 0.5, np.zeros((6, 8)))
    o1, l1 = M.attend_biased(q, k, v, 0.5, np.broadcast_to(c, (6, 8)))
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l0 + c[:, 0], rtol=1e-12)


def test_log_weights_act_as_prior_weights():
    q, k, v = _rand((5, 3), 8), _rand((7, 3), 9), _rand((7, 3), 10)
    w = np.random.default_rng(11).uniform(0.1, 3.0, (5, 7))
    o, lse = M.attend_biased(q, k, v, 0.8, np.log(w))
    e = w * np.exp(0.8 * (q @ k.T))
    np.testing.assert_allclose(o, (e @ v) / e.sum(axis=1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(lse, np.log(e.sum(axis=1)), rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bool_mask_matches_brute_force_and_neg_inf_bias(causal):
    rng = np.random.default_rng(12)
    q, k, v = _rand((7, 3), 13), _rand((9, 3), 14), _rand((9, 3), 15)
    mask = rng.integers(0, 2, (7, 9)).astype(np.uint8)
    mask[3] = 0                                   # a row that sees nothing
    o, lse = M.attend_biased(q, k, v, 0.7, M.bias_of(mask, "bool"), causal)
    ob, lb = brute.attend(q.tolist(), k.tolist(), v.tolist(), 0.7, causal,
                          allowed=lambda i, j: mask[i, j] != 0)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12)
    assert np.all(o[3] == 0) and lse[3] == -np.inf
    bias = np.where(mask != 0, 0.0, -np.inf)
    o2, l2 = M.attend_biased(q, k, v, 0.7, bias, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


def test_broadcast_equals_repeated_mask():
    q, k, v = _rand((2, 3, 5, 4), 16), _rand((2, 3, 6, 4), 17), _rand((2, 3, 6, 4), 18)
    m = _rand((1, 3, 5, 6), 19)
    a = M.sdpa_fwd_masked(q, k, v, m, "add", 0.5)
    b = M.sdpa_fwd_masked(q, k, v, np.repeat(m, 2, axis=0), "add", 0.5)
    np.testing.assert_array_equal(a[0], b[0])


def _mutant(q, k, v, scale, bias, mistake):
    s = scale * (q @ k.T)
    if mistake == "transposed":
        s = s + bias.T[: s.shape[0], : s.shape[1]]
    elif mistake == "bias_in_score_units":
        s = scale * (q @ k.T + bias)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    if mistake == "after_softmax":
        p = p + bias
    return p @ v


@pytest.mark.parametrize("mistake", ["transposed", "bias_in_score_units", "after_softmax"])
def test_planted_mistakes_are_caught(mistake):
    q, k, v = _rand((6, 3), 20), _rand((6, 3), 21), _rand((6, 3), 22)
    w = np.random.default_rng(23).uniform(0.1, 3.0, (6, 6))
    e = w * np.exp(0.8 * (q @ k.T))
    want = (e @ v) / e.sum(axis=1, keepdims=True)
    got = _mutant(q, k, v, 0.8, np.log(w), mistake)
    assert not np.allclose(got, want, rtol=1e-6, atol=1e-8)
    ok, _ = M.attend_biased(q, k, v, 0.8, np.log(w))
    np.testing.assert_allclose(ok, want, rtol=1e-12)

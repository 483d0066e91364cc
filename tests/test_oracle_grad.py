"""Pins of the gradient oracle (oracle/grad.py), independent of its formulas.

* Finite differences of the forward oracle: the gradient of
  L = sum(dO * O(q, k, v)) by central differences in float64 must match.
* Invariants: every row of dS sums to zero, so the key gradients sum to zero
  over keys; every row of P sums to one, so the value gradients sum to the
  sum of the upstream gradient rows.
* Closed forms: identical key rows give a uniform P and dQ = 0; a single key
  gives P = 1, dQ = dK = 0 and dV = sum of dO rows.
* The identity the GPU path uses for the softmax Jacobian term:
  sum_j P_ij dP_ij = <dO_i, O_i>.
* Planted mistakes (a dropped term, a wrong operand, a missing scale, a
  wrong axis) each fail at least one pin.
"""
import numpy as np
import pytest

from oracle import grad
from oracle import sdpa as fwd


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, scale, causal):
    o, _ = fwd._attend_unit(q, k, v, scale, causal)
    return float(np.sum(do * o))


def _fd(q, k, v, do, scale, causal, h=1e-6):
    out = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


CASES = [(5, 7, 4, False), (6, 6, 3, True), (4, 9, 5, True), (8, 3, 2, False)]


@pytest.mark.parametrize("nq,nk,d,causal", CASES)
def test_grads_match_finite_differences(nq, nk, d, causal):
    q, k, v = _rand((nq, d), 1), _rand((nk, d), 2), _rand((nk, d), 3)
    do = _rand((nq, d), 4)
    scale = 0.7
    want = _fd(q, k, v, do, scale, causal)
    got = grad.attention_grads(q, k, v, do, scale, causal)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_key_grads_sum_to_zero_and_value_grads_sum_to_do(causal):
    q, k, v, do = _rand((9, 5), 5), _rand((9, 5), 6), _rand((9, 5), 7), _rand((9, 5), 8)
    dq, dk, dv = grad.attention_grads(q, k, v, do, 0.4, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_identical_keys_give_zero_query_grad():
    q, v, do = _rand((6, 4), 9), _rand((5, 4), 10), _rand((6, 4), 11)
    k = np.tile(_rand((1, 4), 12), (5, 1))
    dq, dk, dv = grad.attention_grads(q, k, v, do, 0.9, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dv, np.tile(do.sum(axis=0) / 5, (5, 1)), rtol=1e-12)


def test_single_key():
    q, k, v, do = _rand((4, 3), 13), _rand((1, 3), 14), _rand((1, 3), 15), _rand((4, 3), 16)
    dq, dk, dv = grad.attention_grads(q, k, v, do, 1.3, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, do.sum(axis=0, keepdims=True), rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_rowsum_identity(causal):
    q, k, v, do = _rand((7, 4), 17), _rand((7, 4), 18), _rand((7, 4), 19), _rand((7, 4), 20)
    p = grad._probs(q, k, 0.5, causal)
    o, _ = fwd._attend_unit(q, k, v, 0.5, causal)
    np.testing.assert_allclose(np.sum(p * (do @ v.T), axis=1), np.sum(do * o, axis=1),
                               rtol=1e-12, atol=1e-12)


def test_dense_driver_matches_units():
    q, k, v, do = (_rand((2, 3, 5, 4), s) for s in (21, 22, 23, 24))
    dq, dk, dv = grad.sdpa_bwd(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(3):
            u = grad.attention_grads(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            for a, bb in zip((dq, dk, dv), u):
                np.testing.assert_array_equal(a[b, h], bb)


# ---- planted mistakes: each must fail the finite-difference pin or an invariant

def _mutant(q, k, v, do, scale, causal, mistake):
    p = grad._probs(q, k, scale, causal)
    dp = do @ (k.T if mistake == "dp_wrong_operand" else v.T)
    d = np.sum(p * dp, axis=1, keepdims=True)
    if mistake == "jacobian_term_dropped":
        d = 0.0
    if mistake == "jacobian_wrong_axis":
        d = np.sum(p * dp, axis=0, keepdims=True)
    ds = p * (dp - d)
    sc = 1.0 if mistake == "scale_dropped" else float(scale)
    dv = ds.T @ do if mistake == "dv_uses_ds" else p.T @ do
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ (k if mistake == "dk_wrong_operand" else q))
    return dq, dk, dv


@pytest.mark.parametrize("mistake", ["jacobian_term_dropped", "jacobian_wrong_axis",
                                     "scale_dropped", "dk_wrong_operand", "dp_wrong_operand",
                                     "dv_uses_ds"])
def test_planted_mistakes_are_caught(mistake):
    nq, nk, d, causal = 6, 6, 3, True
    q, k, v, do = _rand((nq, d), 31), _rand((nk, d), 32), _rand((nk, d), 33), _rand((nq, d), 34)
    want = _fd(q.copy(), k.copy(), v.copy(), do, 0.8, causal)
    got = _mutant(q, k, v, do, 0.8, causal, mistake)
    assert not all(np.allclose(g, w, rtol=1e-5, atol=1e-6) for g, w in zip(got, want))
    # control: the unmutated formulas pass the same comparison
    ok = grad.attention_grads(q, k, v, do, 0.8, causal)
    assert all(np.allclose(g, w, rtol=1e-5, atol=1e-6) for g, w in zip(ok, want))


# ---- gradients through dropout (the mask is a constant of the seed) -----------

def _loss_dropout(q, k, v, do, scale, causal, p, seed):
    from oracle import dropout as odrop
    o, _ = odrop.attend_dropout(q, k, v, scale, causal, p, seed, 3, 0)
    return float(np.sum(do * o))


@pytest.mark.parametrize("nq,nk,d,causal", [(5, 7, 4, False), (6, 6, 3, True), (4, 20, 2, True)])
def test_dropout_grads_match_finite_differences(nq, nk, d, causal):
    q, k, v = _rand((nq, d), 41), _rand((nk, d), 42), _rand((nk, d), 43)
    do = _rand((nq, d), 44)
    p, seed, h = 0.3, 17, 1e-6
    want = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss_dropout(q, k, v, do, 0.7, causal, p, seed)
            x[idx] = old - h
            lm = _loss_dropout(q, k, v, do, 0.7, causal, p, seed)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        want.append(g)
    got = grad.attention_grads_dropout(q, k, v, do, 0.7, causal, p, seed, 3, 0)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-6, atol=1e-7)
    # the mask matters: some weight of this case is dropped
    from oracle import dropout as odrop
    assert not odrop.keep_mask(nq, nk, 0, p, seed, 3).all()


def test_dropout_grads_at_p_zero_are_the_plain_grads():
    q, k, v, do = (_rand((2, 3, 9, 4), s) for s in (51, 52, 53, 54))
    a = grad.sdpa_bwd_dropout(q, k, v, do, 0.5, True, 0.0, 5)
    b = grad.sdpa_bwd(q, k, v, do, 0.5, True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)


def test_dropout_rowsum_identity():
    """sum_j P_ij dP_ij = <dO_i, O_i> also with dropout (the GPU path's D)."""
    from oracle import dropout as odrop
    q, k, v, do = _rand((7, 4), 61), _rand((9, 4), 62), _rand((9, 4), 63), _rand((7, 4), 64)
    P = grad._probs(q, k, 0.5, False)
    kappa = np.floor((1.0 - float(np.float32(0.4))) * 65536.0 + 0.5) / 65536.0
    zr = odrop.keep_mask(7, 9, 2, 0.4, 8, 1) / kappa
    o, _ = odrop.attend_dropout(q, k, v, 0.5, False, 0.4, 8, 1, 2)
    np.testing.assert_allclose(np.sum(P * (do @ v.T) * zr, axis=1), np.sum(do * o, axis=1),
                               rtol=1e-12, atol=1e-12)

"""Pins of the masked-attention gradient oracle (oracle/grad.py:
attention_grads_biased, sdpa_bwd_masked), independent of its formulas.

* Finite differences of the masked forward oracle (oracle/masked.py): the
  gradient of L = sum(dO * O) by central differences in float64, for
  additive and boolean masks, causal on and off, Nq != Nk.
* A zero bias, or an all-true boolean mask, gives the plain gradients.
* -inf entries of an additive mask are the boolean mask's drops.
* A bias constant along each row changes nothing (softmax shift
  invariance, so O and every gradient are unchanged).
* A row with no visible key has zero gradients everywhere it reaches.
* Broadcast masks equal their repeated copies.
* Planted mistakes (bias scaled like the scores, mask transposed, dropped
  Jacobian term) each fail the finite-difference pin.
"""
import numpy as np
import pytest

from oracle import grad
from oracle import masked as M


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, scale, bias, causal):
    o, _ = M.attend_biased(q, k, v, scale, bias, causal)
    return float(np.sum(do * o))


def _fd(q, k, v, do, scale, bias, causal, h=1e-6):
    out = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, bias, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, bias, causal)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


def _bias(nq, nk, seed, kind):
    rng = np.random.default_rng(seed)
    keep = rng.random((nq, nk)) < 0.7
    keep[:, 0] = True   # every row keeps a key (empty rows are pinned apart)
    if kind == "bool":
        return np.where(keep, 0.0, -np.inf)
    return np.where(keep, rng.standard_normal((nq, nk)) * 2.0, -np.inf)


CASES = [(5, 7, 4, False, "add"), (6, 6, 3, True, "add"), (4, 9, 5, True, "bool"),
         (8, 3, 2, False, "bool")]


@pytest.mark.parametrize("nq,nk,d,causal,kind", CASES)
def test_masked_grads_match_finite_differences(nq, nk, d, causal, kind):
    q, k, v, do = _rand((nq, d), 1), _rand((nk, d), 2), _rand((nk, d), 3), _rand((nq, d), 4)
    bias = _bias(nq, nk, 5, kind)
    got = grad.attention_grads_biased(q, k, v, do, 0.7, bias, causal)
    want = _fd(q.copy(), k.copy(), v.copy(), do, 0.7, bias, causal)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_bias_and_all_true_mask_give_plain_grads(causal):
    q, k, v, do = _rand((6, 4), 6), _rand((6, 4), 7), _rand((6, 4), 8), _rand((6, 4), 9)
    plain = grad.attention_grads(q, k, v, do, 0.5, causal)
    for got in (grad.attention_grads_biased(q, k, v, do, 0.5, np.zeros((6, 6)), causal),
                grad.sdpa_bwd_masked(q[None, None], k[None, None], v[None, None],
                                     do[None, None], np.ones((1, 1, 6, 6), np.uint8), "bool",
                                     0.5, causal)):
        got = [g.reshape(p.shape) for g, p in zip(got, plain)]
        for g, p in zip(got, plain):
            np.testing.assert_allclose(g, p, rtol=1e-12, atol=1e-14)


def test_neg_inf_bias_equals_bool_mask():
    q, k, v, do = _rand((5, 3), 10), _rand((8, 3), 11), _rand((8, 3), 12), _rand((5, 3), 13)
    keep = np.random.default_rng(14).random((5, 8)) < 0.6
    keep[:, 2] = True
    a = grad.sdpa_bwd_masked(q[None, None], k[None, None], v[None, None], do[None, None],
                             keep[None, None].astype(np.uint8), "bool", 0.9)
    b = grad.sdpa_bwd_masked(q[None, None], k[None, None], v[None, None], do[None, None],
                             np.where(keep, 0.0, -np.inf)[None, None], "add", 0.9)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_row_constant_bias_changes_nothing():
    q, k, v, do = _rand((6, 4), 15), _rand((7, 4), 16), _rand((7, 4), 17), _rand((6, 4), 18)
    bias = _bias(6, 7, 19, "add")
    shift = _rand((6, 1), 20) * 30.0
    a = grad.attention_grads_biased(q, k, v, do, 0.6, bias, False)
    b = grad.attention_grads_biased(q, k, v, do, 0.6, bias + shift, False)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-12)


def test_empty_row_has_no_gradient():
    q, k, v, do = _rand((4, 3), 21), _rand((5, 3), 22), _rand((5, 3), 23), _rand((4, 3), 24)
    bias = np.zeros((4, 5))
    bias[2] = -np.inf
    dq, dk, dv = grad.attention_grads_biased(q, k, v, do, 0.8, bias, False)
    assert np.all(dq[2] == 0.0)
    # the same gradients as dropping row 2 from the problem (its O is the
    # constant 0, so it reaches neither K nor V)
    keep = [0, 1, 3]
    dq2, dk2, dv2 = grad.attention_grads_biased(q[keep], k, v, do[keep], 0.8, bias[keep], False)
    np.testing.assert_allclose(dq[keep], dq2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk, dk2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv, dv2, rtol=1e-12, atol=1e-14)


def test_broadcast_mask_equals_repeated():
    B, H, N, d = 2, 3, 5, 4
    q, k, v, do = (_rand((B, H, N, d), s) for s in (25, 26, 27, 28))
    m = (np.random.default_rng(29).random((1, H, N, N)) < 0.7).astype(np.uint8)
    m[..., 0] = 1
    a = grad.sdpa_bwd_masked(q, k, v, do, m, "bool", 0.5)
    b = grad.sdpa_bwd_masked(q, k, v, do, np.repeat(m, B, axis=0), "bool", 0.5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def _mutant(q, k, v, do, scale, bias, causal, mistake):
    if mistake == "bias_scaled":
        bias = scale * bias
    elif mistake == "transposed":
        bias = bias.T
    s = scale * (q @ k.T) + bias
    if causal:
        s = np.where(np.arange(s.shape[1])[None, :] <= np.arange(s.shape[0])[:, None], s, -np.inf)
    e = np.exp(s - np.max(s, axis=1, keepdims=True))
    P = e / np.sum(e, axis=1, keepdims=True)
    dp = do @ v.T
    ds = P * dp if mistake == "no_jacobian" else P * (dp - np.sum(P * dp, axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), P.T @ do


@pytest.mark.parametrize("mistake", ["bias_scaled", "transposed", "no_jacobian"])
def test_planted_mistakes_are_caught(mistake):
    n, d = 6, 3
    q, k, v, do = _rand((n, d), 30), _rand((n, d), 31), _rand((n, d), 32), _rand((n, d), 33)
    bias = _rand((n, n), 34) * 2.0   # finite, asymmetric
    want = _fd(q.copy(), k.copy(), v.copy(), do, 0.7, bias, False)
    got = _mutant(q, k, v, do, 0.7, bias, False, mistake)
    assert not all(np.allclose(g, w, rtol=1e-5, atol=1e-6) for g, w in zip(got, want))
    ok = grad.attention_grads_biased(q, k, v, do, 0.7, bias, False)
    for g, w in zip(ok, want):
        np.testing.assert_allclose(g, w, rtol=1e-6, atol=1e-7)

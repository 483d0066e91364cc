"""Pins of the oracle for an elementwise mask together with dropout
(oracle/dropout.py: attend_masked_dropout, sdpa_fwd_masked_dropout;
oracle/grad.py: attention_grads_masked_dropout, sdpa_bwd_masked_dropout),
independent of their formulas.

* p = 0 keeps every weight (T = 65536, kappa = 1): the masked oracle.
* An all-true boolean mask, or a zero additive one: the dropout oracle.
* A boolean mask that keeps one key per row: O_i = z_ij v_j / kappa and
  lse_i = s_ij (closed form), so the mask and the keep decisions of the
  right pairs meet.
* A pure-Python triple loop (math.exp, math.fsum, no max shift) on tiny
  shapes, with the keep decisions read from the pinned Philox layout.
* A row whose every pair is masked: O = 0, lse = -inf, whatever the draws.
* Gradients: central finite differences of the forward oracle's
  L = sum(dO * O) (the keep mask is a constant); p = 0 gives the masked
  gradients and an all-true mask the dropout gradients.
* Planted mistakes (normalising over the kept weights, dropping before the
  mask so that dropped pairs leave the softmax, scaling by 1 - p instead of
  kappa, the mask transposed) each fail a pin.
"""
import math

import numpy as np
import pytest

from oracle import dropout as D
from oracle import grad
from oracle import masked as M

SEED, OFF = 0x5EED1234ABCD, 3


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _mask(shape, seed, kind, keep=0.7):
    rng = np.random.default_rng(seed)
    k = rng.random(shape) < keep
    k[..., 0] = True
    if kind == "bool":
        return k.astype(np.uint8)
    return np.where(k, rng.standard_normal(shape) * 2.0, -np.inf)


@pytest.mark.parametrize("kind", ["bool", "add"])
@pytest.mark.parametrize("causal", [False, True])
def test_no_dropout_is_the_masked_oracle(kind, causal):
    q, k, v = _rand((2, 3, 9, 8), 1), _rand((2, 3, 11, 8), 2), _rand((2, 3, 11, 8), 3)
    m = _mask((2, 3, 9, 11), 4, kind)
    o, l = D.sdpa_fwd_masked_dropout(q, k, v, m, kind, 0.4, causal, 0.0, SEED, OFF)
    ro, rl = M.sdpa_fwd_masked(q, k, v, m, kind, 0.4, causal)
    assert np.allclose(o, ro, rtol=0, atol=1e-13) and np.array_equal(np.isneginf(l), np.isneginf(rl))
    assert np.allclose(l[np.isfinite(rl)], rl[np.isfinite(rl)], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_all_true_mask_is_the_dropout_oracle(causal):
    q, k, v = _rand((2, 2, 10, 8), 5), _rand((2, 2, 13, 8), 6), _rand((2, 2, 13, 8), 7)
    for kind, m in (("bool", np.ones((1, 1, 10, 13), np.uint8)), ("add", np.zeros((1, 2, 10, 13)))):
        o, l = D.sdpa_fwd_masked_dropout(q, k, v, m, kind, 0.3, causal, 0.25, SEED, OFF)
        ro, rl = D.sdpa_fwd_dropout(q, k, v, 0.3, causal, 0.25, SEED, OFF)
        assert np.allclose(o, ro, rtol=0, atol=1e-13) and np.allclose(l, rl, rtol=0, atol=1e-13)


def test_one_key_per_row_closed_form():
    nq, nk, d, scale, p = 7, 12, 4, 0.5, 0.4
    q, k, v = _rand((1, 1, nq, d), 8), _rand((1, 1, nk, d), 9), _rand((1, 1, nk, d), 10)
    pick = np.random.default_rng(11).integers(0, nk, nq)
    m = np.zeros((1, 1, nq, nk), np.uint8)
    m[0, 0, np.arange(nq), pick] = 1
    o, l = D.sdpa_fwd_masked_dropout(q, k, v, m, "bool", scale, False, p, SEED, OFF)
    z = D.keep_mask(nq, nk, 0, p, SEED, OFF)
    kappa = D.keep_probability(p)
    for i in range(nq):
        j = pick[i]
        assert np.allclose(o[0, 0, i], z[i, j] * v[0, 0, j] / kappa, rtol=0, atol=1e-13)
        assert abs(l[0, 0, i] - scale * float(q[0, 0, i] @ k[0, 0, j])) < 1e-13
    assert 0 < int(z[np.arange(nq), pick].sum()) < nq   # both outcomes occur here


def _brute(q, k, v, bias, scale, causal, z, kappa):
    nq, nk, dv = len(q), len(k), len(v[0])
    out, lse = [], []
    for i in range(nq):
        w = []
        for j in range(nk):
            s = scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i]))) + bias[i][j]
            w.append(0.0 if (causal and j > i) or s == -math.inf else math.exp(s))
        tot = math.fsum(w)
        if tot == 0.0:
            out.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        out.append([math.fsum(w[j] / tot * (z[i][j] / kappa) * v[j][c] for j in range(nk))
                    for c in range(dv)])
        lse.append(math.log(tot))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("kind", ["bool", "add"])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(kind, causal):
    nq, nk, d, p = 5, 6, 3, 0.35
    q, k, v = _rand((1, 1, nq, d), 12), _rand((1, 1, nk, d), 13), _rand((1, 1, nk, 2), 14)
    m = _mask((1, 1, nq, nk), 15, kind, keep=0.6)
    bias = M.bias_of(m[0, 0], kind)
    o, l = D.sdpa_fwd_masked_dropout(q, k, v, m, kind, 0.7, causal, p, SEED, OFF)
    z = D.keep_mask(nq, nk, 0, p, SEED, OFF)
    bo, bl = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), bias.tolist(), 0.7,
                    causal, z.tolist(), D.keep_probability(p))
    assert np.allclose(o[0, 0], bo, rtol=0, atol=1e-12)
    assert np.allclose(l[0, 0], bl, rtol=0, atol=1e-12)


def test_fully_masked_row():
    q, k, v = _rand((1, 2, 4, 8), 16), _rand((1, 2, 5, 8), 17), _rand((1, 2, 5, 8), 18)
    m = np.ones((1, 1, 4, 5), np.uint8)
    m[0, 0, 2] = 0
    o, l = D.sdpa_fwd_masked_dropout(q, k, v, m, "bool", 0.3, False, 0.5, SEED, OFF)
    assert np.all(o[:, :, 2] == 0.0) and np.all(np.isneginf(l[:, :, 2]))
    assert np.all(np.isfinite(l[:, :, [0, 1, 3]]))


def _loss(q, k, v, do, scale, bias, causal, p):
    o, _ = D.attend_masked_dropout(q, k, v, scale, bias, causal, p, SEED, OFF, 0)
    return float(np.sum(do * o))


def _fd(q, k, v, do, scale, bias, causal, p, h=1e-6):
    out = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, bias, causal, p)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, bias, causal, p)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


@pytest.mark.parametrize("nq,nk,d,causal,kind", [(5, 7, 4, False, "add"), (6, 6, 3, True, "bool"),
                                                 (4, 9, 5, True, "add")])
def test_gradients_by_finite_differences(nq, nk, d, causal, kind):
    q, k, v, do = (_rand(s, 20 + i) for i, s in enumerate([(nq, d), (nk, d), (nk, d), (nq, d)]))
    bias = M.bias_of(_mask((nq, nk), 24, kind), kind)
    got = grad.attention_grads_masked_dropout(q, k, v, do, 0.6, bias, causal, 0.3, SEED, OFF, 0)
    fd = _fd(q.copy(), k.copy(), v.copy(), do, 0.6, bias, causal, 0.3)
    for g, f in zip(got, fd):
        assert np.allclose(g, f, rtol=1e-6, atol=1e-7)


def test_gradients_reduce_to_masked_and_dropout():
    q, k, v, do = _rand((1, 2, 6, 4), 30), _rand((1, 2, 8, 4), 31), _rand((1, 2, 8, 4), 32), \
        _rand((1, 2, 6, 4), 33)
    m = _mask((1, 2, 6, 8), 34, "add")
    a = grad.sdpa_bwd_masked_dropout(q, k, v, do, m, "add", 0.5, True, 0.0, SEED, OFF)
    b = grad.sdpa_bwd_masked(q, k, v, do, m, "add", 0.5, True)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-13)
    ones = np.ones((1, 1, 6, 8), np.uint8)
    a = grad.sdpa_bwd_masked_dropout(q, k, v, do, ones, "bool", 0.5, False, 0.2, SEED, OFF)
    b = grad.sdpa_bwd_dropout(q, k, v, do, 0.5, False, 0.2, SEED, OFF)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-13)


# ---- planted mistakes, each of which a pin above must catch

def _mutant_normalise_kept(q, k, v, scale, bias, causal, p, seed, off, unit):
    o, l = D.attend_masked_dropout(q, k, v, scale, bias, causal, p, seed, off, unit)
    s = scale * (q @ k.T) + bias
    z = D.keep_mask(len(q), len(k), unit, p, seed, off)
    e = np.where(z, np.exp(s - np.max(s, axis=1, keepdims=True)), 0.0)
    return (e / np.maximum(e.sum(1, keepdims=True), 1e-300)) @ v, l


def _mutant_drop_before_mask(q, k, v, scale, bias, causal, p, seed, off, unit):
    z = D.keep_mask(len(q), len(k), unit, p, seed, off)
    return M.attend_biased(q, k, v, scale, np.where(z, bias, -np.inf), causal)


def _mutant_one_minus_p(q, k, v, scale, bias, causal, p, seed, off, unit):
    o, l = D.attend_masked_dropout(q, k, v, scale, bias, causal, p, seed, off, unit)
    return o * D.keep_probability(p) / (1.0 - p), l


@pytest.mark.parametrize("mutant", [_mutant_normalise_kept, _mutant_drop_before_mask,
                                    _mutant_one_minus_p])
def test_planted_mistakes_fail_the_brute_force(mutant):
    nq, nk, d, p = 5, 6, 3, 0.3
    q, k, v = _rand((nq, d), 40), _rand((nk, d), 41), _rand((nk, 2), 42)
    bias = M.bias_of(_mask((nq, nk), 43, "add", keep=0.7), "add")
    o, l = mutant(q, k, v, 0.7, bias, False, p, SEED, OFF, 0)
    z = D.keep_mask(nq, nk, 0, p, SEED, OFF)
    bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), bias.tolist(), 0.7, False, z.tolist(),
                    D.keep_probability(p))
    assert not (np.allclose(o, bo, rtol=0, atol=1e-9) and np.allclose(l, bl, rtol=0, atol=1e-9))


def test_planted_transposed_mask_fails_the_closed_form():
    nq = nk = 6
    q, k, v = _rand((1, 1, nq, 4), 50), _rand((1, 1, nk, 4), 51), _rand((1, 1, nk, 4), 52)
    pick = np.random.default_rng(53).integers(0, nk, nq)
    m = np.zeros((1, 1, nq, nk), np.uint8)
    m[0, 0, np.arange(nq), pick] = 1
    o, _ = D.sdpa_fwd_masked_dropout(q, k, v, m.transpose(0, 1, 3, 2), "bool", 0.5, False, 0.4,
                                     SEED, OFF)
    z = D.keep_mask(nq, nk, 0, 0.4, SEED, OFF)
    want = np.stack([z[i, pick[i]] * v[0, 0, pick[i]] / D.keep_probability(0.4) for i in range(nq)])
    assert not np.allclose(o[0, 0], want, rtol=0, atol=1e-9)

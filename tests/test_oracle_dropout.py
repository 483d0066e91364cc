"""Pins of the Philox generator (oracle/philox.py) and the dropout oracle
(oracle/dropout.py), independent of their own formulas.

Generator:
* the same round code at W = 64 reproduces numpy's Philox4x64-10 bit
  generator (round structure, key schedule, round count);
* the Weyl key increments equal the W-bit fractional parts of the golden
  ratio and of sqrt(3), computed here with exact integer square roots;
* Philox4x32-10 reproduces the known-answer values published with the
  Random123 library (the reference implementation of the SC 2011 paper);
* the vectorised (numpy) and scalar (Python int) paths agree.

Dropout:
* a hand-worked element of the counter layout;
* the layout visits every (call, half) once per 16 keys;
* the keep rate and the 16-bit numbers' distribution match the contract
  within binomial / chi-square bounds;
* p = 0 is the dense oracle exactly; lse never depends on the mask;
* a single key gives O = z v / kappa, kappa = floor((1 - p) 65536 + 1/2) / 65536
  (the keep probability actually drawn), which differs from 1 - p at p = 0.3;
* averaged over many seeds, O is unbiased (mean = dense O within 5
  standard errors);
* packed sequences are per-sequence dense units with u = s*H + h;
* planted mistakes (inverted keep test, 1/p scaling, normalising by the
  kept weights, a row-independent mask) each fail a pin.
"""
import math

import numpy as np
import pytest

from oracle import dropout as D
from oracle import philox as PH
from oracle import sdpa as dense


# ---- generator ---------------------------------------------------------------

@pytest.mark.parametrize("ctr,key", [((0, 0, 0, 0), (0, 0)), ((5, 7, 11, 13), (17, 19)),
                                     ((2 ** 64 - 2, 2 ** 63, 1, 2 ** 40), (2 ** 64 - 1, 12345))])
def test_round_code_matches_numpy_philox4x64(ctr, key):
    # numpy advances the counter before producing a block
    bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    want = [int(x) for x in bg.random_raw(4)]
    c0 = (ctr[0] + 1) % 2 ** 64
    c1 = (ctr[1] + (1 if c0 == 0 else 0)) % 2 ** 64
    got = PH.philox4((c0, c1, ctr[2], ctr[3]), key, width=64, rounds=10)
    assert [int(x) for x in got] == want


@pytest.mark.parametrize("width", [32, 64])
def test_weyl_constants_are_golden_ratio_and_sqrt3_fractions(width):
    one = 1 << width
    # floor(frac(phi) * 2^W) = floor((sqrt(5) - 1) / 2 * 2^W)
    s5 = math.isqrt(5 * one * one)            # floor(sqrt(5) * 2^W)
    phi = (s5 - one) // 2
    s3 = math.isqrt(3 * one * one) - one      # floor((sqrt(3) - 1) * 2^W)
    assert PH.PARAMS[width][2] == phi
    assert PH.PARAMS[width][3] == s3


# Philox4x32-10 known-answer values distributed with Random123 (counter,
# key -> output), all words hexadecimal
KAT_4X32_10 = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT_4X32_10)
def test_philox4x32_10_known_answers(ctr, key, want):
    assert tuple(int(x) for x in PH.philox4(ctr, key, 32, 10)) == want


def test_vector_and_scalar_paths_agree():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2 ** 32, (4, 50), dtype=np.uint64)
    k = (0x12345678, 0x9ABCDEF0)
    vec = PH.philox4(tuple(c), k, 32, 10)
    for t in range(50):
        sc = PH.philox4(tuple(int(c[w, t]) for w in range(4)), k, 32, 10)
        assert tuple(int(vec[w][t]) for w in range(4)) == tuple(int(x) for x in sc)


# ---- counter layout ----------------------------------------------------------

def test_hand_worked_element():
    # row 5, key 37 of unit 3, seed 0x0000000100000002, offset 9:
    # call n = 2*(37 >> 4) + ((37 >> 2) & 1) = 2*2 + 1 = 5;
    # half e = 4*((37 >> 3) & 1) + (37 & 3) = 0 + 1 = 1 -> word 0, bits 16..31
    w = PH.philox4((5, 5, 3, 9), (2, 1), 32, 10)
    r = D.draw16(6, 40, 3, 0x0000000100000002, 9)
    assert int(r[5, 37]) == (int(w[0]) >> 16) & 0xFFFF
    # key 10 of row 0: n = 0 + ((10 >> 2) & 1) = 0; e = 4*1 + 2 = 6 -> word 3, bits 0..15
    w = PH.philox4((0, 0, 3, 9), (2, 1), 32, 10)
    assert int(r[0, 10]) == int(w[3]) & 0xFFFF


def test_layout_uses_each_half_once():
    j = np.arange(64)
    n = 2 * (j >> 4) + ((j >> 2) & 1)
    e = 4 * ((j >> 3) & 1) + (j & 3)
    pairs = set(zip(n.tolist(), e.tolist()))
    assert len(pairs) == 64 and {p[0] for p in pairs} == set(range(8))
    assert {p[1] for p in pairs} == set(range(8))


def test_keep_rate_and_uniformity():
    r = D.draw16(512, 1024, 7, 2024, 0)
    # top byte of the 16-bit numbers: chi-square over 256 bins, 255 dof
    hist = np.bincount((r >> 8).ravel(), minlength=256)
    exp = r.size / 256
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    assert 160 < chi2 < 370
    for p in (0.1, 0.5, 0.9):
        t = D.keep_threshold(p)
        z = r < t
        q = t / 65536
        sd = math.sqrt(q * (1 - q) / r.size)
        assert abs(z.mean() - q) < 5 * sd
        assert abs(q - (1 - np.float32(p))) <= 2 ** -17
    # neighbouring keys of a row are uncorrelated
    x = r.astype(np.float64)
    c = np.corrcoef(x[:, :-1].ravel(), x[:, 1:].ravel())[0, 1]
    assert abs(c) < 5 / math.sqrt(x[:, 1:].size)


def test_units_rows_seeds_offsets_give_different_masks():
    base = D.draw16(64, 64, 0, 1, 0)
    for other in (D.draw16(64, 64, 1, 1, 0), D.draw16(64, 64, 0, 2, 0),
                  D.draw16(64, 64, 0, 1, 1), D.draw16(64, 64, 0, 1 << 32, 0)):
        assert np.mean(base == other) < 0.01
    assert np.mean(base[1:] == base[:-1]) < 0.01


# ---- attention with dropout ---------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_dense(causal):
    q, k, v = _rand((2, 3, 40, 8), 1), _rand((2, 3, 40, 8), 2), _rand((2, 3, 40, 8), 3)
    o, l = D.sdpa_fwd_dropout(q, k, v, 0.35, causal, 0.0, 99)
    od, ld = dense.sdpa_fwd(q, k, v, 0.35, causal)
    np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l, ld, rtol=1e-13, atol=1e-14)


def test_lse_ignores_the_mask():
    q, k, v = _rand((1, 2, 33, 8), 4), _rand((1, 2, 50, 8), 5), _rand((1, 2, 50, 8), 6)
    _, l1 = D.sdpa_fwd_dropout(q, k, v, 0.3, False, 0.5, 1)
    _, l2 = D.sdpa_fwd_dropout(q, k, v, 0.3, False, 0.2, 2)
    _, ld = dense.sdpa_fwd(q, k, v, 0.3, False)
    np.testing.assert_allclose(l1, ld, rtol=1e-13)
    np.testing.assert_array_equal(l1, l2)


def test_single_key():
    q, k, v = _rand((1, 1, 20, 4), 7), _rand((1, 1, 1, 4), 8), _rand((1, 1, 1, 4), 9)
    p = 0.3
    o, l = D.sdpa_fwd_dropout(q, k, v, 0.5, False, p, 11)
    z = D.keep_mask(20, 1, 0, p, 11, 0)
    kappa = math.floor((1.0 - float(np.float32(p))) * 65536.0 + 0.5) / 65536.0
    assert abs(kappa - 0.7) > 1e-6       # the pin tells kappa from 1 - p
    want = z * v[0, 0, 0][None, :] / kappa
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-13)
    np.testing.assert_allclose(l[0, 0], 0.5 * (q[0, 0] @ k[0, 0, 0]), rtol=1e-12)
    assert 0 < z.sum() < 20


def _mean_over_seeds(fn, n=3000):
    outs = np.stack([fn(s) for s in range(n)])
    return outs.mean(axis=0), outs.std(axis=0) / math.sqrt(n)


def _unbiased_ok(fn, ref):
    mean, se = _mean_over_seeds(fn)
    return bool(np.all(np.abs(mean - ref) <= 5 * se + 1e-12))


def test_unbiased_over_seeds():
    q, k, v = _rand((3, 4), 10), _rand((20, 4), 11), _rand((20, 4), 12)
    ref, _ = dense._attend_unit(q, k, v, 0.6, True)
    fn = lambda s: D.attend_dropout(q, k, v, 0.6, True, 0.4, s, 0, 0)[0]
    assert _unbiased_ok(fn, ref)


def test_packed_is_per_sequence_dense_units():
    lens = [5, 0, 17, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H = int(cu[-1]), 2
    q, k, v = _rand((T, H, 8), 13), _rand((T, H, 8), 14), _rand((T, H, 8), 15)
    o, l = D.sdpa_fwd_dropout_varlen(q, k, v, cu, 0.4, True, 0.25, 77, 3)
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            if b > a:
                ou, lu = D.attend_dropout(q[a:b, h], k[a:b, h], v[a:b, h], 0.4, True, 0.25, 77,
                                          3, s * H + h)
                np.testing.assert_array_equal(o[a:b, h], ou)
                np.testing.assert_array_equal(l[a:b, h], lu)


# ---- planted mistakes -----------------------------------------------------------

def _mutant(q, k, v, scale, causal, p, seed, mistake):
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    r = D.draw16(nq, nk, 0, seed, 0)
    if mistake == "row_independent_mask":
        r = np.broadcast_to(r[:1], r.shape)
    t = D.keep_threshold(p)
    z = (r >= t) if mistake == "inverted_keep" else (r < t)
    if mistake == "normalised_by_kept":
        P = e * z / np.maximum((e * z).sum(axis=1, keepdims=True), 1e-300)
        return P @ v
    P = e / e.sum(axis=1, keepdims=True)
    keep = float(np.float32(p)) if mistake == "scaled_by_p" else t / 65536.0
    return (P * z / keep) @ v


@pytest.mark.parametrize("mistake", ["inverted_keep", "scaled_by_p", "normalised_by_kept",
                                     "row_independent_mask"])
def test_planted_mistakes_are_caught(mistake):
    q, k, v = _rand((3, 4), 10), _rand((20, 4), 11), _rand((20, 4), 12)
    ref, _ = dense._attend_unit(q, k, v, 0.6, True)
    fn = lambda s: _mutant(q, k, v, 0.6, True, 0.4, s, mistake)
    caught = not _unbiased_ok(fn, ref)
    if mistake == "row_independent_mask":
        # unbiased, but rows no longer draw independently: every row keeps
        # the same keys, which the correlation of row masks shows
        r = D.draw16(64, 64, 0, 5, 0)
        z_ok = (r < D.keep_threshold(0.4)).astype(float)
        z_bad = np.broadcast_to(z_ok[:1], z_ok.shape)
        caught = np.mean(z_bad[1:] == z_bad[:-1]) == 1.0 and np.mean(z_ok[1:] == z_ok[:-1]) < 0.7
    assert caught
    # control: the oracle itself passes the unbiasedness pin
    assert _unbiased_ok(lambda s: D.attend_dropout(q, k, v, 0.6, True, 0.4, s, 0, 0)[0], ref)

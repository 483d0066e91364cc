"""Pins for the CPU oracle: checks against facts fixed by the pages and by
mathematics, not by the oracle itself.

Each ``pin_*`` takes an implementation namespace ``impl`` exposing
``sdpa_fwd(q,k,v,scale,is_causal)``, ``sdpa_fwd_rows(q,k,v,scale,is_causal,
rows)`` and ``sdpa_fwd_varlen(q,k,v,cu,scale,is_causal)`` and raises
AssertionError on a mismatch.  ``tests/test_oracle_pins.py`` runs them on the
oracle; ``tests/test_oracle_mutants.py`` runs them on deliberately broken
copies of it to show that each plausible mistake is caught by some pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy import special

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --- brute force on tiny inputs ---------------------------------------------

def pin_brute_force(impl):
    """Agreement with the pure-Python loop implementation (oracle/brute.py)
    on the tutorial's 2x3x8 example shape and on random tiny shapes, with
    and without the causal mask, and with Nq != Nk."""
    shapes = [(2, 1, 3, 3, 8, False), (2, 1, 3, 3, 8, True), (1, 2, 5, 7, 4, False),
              (2, 2, 6, 6, 3, True), (1, 1, 9, 4, 16, False), (1, 1, 4, 9, 5, True),
              (1, 1, 1, 1, 2, True)]
    for n, (B, H, Nq, Nk, d, causal) in enumerate(shapes):
        r = _rng(100 + n)
        q = r.standard_normal((B, H, Nq, d))
        k = r.standard_normal((B, H, Nk, d))
        v = r.standard_normal((B, H, Nk, d))
        scale = 1.0 / math.sqrt(d)
        O, L = impl.sdpa_fwd(q, k, v, scale, causal)
        for b in range(B):
            for h in range(H):
                ob, lb = brute.attend(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(),
                                      scale, causal)
                _close(O[b, h], ob, 1e-12, f"brute O {B,H,Nq,Nk,d,causal}")
                _close(L[b, h], lb, 1e-12, f"brute lse {B,H,Nq,Nk,d,causal}")


def pin_library_softmax(impl):
    """Special case reducing to library routines: with the scores formed
    explicitly, O = scipy.special.softmax(s) @ v and lse = logsumexp(s)."""
    r = _rng(7)
    q, k, v = (r.standard_normal((1, 1, 6, 5)), r.standard_normal((1, 1, 8, 5)),
               r.standard_normal((1, 1, 8, 5)))
    s = 0.7 * np.einsum("id,jd->ij", q[0, 0], k[0, 0])
    O, L = impl.sdpa_fwd(q, k, v, 0.7, False)
    _close(O[0, 0], special.softmax(s, axis=1) @ v[0, 0], 1e-12, "softmax O")
    _close(L[0, 0], special.logsumexp(s, axis=1), 1e-12, "logsumexp")


# --- closed forms ------------------------------------------------------------

def pin_scale_zero(impl):
    """scale = 0 makes every allowed key equally likely: O_i is the mean of
    the allowed value rows and lse_i = ln |A_i|."""
    r = _rng(8)
    n, d = 7, 4
    q, k, v = (r.standard_normal((1, 1, n, d)) for _ in range(3))
    for causal in (False, True):
        O, L = impl.sdpa_fwd(q, k, v, 0.0, causal)
        for i in range(n):
            cnt = i + 1 if causal else n
            _close(O[0, 0, i], v[0, 0, :cnt].mean(axis=0), 1e-12, "scale0 O")
            _close(L[0, 0, i], math.log(cnt), 1e-12, "scale0 lse")


def pin_identical_keys(impl):
    """All keys equal to one vector kappa: every score in a row is the same,
    so O_i = mean of the allowed values and lse_i = scale<q_i,kappa> + ln|A_i|."""
    r = _rng(9)
    n, d, scale = 6, 5, 0.37
    q = r.standard_normal((1, 1, n, d))
    kappa = r.standard_normal(d)
    k = np.broadcast_to(kappa, (1, 1, n, d)).copy()
    v = r.standard_normal((1, 1, n, d))
    for causal in (False, True):
        O, L = impl.sdpa_fwd(q, k, v, scale, causal)
        for i in range(n):
            cnt = i + 1 if causal else n
            _close(O[0, 0, i], v[0, 0, :cnt].mean(axis=0), 1e-12, "identical-keys O")
            _close(L[0, 0, i], scale * float(q[0, 0, i] @ kappa) + math.log(cnt), 1e-12,
                   "identical-keys lse")


def pin_causal_row0(impl):
    """Under the causal mask the first query sees only the first key:
    O_0 = V_0 exactly and lse_0 = scale<q_0,k_0>."""
    r = _rng(10)
    q, k, v = (r.standard_normal((2, 3, 5, 8)) for _ in range(3))
    O, L = impl.sdpa_fwd(q, k, v, 0.35, True)
    _close(O[:, :, 0], v[:, :, 0], 0.0, "causal row 0 O")
    _close(L[:, :, 0], 0.35 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-13,
           "causal row 0 lse")


def pin_two_keys_logistic(impl):
    """With two keys the weight on key 1 is the logistic function of the score
    gap: O = sigma(D) v_1 + (1 - sigma(D)) v_0, lse = s_0 + softplus(D)."""
    r = _rng(11)
    d, scale = 3, 0.9
    q = r.standard_normal((1, 1, 4, d))
    k = r.standard_normal((1, 1, 2, d))
    v = r.standard_normal((1, 1, 2, d))
    O, L = impl.sdpa_fwd(q, k, v, scale, False)
    for i in range(4):
        s0 = scale * float(q[0, 0, i] @ k[0, 0, 0])
        s1 = scale * float(q[0, 0, i] @ k[0, 0, 1])
        sig = special.expit(s1 - s0)
        _close(O[0, 0, i], sig * v[0, 0, 1] + (1 - sig) * v[0, 0, 0], 1e-14, "logistic O")
        _close(L[0, 0, i], s0 + np.logaddexp(0.0, s1 - s0), 1e-13, "softplus lse")


def pin_one_hot_selection(impl):
    """A key whose score beats every other by a wide margin (here >= 60)
    selects its value row: O_i = v_{j*} up to N * exp(-60) * max|v|."""
    r = _rng(12)
    n = d = 16
    q = 3.0 * np.eye(n)[None, None]                  # q_i = 3 e_i
    jstar = r.permutation(n)                          # query i picks key jstar[i]
    k = 0.05 * r.standard_normal((1, 1, n, d))
    for i in range(n):
        k[0, 0, jstar[i], i] += 30.0                  # score 90 vs |noise| < 1
    v = r.standard_normal((1, 1, n, d))
    O, _ = impl.sdpa_fwd(q, k, v, 1.0, False)
    for i in range(n):
        s = np.sort(k[0, 0] @ q[0, 0, i])
        assert s[-1] - s[-2] >= 60.0
        _close(O[0, 0, i], v[0, 0, jstar[i]], n * math.exp(-60) * np.abs(v).max(),
               "one-hot O")


def pin_values_constant(impl):
    """V equal to a constant vector c in every row gives O_i = c."""
    r = _rng(13)
    q, k = r.standard_normal((2, 2, 5, 4)), r.standard_normal((2, 2, 7, 4))
    c = np.array([1.0, -2.0, 0.5, 3.0])
    v = np.broadcast_to(c, (2, 2, 7, 4)).copy()
    for causal in (False, True):
        O, _ = impl.sdpa_fwd(q, k, v, 0.5, causal)
        _close(O, np.broadcast_to(c, O.shape), 1e-14, "constant V")


def pin_hand_example(impl):
    """A worked example derived by hand (tests/golden/hand_example.json)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    O, L = impl.sdpa_fwd(q, k, v, g["scale"], g["is_causal"])
    _close(O[0, 0], np.array(g["out"]), 1e-13, "hand example O")
    _close(L[0, 0], np.array([math.log(x) for x in g["lse_exp"]]), 1e-13, "hand example lse")


# --- invariants --------------------------------------------------------------

def pin_permutations(impl):
    """Non-causal: permuting (key, value) pairs together changes nothing;
    permuting the queries permutes the output rows."""
    r = _rng(14)
    q, k, v = (r.standard_normal((1, 2, 9, 6)) for _ in range(3))
    O, L = impl.sdpa_fwd(q, k, v, 0.4, False)
    pk = r.permutation(9)
    O2, L2 = impl.sdpa_fwd(q, k[:, :, pk], v[:, :, pk], 0.4, False)
    _close(O2, O, 1e-13, "kv permutation O")
    _close(L2, L, 1e-13, "kv permutation lse")
    pq = r.permutation(9)
    O3, L3 = impl.sdpa_fwd(q[:, :, pq], k, v, 0.4, False)
    _close(O3, O[:, :, pq], 1e-13, "q permutation O")
    _close(L3, L[:, :, pq], 1e-13, "q permutation lse")


def pin_key_shift(impl):
    """Adding one vector u to every key adds scale<q_i,u> to each score of
    row i: O is unchanged and lse_i grows by scale<q_i,u>."""
    r = _rng(15)
    q, k, v = (r.standard_normal((1, 1, 8, 5)) for _ in range(3))
    u = r.standard_normal(5)
    for causal in (False, True):
        O, L = impl.sdpa_fwd(q, k, v, 0.6, causal)
        O2, L2 = impl.sdpa_fwd(q, k + u, v, 0.6, causal)
        _close(O2, O, 1e-12, "key shift O")
        _close(L2, L + 0.6 * (q[0, 0] @ u)[None, None], 1e-12, "key shift lse")


def pin_convexity(impl):
    """Each output entry lies between the smallest and largest value entry
    of its column over the allowed keys."""
    r = _rng(16)
    q, k, v = (r.standard_normal((1, 1, 10, 4)) for _ in range(3))
    for causal in (False, True):
        O, _ = impl.sdpa_fwd(q, k, v, 1.3, causal)
        for i in range(10):
            vv = v[0, 0, : (i + 1 if causal else 10)]
            assert np.all(O[0, 0, i] >= vv.min(axis=0) - 1e-14)
            assert np.all(O[0, 0, i] <= vv.max(axis=0) + 1e-14)


def pin_merge(impl):
    """Splitting the keys into two sets a, b and merging the partial results
    with lse = logaddexp(lse_a, lse_b), O = e^(lse_a-lse) O_a + e^(lse_b-lse) O_b
    gives the full result.  This is the identity the tiled online softmax
    relies on (the FlashAttention article's block-by-block computation)."""
    r = _rng(17)
    q, k, v = (r.standard_normal((1, 1, 6, 4)) for _ in range(3))
    k = np.concatenate([k, r.standard_normal((1, 1, 5, 4))], axis=2)
    v = np.concatenate([v, r.standard_normal((1, 1, 5, 4))], axis=2)
    O, L = impl.sdpa_fwd(q, k, v, 0.8, False)
    Oa, La = impl.sdpa_fwd(q, k[:, :, :4], v[:, :, :4], 0.8, False)
    Ob, Lb = impl.sdpa_fwd(q, k[:, :, 4:], v[:, :, 4:], 0.8, False)
    Lm = np.logaddexp(La, Lb)
    Om = np.exp(La - Lm)[..., None] * Oa + np.exp(Lb - Lm)[..., None] * Ob
    _close(Lm, L, 1e-13, "merge lse")
    _close(Om, O, 1e-13, "merge O")


def pin_causal_prefix(impl):
    """Causal row i equals non-causal attention of q_i over keys 0..i."""
    r = _rng(18)
    q, k, v = (r.standard_normal((1, 1, 7, 3)) for _ in range(3))
    O, L = impl.sdpa_fwd(q, k, v, 0.9, True)
    for i in range(7):
        Oi, Li = impl.sdpa_fwd(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.9, False)
        _close(O[0, 0, i], Oi[0, 0, 0], 1e-14, "causal prefix O")
        _close(L[0, 0, i], Li[0, 0, 0], 1e-14, "causal prefix lse")


def pin_causal_wide(impl):
    """Top-left causal alignment with more keys than queries: row i still
    sees keys 0..i only, so keys past the last query never matter."""
    r = _rng(19)
    q = r.standard_normal((1, 1, 4, 3))
    k, v = r.standard_normal((1, 1, 9, 3)), r.standard_normal((1, 1, 9, 3))
    O, L = impl.sdpa_fwd(q, k, v, 0.5, True)
    O2, L2 = impl.sdpa_fwd(q, k[:, :, :4], v[:, :, :4], 0.5, True)
    _close(O, O2, 1e-14, "causal wide O")
    _close(L, L2, 1e-14, "causal wide lse")


def pin_varlen_concat(impl):
    """A packed batch equals the concatenation of per-sequence dense results
    (each sequence attends only to itself), including a length-1 sequence."""
    r = _rng(20)
    lens = [3, 1, 6, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 5
    q, k, v = (r.standard_normal((T, H, d)) for _ in range(3))
    for causal in (False, True):
        O, L = impl.sdpa_fwd_varlen(q, k, v, cu, 0.45, causal)
        assert O.shape == (T, H, d) and L.shape == (T, H)
        for s in range(len(lens)):
            a, b = cu[s], cu[s + 1]
            tr = lambda x: np.transpose(x[a:b], (1, 0, 2))[None]  # [1,H,n,d]
            Od, Ld = impl.sdpa_fwd(tr(q), tr(k), tr(v), 0.45, causal)
            _close(O[a:b], np.transpose(Od[0], (1, 0, 2)), 1e-14, "varlen O")
            _close(L[a:b], Ld[0].T, 1e-14, "varlen lse")


def pin_rows(impl):
    """Row sampling returns exactly the selected rows of the full result,
    also under the causal mask (rows keep their own query index)."""
    r = _rng(21)
    q, k, v = (r.standard_normal((1, 2, 12, 4)) for _ in range(3))
    rows = np.array([0, 3, 7, 11])
    for causal in (False, True):
        O, L = impl.sdpa_fwd(q, k, v, 0.5, causal)
        Or, Lr = impl.sdpa_fwd_rows(q, k, v, 0.5, causal, rows)
        _close(Or, O[:, :, rows], 1e-14, "rows O")
        _close(Lr, L[:, :, rows], 1e-14, "rows lse")


def pin_tutorial_example_shape(impl):
    """The tutorial prints the output of its 2x3x8 randn example
    (tests/golden/tutorial_example_output.txt).  Its inputs are unseeded and
    not printed, so only the shape (2,3,8) is pinned; values are unpinned."""
    with open(os.path.join(GOLDEN, "tutorial_example_output.txt")) as f:
        body = "".join(ln for ln in f if not ln.startswith("#"))
        nums = [float(x) for x in body.replace("[", " ").replace("]", " ")
                .replace(",", " ").split() if _isnum(x)]
    assert len(nums) == 2 * 3 * 8
    r = _rng(22)
    q, k, v = (r.standard_normal((2, 1, 3, 8)) for _ in range(3))
    O, L = impl.sdpa_fwd(q, k, v, 1 / math.sqrt(8), False)
    assert O.shape[0] * O.shape[2] * O.shape[3] == len(nums)
    assert L.shape == (2, 1, 3)


def _isnum(x):
    try:
        float(x)
        return True
    except ValueError:
        return False


ALL_PINS = [pin_brute_force, pin_library_softmax, pin_scale_zero, pin_identical_keys,
            pin_causal_row0, pin_two_keys_logistic, pin_one_hot_selection,
            pin_values_constant, pin_hand_example, pin_permutations, pin_key_shift,
            pin_convexity, pin_merge, pin_causal_prefix, pin_causal_wide,
            pin_varlen_concat, pin_rows, pin_tutorial_example_shape]

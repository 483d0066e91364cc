"""Pins of the block-sparse oracle (oracle/block_sparse.py).

* An all-ones mask gives the dense oracle; an all-zero mask gives O = 0,
  lse = -inf.
* A lower-triangular block mask with causal masking gives plain causal
  attention.
* One allowed key block per row equals dense attention over that block's
  keys alone.
* Random masks match the pure-Python brute force (its own visibility
  callback) on tiny shapes.
* Planted mistakes (transposed mask, off-by-one block index, mask ignored)
  are caught.
"""
import numpy as np
import pytest

from oracle import block_sparse as bs
from oracle import brute
from oracle import sdpa as dense


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_ones_is_dense():
    q, k, v = _rand((2, 3, 10, 4), 1), _rand((2, 3, 13, 4), 2), _rand((2, 3, 13, 4), 3)
    for causal in (False, True):
        o, l = bs.sdpa_fwd_block_sparse(q, k, v, np.ones((1, 3, 4), np.uint8), 0.6, causal, block=4)
        od, ld = dense.sdpa_fwd(q, k, v, 0.6, causal)
        np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l, ld, rtol=1e-13, atol=1e-13)


def test_all_zero_gives_empty_rows():
    q, k, v = _rand((1, 2, 7, 3), 4), _rand((1, 2, 7, 3), 5), _rand((1, 2, 7, 3), 6)
    o, l = bs.sdpa_fwd_block_sparse(q, k, v, np.zeros((2, 2, 2), np.uint8), 0.5, False, block=4)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_lower_triangular_blocks_with_causal_is_causal():
    q, k, v = _rand((1, 2, 12, 4), 7), _rand((1, 2, 12, 4), 8), _rand((1, 2, 12, 4), 9)
    tri = np.tril(np.ones((3, 3), np.uint8))[None]
    o, l = bs.sdpa_fwd_block_sparse(q, k, v, tri, 0.7, True, block=4)
    od, ld = dense.sdpa_fwd(q, k, v, 0.7, True)
    np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l, ld, rtol=1e-13, atol=1e-13)


def test_single_block_per_row_is_attention_over_that_block():
    q, k, v = _rand((1, 1, 8, 3), 10), _rand((1, 1, 12, 3), 11), _rand((1, 1, 12, 3), 12)
    m = np.zeros((1, 2, 3), np.uint8)
    m[0, 0, 2] = 1   # query block 0 sees key block 2 only
    m[0, 1, 0] = 1   # query block 1 sees key block 0 only
    o, l = bs.sdpa_fwd_block_sparse(q, k, v, m, 0.8, False, block=4)
    o0, l0 = dense.sdpa_fwd(q[:, :, :4], k[:, :, 8:12], v[:, :, 8:12], 0.8, False)
    o1, l1 = dense.sdpa_fwd(q[:, :, 4:], k[:, :, 0:4], v[:, :, 0:4], 0.8, False)
    np.testing.assert_allclose(o[:, :, :4], o0, rtol=1e-13)
    np.testing.assert_allclose(o[:, :, 4:], o1, rtol=1e-13)
    np.testing.assert_allclose(l[:, :, :4], l0, rtol=1e-13)
    np.testing.assert_allclose(l[:, :, 4:], l1, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_masks_match_brute_force(causal, seed):
    nq, nk, blk = 9, 11, 3
    q, k, v = _rand((1, 2, nq, 3), 20 + seed), _rand((1, 2, nk, 3), 30 + seed), _rand((1, 2, nk, 3), 40 + seed)
    m = (np.random.default_rng(seed).random((2, 3, 4)) < 0.5).astype(np.uint8)
    o, l = bs.sdpa_fwd_block_sparse(q, k, v, m, 0.9, causal, block=blk)
    for h in range(2):
        bo, bl = brute.attend(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), 0.9, causal,
                              allowed=lambda i, j, h=h: m[h, i // blk, j // blk] != 0)
        np.testing.assert_allclose(o[0, h], np.array(bo), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l[0, h], np.array(bl), rtol=1e-12, atol=1e-12)


def _mutant(q, k, v, m, scale, causal, blk, mistake):
    nq, nk = q.shape[0], k.shape[0]
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    if mistake == "transposed":   # query and key block indices swapped
        vis = m[j // blk, i // blk] != 0
    elif mistake == "off_by_one":
        vis = m[i // blk, np.minimum(j // blk + 1, m.shape[1] - 1)] != 0
    else:  # ignored
        vis = np.ones((nq, nk), bool)
    if causal:
        vis = vis & (j <= i)
    return bs.attend_masked(q, k, v, scale, vis)


@pytest.mark.parametrize("mistake", ["transposed", "off_by_one", "ignored"])
def test_planted_mistakes_are_caught(mistake):
    nq = nk = 9
    blk = 3
    q, k, v = _rand((nq, 3), 50), _rand((nk, 3), 51), _rand((nk, 3), 52)
    m = np.array([[1, 0, 0], [1, 1, 0], [0, 1, 1]], np.uint8)
    want = brute.attend(q.tolist(), k.tolist(), v.tolist(), 0.7, False,
                        allowed=lambda i, j: m[i // blk, j // blk] != 0)
    o, l = _mutant(q, k, v, m, 0.7, False, blk, mistake)
    assert not np.allclose(o, np.array(want[0]), rtol=1e-9, atol=1e-9)
    ok, _ = bs.attend_masked(q, k, v, 0.7, bs.visibility(nq, nk, m, blk, False))
    np.testing.assert_allclose(ok, np.array(want[0]), rtol=1e-12, atol=1e-12)


def test_visibility_rows_selects_rows():
    m = np.random.default_rng(3).integers(0, 2, (3, 2))
    full = bs.visibility(20, 13, m, 7, True)
    rows = np.array([0, 6, 7, 19])
    np.testing.assert_array_equal(bs.visibility(20, 13, m, 7, True, rows), full[rows])

"""GPU parity of the block-sparse forward (sdpa_fwd_block_sparse) against the
fp64 block-sparse oracle, through the C ABI.

Tolerances are those of the dense forward (tests/gpu_util.py).  Rows that
see no key must come back as exact zeros with lse = -inf, on both sides.
Masks are seeded Bernoulli draws per 128x128 block (inputs.make_block_mask).
"""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from oracle import block_sparse as obsp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _run(w, mask, out_f32=False, q=None, k=None, v=None):
    q, k, v = (G.to_device(x, w.dtype) if t is None else t
               for x, t in ((w.q, q), (w.k, k), (w.v, v)))
    m = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, is_causal=w.is_causal, scale=float(w.scale), block_mask=m,
        out_dtype=torch.float32 if out_f32 else None, return_lse=True)
    torch.cuda.synchronize()
    return out.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def _check(o, lse, ref, lref, dtype, what):
    empty = np.isneginf(lref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: rows with no key are not zero"
    live = ~empty
    if np.any(live):
        G.assert_parity(o[live], ref[live], dtype, what, lse[live], lref[live])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_sweep(dtype, d, causal):
    # 300 rows: three mask rows, the last one ragged; per-head masks at half
    # density, so some query blocks see no key block at all
    w = inputs.make_dense(2, 3, 300, 300, d, dtype, "normal", causal, seed=d, cfg=80)
    mask = inputs.make_block_mask(3, 300, 300, 0.5, seed=d + int(causal), cfg=80)
    o, lse = _run(w, mask, out_f32=dtype == "bf16")
    ref, lref = obsp.sdpa_fwd_block_sparse(w.q64, w.k64, w.v64, mask, w.scale, causal)
    _check(o, lse, ref, lref, dtype, f"{dtype} d{d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 300), (300, 1), (129, 700), (700, 129), (513, 513)])
def test_block_sparse_shapes_shared_mask(causal, nq, nk):
    w = inputs.make_dense(2, 4, nq, nk, 64, "f16", "normal", causal, seed=nq + nk, cfg=81)
    mask = inputs.make_block_mask(1, nq, nk, 0.6, seed=nq, cfg=81)
    o, lse = _run(w, mask)
    ref, lref = obsp.sdpa_fwd_block_sparse(w.q64, w.k64, w.v64, mask, w.scale, causal)
    _check(o, lse, ref, lref, "f16", f"nq{nq} nk{nk} causal={causal}")


def test_block_sparse_2048_local_and_random():
    """Diagonal plus random blocks at a quarter density, 16 x 16 blocks."""
    w = inputs.make_dense(1, 4, 2048, 2048, 64, "bf16", "normal", False, seed=5, cfg=82)
    mask = inputs.make_block_mask(4, 2048, 2048, 0.25, diagonal=True, seed=5, cfg=82)
    o, lse = _run(w, mask, out_f32=True)
    ref, lref = obsp.sdpa_fwd_block_sparse(w.q64, w.k64, w.v64, mask, w.scale, False)
    assert not np.any(np.isneginf(lref))
    _check(o, lse, ref, lref, "bf16", "N2048 local+random")


def test_all_zero_mask_gives_zeros_and_neg_inf():
    w = inputs.make_dense(1, 2, 200, 200, 64, "f16", "normal", False, seed=6, cfg=83)
    o, lse = _run(w, np.zeros((1, 2, 2), np.uint8))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_equals_dense_path(d, causal):
    """With every block visible the block-sparse kernel takes the same
    arithmetic steps as the dense one, key tile by key tile from key 0:
    bit-identical results.  2 x 65 units of two query tiles: above the tile
    count under which plain launches split each workgroup's keys over two
    wave groups (another order of additions)."""
    w = inputs.make_dense(2, 65, 333, 333, d, "f16", "normal", causal, seed=d, cfg=84)
    o, lse = _run(w, np.ones((1, 3, 3), np.uint8))
    od, ld = G.run(w)
    assert np.array_equal(o, od) and np.array_equal(lse, ld)


def test_shared_mask_equals_replicated_per_head_mask():
    w = inputs.make_dense(2, 3, 400, 400, 64, "f16", "normal", True, seed=7, cfg=85)
    shared = inputs.make_block_mask(1, 400, 400, 0.5, seed=7, cfg=85)
    a = _run(w, shared)
    b = _run(w, np.repeat(shared, 3, axis=0))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_masked_blocks_are_never_read():
    """Key blocks no query block may see hold NaN in K and V; the result must
    match the oracle run on the same inputs with those blocks zeroed."""
    w = inputs.make_dense(1, 2, 512, 512, 64, "f16", "normal", False, seed=8, cfg=86)
    mask = inputs.make_block_mask(2, 512, 512, 0.6, diagonal=True, seed=8, cfg=86)
    mask[:, :, 1] = 0
    mask[:, 2, :] = 0                # a query block that sees nothing
    k = G.to_device(w.k, "f16")
    v = G.to_device(w.v, "f16")
    k[:, :, 128:256] = float("nan")
    v[:, :, 128:256] = float("nan")
    o, lse = _run(w, mask, k=k, v=v)
    k64, v64 = w.k64.copy(), w.v64.copy()
    k64[:, :, 128:256] = 0.0
    v64[:, :, 128:256] = 0.0
    ref, lref = obsp.sdpa_fwd_block_sparse(w.q64, k64, v64, mask, w.scale, False)
    _check(o, lse, ref, lref, "f16", "NaN in masked blocks")
    assert np.all(np.isneginf(lse[:, :, 256:384]))


def test_binding_rejects_bad_masks():
    q = torch.zeros(1, 2, 200, 64, device="cuda", dtype=torch.float16)
    bad = [torch.ones(2, 2, 2, device="cuda", dtype=torch.float32),   # dtype
           torch.ones(3, 2, 2, device="cuda", dtype=torch.uint8),     # heads not 1 or H
           torch.ones(2, 1, 2, device="cuda", dtype=torch.uint8),     # too few block rows
           torch.ones(2, 2, 2, dtype=torch.uint8)]                    # host memory
    for m in bad:
        with pytest.raises(sdpa.SdpaError):
            sdpa.scaled_dot_product_attention(q, q, q, block_mask=m)
    with pytest.raises(sdpa.SdpaError):
        q32 = q.float()
        sdpa.scaled_dot_product_attention(q32, q32, q32,
                                          block_mask=torch.ones(1, 2, 2, device="cuda",
                                                                dtype=torch.uint8))


def test_block_sparse_workload_full_size():
    """The benchmarked block-sparse workload (B1 H16 N65536 d64 bf16, one
    mask per head) in the benchmark's launch configuration, checked on its
    256 sampled query rows in four heads."""
    w = inputs.make_config(6)
    q, k, v = (G.to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    bm = torch.from_numpy(w.block_mask).to("cuda")
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, scale=float(w.scale), block_mask=bm, out_dtype=torch.float32,
        return_lse=True)
    torch.cuda.synchronize()
    rows = torch.from_numpy(w.rows).to("cuda")
    for h in (0, 5, 10, 15):
        vis = obsp.visibility(w.Nq, w.Nk, w.block_mask[h], 128, False, w.rows)
        ref, lref = obsp.attend_masked(inputs.storage_to_f64(w.q[0, h, w.rows], w.dtype),
                                       inputs.storage_to_f64(w.k[0, h], w.dtype),
                                       inputs.storage_to_f64(w.v[0, h], w.dtype), w.scale, vis)
        o = out[0, h].index_select(0, rows).double().cpu().numpy()
        ls = lse[0, h].index_select(0, rows).double().cpu().numpy()
        _check(o, ls, ref, lref, "bf16", f"block_sparse head {h}")

"""Seeded random sweep over the forward and backward entry points, through
the binding and the C ABI, against the fp64 oracles.

Each case draws an entry point (dense, packed, dropout, elementwise mask of
each kind, mask with dropout, block-sparse), an input type, a head
dimension, the causal flag and ragged sizes (query and key lengths that are
rarely tile multiples, Nq != Nk), so that combinations the targeted tests
do not enumerate are still compared element by element at the tolerances
of tests/gpu_util.py.  The draws come from a fixed seed: a failure names
its case and reproduces.
"""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
import oracle
from exact_attention_sdpa_amd import inputs
from oracle import block_sparse as obsp
from oracle import dropout as odrop
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

FWD_KINDS = ["dense", "packed", "dropout", "packed_dropout", "mask_bool", "mask_add",
             "mask_add_f32", "mask_bool_dropout", "mask_add_dropout", "block_sparse"]
N_FWD = 120
N_BWD = 48


def _fwd_case(i):
    r = np.random.default_rng([2024, i])
    kind = FWD_KINDS[i % len(FWD_KINDS)]
    dtype = ["f16", "bf16"][int(r.integers(2))]
    d = [32, 64, 128][int(r.integers(3))]
    causal = bool(r.integers(2))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    nq = int(r.integers(1, 520))
    nk = nq if (causal or kind.startswith("packed")) else int(r.integers(1, 520))
    p = float(r.choice([0.1, 0.3, 0.6]))
    return r, kind, dtype, d, causal, B, H, nq, nk, p


@pytest.mark.parametrize("i", range(N_FWD))
def test_forward_fuzz(i):
    r, kind, dtype, d, causal, B, H, nq, nk, p = _fwd_case(i)
    what = f"case {i}: {kind} {dtype} d{d} causal={causal} B{B} H{H} Nq{nq} Nk{nk}"
    print(what, flush=True)
    seed, off = int(r.integers(1 << 30)), int(r.integers(1 << 20))
    drop = "dropout" in kind
    kw = dict(is_causal=causal, return_lse=True,
              out_dtype=torch.float32 if dtype == "bf16" else None)
    if drop:
        kw.update(dropout_p=p, dropout_seed=seed, dropout_offset=off)
    if kind.startswith("packed"):
        lens = [int(x) for x in r.integers(0, 400, size=int(r.integers(1, 5)))]
        lens[0] = max(lens[0], 1)   # at least one row in the batch
        w = inputs.make_varlen(lens, H, d, dtype, "normal", causal, seed=i, cfg=150)
        kw.update(cu_seqlens=torch.from_numpy(w.cu_seqlens).cuda(), max_seqlen=w.Nq)
    else:
        w = inputs.make_dense(B, H, nq, nk, d, dtype, "normal", causal, seed=i, cfg=150)
    kw["scale"] = float(w.scale)
    q, k, v = (G.to_device(x, dtype) for x in (w.q, w.k, w.v))
    mask = mkind = None
    if kind.startswith("mask"):
        mkind = "bool" if kind.startswith("mask_bool") else "add"
        mdt = "f32" if kind == "mask_add_f32" else dtype
        mask = inputs.make_attn_mask((B, H, nq, nk), mkind, keep=0.85, bias_std=2.0,
                                     seed=i, cfg=151, dtype=mdt)
        kw["attn_mask"] = (torch.from_numpy(mask).cuda().bool() if mkind == "bool"
                           else G.to_device(mask, mdt))
    if kind == "block_sparse":
        mask = inputs.make_block_mask(H, nq, nk, 0.5, diagonal=True, seed=i, cfg=152)
        kw["block_mask"] = torch.from_numpy(mask).cuda()
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, **kw)
    torch.cuda.synchronize()
    o, l = out.double().cpu().numpy(), lse.double().cpu().numpy()

    if kind == "dense":
        ref, lref = oracle.sdpa_fwd(w.q64, w.k64, w.v64, w.scale, causal)
    elif kind == "packed":
        ref, lref = oracle.sdpa_fwd_varlen(w.q64, w.k64, w.v64, w.cu_seqlens, w.scale, causal)
    elif kind == "dropout":
        ref, lref = odrop.sdpa_fwd_dropout(w.q64, w.k64, w.v64, w.scale, causal, p, seed, off)
    elif kind == "packed_dropout":
        ref, lref = odrop.sdpa_fwd_dropout_varlen(w.q64, w.k64, w.v64, w.cu_seqlens, w.scale,
                                                  causal, p, seed, off)
    elif kind == "block_sparse":
        ref, lref = obsp.sdpa_fwd_block_sparse(w.q64, w.k64, w.v64, mask, w.scale, causal)
    else:
        m64 = mask if mkind == "bool" else inputs.storage_to_f64(
            mask, "f32" if kind == "mask_add_f32" else dtype)
        if drop:
            ref, lref = odrop.sdpa_fwd_masked_dropout(w.q64, w.k64, w.v64, m64, mkind, w.scale,
                                                      causal, p, seed, off)
        else:
            ref, lref = oracle.sdpa_fwd_masked(w.q64, w.k64, w.v64, m64, mkind, w.scale, causal)

    # rows that see no key (masks, block masks): zeros and lse = -inf
    dead = np.isneginf(lref)
    assert np.array_equal(np.isneginf(l), dead), f"{what}: empty rows differ"
    assert np.all(o[dead] == 0.0), f"{what}: empty rows not zero"
    live = ~dead
    if not np.any(live):
        return
    scale_o = (1.0 - p) if drop else 1.0   # kept weights carry 1/(1-p), and their rounding
    G.assert_parity(o[live] * scale_o, ref[live] * scale_o, dtype, what, l[live], lref[live])


@pytest.mark.parametrize("i", range(N_BWD))
def test_backward_fuzz(i):
    """Dense, masked and dropout backward on random ragged shapes, within the
    elementwise bounds of the targeted backward tests."""
    from tests import test_parity_bwd_dropout_gpu as TD
    from tests import test_parity_bwd_gpu as TB
    from tests import test_parity_bwd_masked_gpu as TM
    r = np.random.default_rng([2025, i])
    kind = ["dense", "mask", "dropout"][i % 3]
    dtype = ["f16", "bf16"][int(r.integers(2))]
    d = [32, 64, 128][int(r.integers(3))]
    causal = bool(r.integers(2))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    nq = int(r.integers(2, 300))
    nk = nq if causal or kind == "dropout" else int(r.integers(2, 300))
    grad_f32 = bool(r.integers(2))
    what = (f"case {i}: {kind} {dtype} d{d} causal={causal} B{B} H{H} Nq{nq} Nk{nk} "
            f"f32grad={grad_f32}")
    print(what, flush=True)
    w = inputs.make_dense(B, H, nq, nk, d, dtype, "normal", causal, seed=i, cfg=153)
    do = inputs.make_grad_out(w, seed=i, cfg=153)
    if kind == "dense":
        TB._check(TB._run(w, do, grad_f32=grad_f32), TB._ref_and_bound(w, do, grad_f32=grad_f32),
                  what)
    elif kind == "mask":
        mk = ["bool", "add"][int(r.integers(2))]
        m = inputs.make_attn_mask((B, H, nq, nk), mk, keep=0.85, seed=i, cfg=154, dtype=dtype)
        TM._check(w, TM._run(w, do, TM._mask_t(m, mk, dtype), grad_f32=grad_f32), do, m, mk,
                  dtype, grad_f32=grad_f32)
    else:
        p, seed = float(r.choice([0.1, 0.4])), int(r.integers(1 << 30))
        TD._check(TD._run(w, do, p, seed, offset=3, grad_f32=grad_f32),
                  TD._ref_and_bound(w, do, p, seed, 3, grad_f32=grad_f32), what)

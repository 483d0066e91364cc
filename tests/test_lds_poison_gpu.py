"""The forward kernels under the LDS-poisoning debug build (libsdpa_debug.so,
built with SDPA_LDS_POISON=1): LDS is filled with NaN when a tile starts,
and every staging slot is refilled with NaN after the barrier that ends its
reads, before the step that stores the next tile there.  A read of LDS
ahead of its data (a missing or misplaced barrier) then makes the output
NaN; with the barriers right, every variant still matches the fp64 oracles
at the tolerances of tests/gpu_util.py.  The binding is pointed at the
debug library for the duration of each test.
"""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
import oracle
from exact_attention_sdpa_amd import _lib, inputs
from oracle import block_sparse as obsp
from oracle import dropout as odrop
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_lib():
    saved = _lib._lib
    _lib._lib = _lib.lib_debug()
    try:
        yield
    finally:
        _lib._lib = saved


def _fwd(w, out_f32, **kw):
    q, k, v = (G.to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    if w.varlen:
        kw.update(cu_seqlens=torch.from_numpy(w.cu_seqlens).cuda(), max_seqlen=w.Nq)
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, is_causal=w.is_causal, scale=float(w.scale), return_lse=True,
        out_dtype=torch.float32 if out_f32 else None, **kw)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_dense_and_packed(debug_lib, dtype, d, causal):
    # several key tiles with a ragged tail, so every staging buffer is
    # poisoned and refilled more than once
    w = inputs.make_dense(1, 3, 333, 333, d, dtype, "normal", causal, seed=d, cfg=140)
    o, lse = _fwd(w, dtype == "bf16")
    ref, lref = oracle.sdpa_fwd(w.q64, w.k64, w.v64, w.scale, causal)
    G.assert_parity(o, ref, dtype, f"poisoned dense {dtype} d{d} causal={causal}", lse, lref)
    wv = inputs.make_varlen([1, 200, 0, 65, 300], 2, d, dtype, "normal", causal, seed=d, cfg=141)
    o, lse = _fwd(wv, dtype == "bf16")
    ref, lref = oracle.sdpa_fwd_varlen(wv.q64, wv.k64, wv.v64, wv.cu_seqlens, wv.scale, causal)
    G.assert_parity(o, ref, dtype, f"poisoned packed {dtype} d{d} causal={causal}", lse, lref)


@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_variants(debug_lib, causal):
    w = inputs.make_dense(2, 2, 300, 300, 64, "f16", "normal", causal, seed=7, cfg=142)
    # dropout
    o, lse = _fwd(w, True, dropout_p=0.25, dropout_seed=5, dropout_offset=1)
    ref, lref = odrop.sdpa_fwd_dropout(w.q64, w.k64, w.v64, w.scale, causal, 0.25, 5, 1)
    G.assert_parity(o * 0.75, ref * 0.75, "f16", "poisoned dropout", lse, lref)
    # block-sparse (all blocks kept along the diagonal, so no row is empty)
    bm = inputs.make_block_mask(2, 300, 300, 0.5, diagonal=True, seed=7, cfg=142)
    o, lse = _fwd(w, True, block_mask=torch.from_numpy(bm).cuda())
    ref, lref = obsp.sdpa_fwd_block_sparse(w.q64, w.k64, w.v64, bm, w.scale, causal)
    G.assert_parity(o, ref, "f16", "poisoned block-sparse", lse, lref)
    # additive mask, finite everywhere
    m = inputs.make_attn_mask((2, 2, 300, 300), "add", keep=1.0, bias_std=1.0, seed=7, cfg=142,
                              dtype="f16")
    o, lse = _fwd(w, True, attn_mask=G.to_device(m, "f16"))
    ref, lref = oracle.sdpa_fwd_masked(w.q64, w.k64, w.v64, inputs.storage_to_f64(m, "f16"),
                                       "add", w.scale, causal)
    G.assert_parity(o, ref, "f16", "poisoned additive mask", lse, lref)
    assert np.all(np.isfinite(o))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_wide_d32_grid(debug_lib, dtype, causal):
    """A d = 32 grid of at least 2048 query tiles (the kernels with two
    query blocks per wave, whose 16-bit epilogue stages both blocks' rows in
    LDS), plain and with dropout, on sampled units."""
    w = inputs.make_dense(64, 32, 333, 333, 32, dtype, "normal", causal, seed=3, cfg=143)
    assert w.B * w.H * -(-w.Nq // 256) >= 2048
    q64, k64, v64 = w.q64, w.k64, w.v64
    units = [0, w.B * w.H - 1] + [int(u) for u in
                                  np.random.default_rng(9).choice(w.B * w.H, 4, replace=False)]
    o, lse = _fwd(w, dtype == "bf16")
    od, lsed = _fwd(w, dtype == "bf16", dropout_p=0.25, dropout_seed=5, dropout_offset=1)
    for u in units:
        b, h = divmod(u, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref, lref = oracle.sdpa_fwd(q64[sl], k64[sl], v64[sl], w.scale, causal)
        G.assert_parity(o[sl], ref, dtype, f"poisoned wide {dtype} unit {b},{h}", lse[sl], lref)
        ref, lref = odrop.attend_dropout(q64[b, h], k64[b, h], v64[b, h], w.scale, causal, 0.25,
                                         5, 1, u)
        G.assert_parity(od[b, h] * 0.75, ref * 0.75, dtype,
                        f"poisoned wide dropout {dtype} unit {b},{h}", lsed[b, h], lref)


# --- the backward kernels under poisoning: their K/V (dQ kernel) and
# Q/dO/row-statistic/mask (dK/dV kernel) staging buffers are poisoned the
# same way; the bounds are those of the backward parity tests

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_backward(debug_lib, dtype, d, causal):
    from tests import test_parity_bwd_gpu as TB
    # several query and key tiles with ragged tails, so every staging buffer
    # of both kernels is poisoned and refilled more than once; f32 and
    # 16-bit gradients (the latter leave through LDS)
    w = inputs.make_dense(2, 2, 200, 200, d, dtype, "normal", causal, seed=5, cfg=144)
    do = inputs.make_grad_out(w, seed=5, cfg=144)
    for grad_f32 in (True, False):
        TB._check(TB._run(w, do, grad_f32=grad_f32), TB._ref_and_bound(w, do, grad_f32=grad_f32),
                  f"poisoned bwd {dtype} d{d} causal={causal} f32grad={grad_f32}")


@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_backward_variants(debug_lib, causal):
    from tests import test_parity_bwd_dropout_gpu as TD
    from tests import test_parity_bwd_masked_gpu as TM
    w = inputs.make_dense(2, 2, 150, 161, 64, "f16", "normal", causal, seed=6, cfg=145)
    do = inputs.make_grad_out(w, seed=6, cfg=145)
    for kind, mdt in (("bool", "f16"), ("add", "f16")):
        m = inputs.make_attn_mask((2, 2, 150, 161), kind, keep=0.8, seed=6, cfg=146, dtype=mdt)
        TM._check(w, TM._run(w, do, TM._mask_t(m, kind, mdt)), do, m, kind, mdt)
    wd = inputs.make_dense(2, 2, 160, 160, 64, "f16", "normal", causal, seed=7, cfg=147)
    dod = inputs.make_grad_out(wd, seed=7, cfg=147)
    TD._check(TD._run(wd, dod, 0.2, seed=21, offset=2), TD._ref_and_bound(wd, dod, 0.2, 21, 2),
              f"poisoned bwd dropout causal={causal}")

"""GPU parity of the backward pass (sdpa_bwd) against the fp64 gradient
oracle, through the C ABI.

The forward runs on the GPU first (its out and lse feed the backward, as in
training); the oracle differentiates the exact definition from the same
stored q, k, v and dO.

Tolerance, from the arithmetic (elementwise).  q, k, v and dO are exact
matrix-core operands and every product accumulates in fp32.  The roundings
are: P and dS, each rounded to the input type before its product (f16:
relative u = 2^-11, and below 2^-14, f16's subnormal range, the error is
absolute instead, at most U_SUB = 2^-25 per visible pair; bf16: relative
u = 2^-8); the forward's O inside D_i = <dO_i, O_i>,
whose error per element is at most
u_f * sum_j P_ij |v_jc| (its own f16 P, u_f = 2^-11) plus u_o |O_ic| (rounding to the
output dtype), so D_i is off by at most
    e_D,i = sum_c |dO_ic| (u_f (P|V|)_ic + u_o |O_ic|);
the forward's lse, whose error e_lse (at most 1e-4, the forward's bound)
scales P by up to e_lse; and, for gradients stored in f16/bf16, one final
rounding (plus U_SUB for an f16 result in the subnormal range).  So, per
element,
    |err dV_j| <= sum_i ((u + e_lse) P_ij + U_SUB) |dO_i|
    |err dQ_i| <= scale * sum_j (u |dS_ij| + U_SUB + P_ij (e_D,i + e_lse |dP_ij - D_i|)) |k_j|
    |err dK_j| <= the same with q_i in place of k_j,
plus the output rounding.  The sums are taken from fp64 intermediates, and
the test allows twice the bound for fp32 accumulation and exp2.  Note the
bound is relative to the sum of magnitudes, not to the result: dQ and dK are
sums whose terms cancel (every row of dS sums to zero).
"""
import dataclasses
import types

import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from oracle import grad as ograd
from oracle import sdpa as ofwd
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu

U = 2.0 ** -11
U_SUB = 2.0 ** -25   # half the f16 subnormal spacing
E_LSE = 1e-4
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -24}   # bf16 runs keep O in f32
U_GRAD = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# rounding of P and dS before the dV, dK, dQ products: f16 for f16 inputs,
# bf16 (relative 2^-8, no subnormal range in play) for bf16 inputs
U_P = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
U_SUBP = {"f16": 2.0 ** -25, "bf16": 0.0}


def _run(w, do, grad_f32=True):
    q, k, v = (to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    g = to_device(do, w.dtype)
    out_f32 = w.dtype == "bf16"
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, is_causal=w.is_causal, scale=float(w.scale),
        out_dtype=torch.float32 if out_f32 else None, return_lse=True)
    dq, dk, dv = sdpa.scaled_dot_product_attention_backward(
        q, k, v, out, lse, g, is_causal=w.is_causal, scale=float(w.scale),
        grad_dtype=torch.float32 if grad_f32 else None)
    torch.cuda.synchronize()
    return [t.to(torch.float64).cpu().numpy() for t in (dq, dk, dv)]


def _ref_and_bound(w, do, grad_f32=True):
    """Oracle gradients and the elementwise error bound of the docstring."""
    do64 = inputs.storage_to_f64(do, w.dtype)
    ref = ograd.sdpa_bwd(w.q64, w.k64, w.v64, do64, float(w.scale), w.is_causal)
    o64, _ = ofwd.sdpa_fwd(w.q64, w.k64, w.v64, float(w.scale), w.is_causal)
    sc, uo = float(w.scale), U_OUT[w.dtype]
    bq, bk, bv = (np.zeros_like(r) for r in ref)
    for b in range(w.B):
        for h in range(w.H):
            q, k, v, g = w.q64[b, h], w.k64[b, h], w.v64[b, h], do64[b, h]
            p = ograd._probs(q, k, sc, w.is_causal)
            dp = g @ v.T
            dd = np.sum(g * o64[b, h], axis=1, keepdims=True)
            ds_abs = np.abs(p * (dp - dd))
            e_d = np.sum(np.abs(g) * (U * (p @ np.abs(v)) + uo * np.abs(o64[b, h])),
                         axis=1, keepdims=True)
            shift = p * (e_d + E_LSE * np.abs(dp - dd))
            vis = (p > 0).astype(np.float64)
            up, us = U_P[w.dtype], U_SUBP[w.dtype]
            t = up * ds_abs + us * vis + shift
            bv[b, h] = ((up + E_LSE) * p + us * vis).T @ np.abs(g)
            bq[b, h] = sc * (t @ np.abs(k))
            bk[b, h] = sc * (t.T @ np.abs(q))
    bounds = []
    for r, bd in zip(ref, (bq, bk, bv)):
        bd = 2.0 * bd
        if not grad_f32:
            bd = bd + U_GRAD[w.dtype] * np.abs(r) + (U_SUB if w.dtype == "f16" else 0.0)
        bounds.append(bd + 1e-30)
    return ref, bounds


def _check(got, ref_bound, what):
    ref, bounds = ref_bound
    for name, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bounds):
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        ratio = np.abs(g - r) / bd
        worst = float(np.max(ratio))
        assert worst <= 1.0, (f"{what} {name}: error {worst:.3f} x bound at "
                              f"{np.unravel_index(np.argmax(ratio), ratio.shape)}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dense_ragged(dtype, d, causal):
    w = inputs.make_dense(2, 2, 160, 160, d, dtype, "normal", causal, seed=3, cfg=40)
    do = inputs.make_grad_out(w, seed=3, cfg=40)
    _check(_run(w, do), _ref_and_bound(w, do), f"{dtype} d{d} causal={causal}")


@pytest.mark.parametrize("mag", [1e-6, 1e-9])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_bf16_small_upstream_gradients(mag, d, causal):
    """bf16 upstream gradients far below f16's normal range stay exact
    matrix-core operands: dq, dk and dv meet the same elementwise bound as
    for O(1) gradients (the bound is linear in dO), and none is flushed."""
    w = inputs.make_dense(1, 2, 200, 200, d, "bf16", "normal", causal, seed=11, cfg=43)
    do = inputs.make_grad_out(w, seed=11, cfg=43, scale=mag)
    got = _run(w, do)
    ref_bound = _ref_and_bound(w, do)
    _check(got, ref_bound, f"bf16 dO~{mag:g} d{d} causal={causal}")
    for g, r in zip(got, ref_bound[0]):
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        assert rel <= 1e-2, rel


@pytest.mark.parametrize("nq,nk", [(100, 260), (300, 70), (33, 1), (1, 50)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_nq_ne_nk(nq, nk, causal):
    w = inputs.make_dense(1, 3, nq, nk, 64, "f16", "normal", causal, seed=5, cfg=41)
    do = inputs.make_grad_out(w, seed=5, cfg=41)
    got = _run(w, do)
    _check(got, _ref_and_bound(w, do), f"nq{nq} nk{nk} causal={causal}")
    if causal and nk > nq:
        # keys past the last query are attended by no row: zero gradients
        assert np.all(got[1][:, :, nq:] == 0) and np.all(got[2][:, :, nq:] == 0)


def test_bwd_uniform_inputs_and_input_dtype_grads():
    w = inputs.make_dense(2, 4, 256, 256, 32, "f16", "uniform", False, seed=7, cfg=42)
    do = inputs.make_grad_out(w, seed=7, cfg=42)
    _check(_run(w, do, grad_f32=False), _ref_and_bound(w, do, grad_f32=False),
           "uniform f16 grads")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_1024_invariants_and_parity(causal):
    w = inputs.make_dense(1, 4, 1024, 1024, 64, "f16", "normal", causal, seed=9, cfg=43)
    do = inputs.make_grad_out(w, seed=9, cfg=43)
    got = _run(w, do)
    rb = _ref_and_bound(w, do)
    _check(got, rb, f"N1024 causal={causal}")
    dq, dk, dv = got
    do64 = inputs.storage_to_f64(do, w.dtype)
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, within the summed bounds
    assert np.all(np.abs(dk.sum(axis=2)) <= rb[1][1].sum(axis=2))
    assert np.all(np.abs(dv.sum(axis=2) - do64.sum(axis=2)) <= rb[1][2].sum(axis=2))


@pytest.mark.parametrize("cfg", [2, 3])
def test_bwd_full_workload_sampled_units(cfg):
    # the noncausal (B32 H32 N1024 d32) and causal (B32 H8 N1024 d64)
    # workloads at full size, in the launch configuration the benchmark's
    # backward times (gradients in the input dtype); the oracle checks four
    # whole (batch, head) units spread over the grid, the first and the last
    # among them
    w = inputs.make_config(cfg)
    do = inputs.make_grad_out(w, seed=cfg, cfg=46)
    got = _run(w, do, grad_f32=False)
    units = [(0, 0), (w.B // 3, w.H - 1), (2 * w.B // 3, w.H // 2), (w.B - 1, w.H - 1)]
    bi, hi = [b for b, _ in units], [h for _, h in units]
    f64 = lambda a: inputs.storage_to_f64(a[bi, hi][None], w.dtype)
    sub = types.SimpleNamespace(B=1, H=len(units), dtype=w.dtype, scale=w.scale,
                                is_causal=w.is_causal, q64=f64(w.q), k64=f64(w.k), v64=f64(w.v))
    _check([g[bi, hi][None] for g in got], _ref_and_bound(sub, do[bi, hi][None], grad_f32=False),
           f"{w.name} full size, sampled units")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_one_group_grid(dtype, d, causal):
    """The small grids above run the dQ and dK/dV kernels (dQ only at
    d = 128) with two groups of waves that add their sums; 130 units of two
    tiles (N = 300) run the one-group kernels, checked on four units against
    the oracle."""
    B, H, n = 1, 130, 300
    assert B * H * -(-n // 256) > 256
    w = inputs.make_dense(B, H, n, n, d, dtype, "normal", causal, seed=21 + causal, cfg=47)
    do = inputs.make_grad_out(w, seed=21, cfg=47)
    sub = dataclasses.replace(w, H=4, q=w.q[:, :4].copy(), k=w.k[:, :4].copy(),
                              v=w.v[:, :4].copy())
    for grad_f32 in (True, False):
        got = _run(w, do, grad_f32=grad_f32)
        _check([g[:, :4] for g in got], _ref_and_bound(sub, do[:, :4].copy(), grad_f32=grad_f32),
               f"one group {dtype} d{d} causal={causal} f32grad={grad_f32}")


def test_bwd_deterministic():
    w = inputs.make_dense(2, 2, 300, 300, 64, "bf16", "normal", True, seed=11, cfg=44)
    do = inputs.make_grad_out(w, seed=11, cfg=44)
    a, b = _run(w, do), _run(w, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_autograd_matches_explicit_backward():
    w = inputs.make_dense(1, 2, 192, 192, 64, "f16", "normal", True, seed=13, cfg=45)
    do = inputs.make_grad_out(w, seed=13, cfg=45)
    q, k, v = (to_device(x, w.dtype).requires_grad_(True) for x in (w.q, w.k, w.v))
    g = to_device(do, w.dtype)
    out = sdpa.attention(q, k, v, is_causal=True, scale=float(w.scale))
    out.backward(g)
    got = [t.grad.to(torch.float64).cpu().numpy() for t in (q, k, v)]
    _check(got, _ref_and_bound(w, do, grad_f32=False), "autograd")


def test_bwd_unsupported_raise():
    q = torch.zeros(1, 1, 8, 64, device="cuda", dtype=torch.float32)
    with pytest.raises(sdpa.SdpaError):
        sdpa.scaled_dot_product_attention_backward(
            q, q, q, q, torch.zeros(1, 1, 8, device="cuda"), q)

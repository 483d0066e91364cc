"""GPU parity of the backward pass with dropout (sdpa_bwd_dropout) against
the fp64 gradient oracle, through the C ABI.

The bound is the one of tests/test_parity_bwd_gpu.py with the dropped,
rescaled weights W = P z / (1 - p) in place of P wherever they enter (dV,
and the forward's O inside D) and z dP / (1 - p) in place of dP.  The
dK/dV kernel moves the keep bits across lanes; with q = k = 0 and dO the
identity, dV[j, i] = z_ij / ((1 - p) |A_i|) exposes them bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from oracle import dropout as odrop
from oracle import grad as ograd
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu

U = 2.0 ** -11
# rounding of P and dS before the dV, dK, dQ products: f16 for f16 inputs,
# bf16 (relative 2^-8, no subnormal range in play) for bf16 inputs
U_P = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
U_SUBP = {"f16": 2.0 ** -25, "bf16": 0.0}
E_LSE = 1e-4
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -24}
U_GRAD = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _run(w, do, p, seed, offset=0, grad_f32=True):
    q, k, v = (to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    g = to_device(do, w.dtype)
    out_f32 = w.dtype == "bf16"
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, is_causal=w.is_causal, scale=float(w.scale), dropout_p=p, dropout_seed=seed,
        dropout_offset=offset, out_dtype=torch.float32 if out_f32 else None, return_lse=True)
    dq, dk, dv = sdpa.scaled_dot_product_attention_backward(
        q, k, v, out, lse, g, is_causal=w.is_causal, scale=float(w.scale),
        grad_dtype=torch.float32 if grad_f32 else None, dropout_p=p, dropout_seed=seed,
        dropout_offset=offset)
    torch.cuda.synchronize()
    return [t.to(torch.float64).cpu().numpy() for t in (dq, dk, dv)]


def _ref_and_bound(w, do, p, seed, offset=0, grad_f32=True):
    do64 = inputs.storage_to_f64(do, w.dtype)
    ref = ograd.sdpa_bwd_dropout(w.q64, w.k64, w.v64, do64, float(w.scale), w.is_causal, p,
                                 seed, offset)
    o64, _ = odrop.sdpa_fwd_dropout(w.q64, w.k64, w.v64, float(w.scale), w.is_causal, p, seed,
                                    offset)
    sc, uo = float(w.scale), U_OUT[w.dtype]
    rp = 1.0 / (1.0 - float(np.float32(p)))
    bq, bk, bv = (np.zeros_like(r) for r in ref)
    for b in range(w.B):
        for h in range(w.H):
            q, k, v, g = w.q64[b, h], w.k64[b, h], w.v64[b, h], do64[b, h]
            P = ograd._probs(q, k, sc, w.is_causal)
            zr = odrop.keep_mask(w.Nq, w.Nk, b * w.H + h, p, seed, offset) * rp
            W = P * zr
            dp = (g @ v.T) * zr
            dd = np.sum(g * o64[b, h], axis=1, keepdims=True)
            ds_abs = np.abs(P * (dp - dd))
            e_d = np.sum(np.abs(g) * (U * (W @ np.abs(v)) + uo * np.abs(o64[b, h])),
                         axis=1, keepdims=True)
            up, us = U_P[w.dtype], U_SUBP[w.dtype]
            vis = (P > 0).astype(np.float64)
            t = up * ds_abs + us * vis + P * (e_d + E_LSE * np.abs(dp - dd))
            bv[b, h] = ((up + E_LSE) * W + us * vis).T @ np.abs(g)
            bq[b, h] = sc * (t @ np.abs(k))
            bk[b, h] = sc * (t.T @ np.abs(q))
    bounds = []
    for r, bd in zip(ref, (bq, bk, bv)):
        bd = 2.0 * bd
        if not grad_f32:
            bd = bd + U_GRAD[w.dtype] * np.abs(r)
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
def test_bwd_dropout_dense_ragged(dtype, d, causal):
    w = inputs.make_dense(2, 2, 160, 160, d, dtype, "normal", causal, seed=3, cfg=110)
    do = inputs.make_grad_out(w, seed=3, cfg=110)
    got = _run(w, do, 0.2, seed=77 + d, offset=4)
    _check(got, _ref_and_bound(w, do, 0.2, 77 + d, 4), f"{dtype} d{d} causal={causal}")


@pytest.mark.parametrize("p", [0.05, 0.5])
@pytest.mark.parametrize("nq,nk", [(100, 260), (300, 70), (33, 1)])
def test_bwd_dropout_shapes(p, nq, nk):
    w = inputs.make_dense(1, 3, nq, nk, 64, "f16", "normal", True, seed=5, cfg=111)
    do = inputs.make_grad_out(w, seed=5, cfg=111)
    got = _run(w, do, p, seed=9)
    _check(got, _ref_and_bound(w, do, p, 9), f"p={p} nq{nq} nk{nk}")


@pytest.mark.parametrize("causal", [False, True])
def test_transposed_keep_bits_are_exact(causal):
    """q = k = 0 (uniform P), dO = identity: dV[j, i] = z_ij / ((1-p) |A_i|)."""
    n, p, seed, off = 128, 0.35, 0xFEDCBA9876543210, 2
    B, H = 1, 3
    z = torch.zeros(B, H, n, n, dtype=torch.float16, device="cuda")
    eye = torch.eye(n, dtype=torch.float16, device="cuda").expand(B, H, n, n).contiguous()
    v = torch.randn(B, H, n, n, device="cuda").to(torch.float16)
    out, lse = sdpa.scaled_dot_product_attention(z, z, v, is_causal=causal, dropout_p=p,
                                                 dropout_seed=seed, dropout_offset=off,
                                                 return_lse=True)
    dq, dk, dv = sdpa.scaled_dot_product_attention_backward(
        z, z, v, out, lse, eye, is_causal=causal, grad_dtype=torch.float32, dropout_p=p,
        dropout_seed=seed, dropout_offset=off)
    torch.cuda.synchronize()
    dvn = dv.cpu().numpy()
    cnt = np.arange(n) + 1 if causal else np.full(n, n)
    for h in range(H):
        want = odrop.keep_mask(n, n, h, p, seed, off)
        if causal:
            want = want & np.tri(n, dtype=bool)
        assert np.array_equal(dvn[0, h].T > 0, want), f"head {h}"
        kept = np.where(want, 1.0 / ((1.0 - float(np.float32(p))) * cnt[:, None]), 0.0)
        np.testing.assert_allclose(dvn[0, h].T, kept, rtol=2e-3)


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dropout_one_group_grid(d, causal):
    """The small grids above run the dQ and dK/dV dropout kernels with two
    groups of waves; 130 units of two tiles (N = 300) run the one-group
    kernels, checked on the first four units (their keep masks are those of
    units 0..3) against the oracle."""
    B, H, n, p, seed = 1, 130, 300, 0.2, 0x5EED + d
    assert B * H * -(-n // 256) > 256
    w = inputs.make_dense(B, H, n, n, d, "f16", "normal", causal, seed=23 + causal, cfg=114)
    do = inputs.make_grad_out(w, seed=23, cfg=114)
    sub = dataclasses.replace(w, H=4, q=w.q[:, :4].copy(), k=w.k[:, :4].copy(),
                              v=w.v[:, :4].copy())
    got = _run(w, do, p, seed, offset=2)
    _check([g[:, :4] for g in got], _ref_and_bound(sub, do[:, :4].copy(), p, seed, 2),
           f"one group d{d} causal={causal}")


def test_bwd_dropout_deterministic_and_p_zero_is_plain():
    w = inputs.make_dense(2, 2, 200, 200, 64, "bf16", "normal", True, seed=11, cfg=112)
    do = inputs.make_grad_out(w, seed=11, cfg=112)
    a, b = _run(w, do, 0.1, seed=1), _run(w, do, 0.1, seed=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = _run(w, do, 0.1, seed=2)
    assert not np.array_equal(a[0], c[0])
    # p = 0 takes the plain kernels: the same bits as sdpa_bwd
    q, k, v = (to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    g = to_device(do, w.dtype)
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, is_causal=True, scale=float(w.scale),
                                                 out_dtype=torch.float32, return_lse=True)
    plain = sdpa.scaled_dot_product_attention_backward(q, k, v, out, lse, g, is_causal=True,
                                                       scale=float(w.scale))
    zero = sdpa.scaled_dot_product_attention_backward(q, k, v, out, lse, g, is_causal=True,
                                                      scale=float(w.scale), dropout_p=0.0,
                                                      dropout_seed=5)
    torch.cuda.synchronize()
    for x, y in zip(plain, zero):
        assert torch.equal(x, y)


def test_autograd_with_dropout_matches_explicit():
    w = inputs.make_dense(1, 2, 192, 192, 64, "f16", "normal", True, seed=13, cfg=113)
    do = inputs.make_grad_out(w, seed=13, cfg=113)
    q, k, v = (to_device(x, w.dtype).requires_grad_(True) for x in (w.q, w.k, w.v))
    out = sdpa.attention(q, k, v, is_causal=True, scale=float(w.scale), dropout_p=0.25,
                         dropout_seed=31, dropout_offset=7)
    out.backward(to_device(do, w.dtype))
    got = [t.grad.to(torch.float64).cpu().numpy() for t in (q, k, v)]
    _check(got, _ref_and_bound(w, do, 0.25, 31, 7, grad_f32=False), "autograd dropout")


def test_module_training_step_full_size():
    """The tutorial's CausalSelfAttention core in training, forward and
    backward with dropout 0.1 (B32 H8 N1024 d64 f16), checked on sampled
    (batch, head) units by rel-L2 (2e-3: the sums of dQ and dK cancel, so
    the error is measured against smaller results than in the forward)."""
    w = inputs.make_config(3)
    do = inputs.make_grad_out(w, seed=0, cfg=3)
    got = _run(w, do, 0.1, seed=2024)
    rng = np.random.default_rng(1)
    do64 = inputs.storage_to_f64(do, w.dtype)
    q64, k64, v64 = w.q64, w.k64, w.v64
    for u in rng.choice(w.B * w.H, size=3, replace=False):
        b, h = divmod(int(u), w.H)
        ref = ograd.attention_grads_dropout(q64[b, h], k64[b, h], v64[b, h], do64[b, h],
                                            float(w.scale), True, 0.1, 2024, 0, b * w.H + h)
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            err = np.linalg.norm(g[b, h] - r) / np.linalg.norm(r)
            assert err < 2e-3, f"unit {b},{h} {name}: rel-L2 {err:.2e}"

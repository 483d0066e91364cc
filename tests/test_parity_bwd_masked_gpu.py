"""GPU parity of the elementwise-mask backward (sdpa_bwd_masked) against the
fp64 masked gradient oracle (oracle/grad.py: sdpa_bwd_masked), through the C
ABI.  The forward runs on the GPU first with the same mask (its out and lse
feed the backward).  The elementwise bound is the dense backward's (P and
dS rounded to f16, the forward's O inside D_i, the forward's lse error, the
output rounding), with P the masked softmax, allowed twice over.  The f16
rounding of a P or dS value is at most 2^-11 of it or, below f16's smallest
normal (2^-14), half the subnormal spacing, 2^-25: that floor enters for
every visible pair (a masked pair's P is an exact 0).  Masks make such
pairs common enough to matter: a key that only one row sees keeps a tiny P
unaveraged.
"""
import dataclasses
import types

import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from oracle import grad as ograd
from oracle import masked as omask
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu

U = 2.0 ** -11
U_SUB = 2.0 ** -25   # half the f16 subnormal spacing
E_LSE = 1e-4
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -24}   # bf16 runs keep O in f32
# rounding of P and dS before the dV, dK, dQ products: f16 for f16 inputs,
# bf16 (relative 2^-8, no subnormal range in play) for bf16 inputs
U_P = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
U_SUBP = {"f16": 2.0 ** -25, "bf16": 0.0}


def _mask_t(m, kind, mdt):
    return torch.from_numpy(m).cuda().bool() if kind == "bool" else to_device(m, mdt)


def _run(w, do, mt, grad_f32=True):
    q, k, v = (to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    g = to_device(do, w.dtype)
    odt = torch.float32 if w.dtype == "bf16" else None
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, attn_mask=mt, is_causal=w.is_causal,
                                                 scale=float(w.scale), out_dtype=odt,
                                                 return_lse=True)
    dq, dk, dv = sdpa.scaled_dot_product_attention_backward(
        q, k, v, out, lse, g, is_causal=w.is_causal, scale=float(w.scale),
        grad_dtype=torch.float32 if grad_f32 else None, attn_mask=mt)
    torch.cuda.synchronize()
    return [t.double().cpu().numpy() for t in (dq, dk, dv)]


def _check(w, got, do, m4, kind, mdt, grad_f32=True):
    """m4: the mask broadcast to 4-D (bool bytes or stored additive values).
    Gradients stored in f16 add one final rounding (relative 2^-11, or U_SUB
    in the subnormal range)."""
    do64 = inputs.storage_to_f64(do, w.dtype)
    mv = m4 if kind == "bool" else inputs.storage_to_f64(m4, mdt)
    ref = ograd.sdpa_bwd_masked(w.q64, w.k64, w.v64, do64, mv, kind, float(w.scale), w.is_causal)
    sc = float(w.scale)
    for b in range(w.B):
        for h in range(w.H):
            mu = mv[b % mv.shape[0], h % mv.shape[1]]
            bias = omask.bias_of(np.broadcast_to(mu, (w.Nq, w.Nk)), kind)
            q, k, v, g = w.q64[b, h], w.k64[b, h], w.v64[b, h], do64[b, h]
            o, _ = omask.attend_biased(q, k, v, sc, bias, w.is_causal)
            s = sc * (q @ k.T) + bias
            if w.is_causal:
                s = np.where(np.arange(w.Nk)[None, :] <= np.arange(w.Nq)[:, None], s, -np.inf)
            P = np.zeros_like(s)
            live = np.any(s > -np.inf, axis=1)
            e = np.exp(s[live] - np.max(s[live], axis=1, keepdims=True))
            P[live] = e / np.sum(e, axis=1, keepdims=True)
            dp = g @ v.T
            dd = np.sum(g * o, axis=1, keepdims=True)
            e_d = np.sum(np.abs(g) * (U * (P @ np.abs(v)) + U_OUT[w.dtype] * np.abs(o)), axis=1,
                         keepdims=True)
            vis = (s > -np.inf).astype(np.float64)
            up, us = U_P[w.dtype], U_SUBP[w.dtype]
            t = up * np.abs(P * (dp - dd)) + us * vis + P * (e_d + E_LSE * np.abs(dp - dd))
            bounds = (sc * (t @ np.abs(k)), sc * (t.T @ np.abs(q)),
                      ((up + E_LSE) * P + us * vis).T @ np.abs(g))
            for name, gt, r, bd in zip(("dq", "dk", "dv"), got, ref, bounds):
                gu, ru, bu = gt[b, h], r[b, h], 2.0 * bd + 1e-30
                if not grad_f32:
                    bu = bu + U * np.abs(ru) + U_SUB
                assert np.all(np.isfinite(gu)), f"({b},{h}) {name}: non-finite"
                worst = float(np.max(np.abs(gu - ru) / bu))
                assert worst <= 1.0, f"({b},{h}) {name}: error {worst:.3f} x bound"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add", "add_f32"])
def test_bwd_masked_ragged(dtype, d, causal, kind):
    B, H, Nq, Nk = 2, 2, 150, 161
    w = inputs.make_dense(B, H, Nq, Nk, d, dtype, "normal", causal, seed=d, cfg=130)
    do = inputs.make_grad_out(w, seed=d, cfg=130)
    mdt = "f32" if kind == "add_f32" else dtype
    mk = "bool" if kind == "bool" else "add"
    m = inputs.make_attn_mask((B, H, Nq, Nk), mk, keep=0.8, seed=d + causal, cfg=131, dtype=mdt)
    got = _run(w, do, _mask_t(m, mk, mdt))
    _check(w, got, do, m, mk, mdt)


@pytest.mark.parametrize("cfg", [7, 8])
def test_bwd_masked_full_workload_sampled_units(cfg):
    # the masked (additive f16 [32, 8, 1024, 1024]) and padded (key-padding
    # bool [32, 1, 1, 512]) workloads at full size, in the benchmark's launch
    # configuration (f16 gradients); four whole (batch, head) units, the
    # first and the last among them, are checked against the oracle
    w = inputs.make_config(cfg)
    assert w.dtype == "f16"
    do = inputs.make_grad_out(w, seed=cfg, cfg=132)
    kind = w.mask_kind
    got = _run(w, do, _mask_t(w.attn_mask, kind, w.dtype), grad_f32=False)
    units = [(0, 0), (w.B // 3, w.H - 1), (2 * w.B // 3, w.H // 2), (w.B - 1, w.H - 1)]
    bi, hi = [b for b, _ in units], [h for _, h in units]
    f64 = lambda a: inputs.storage_to_f64(a[bi, hi][None], w.dtype)
    sub = types.SimpleNamespace(B=1, H=len(units), Nq=w.Nq, Nk=w.Nk, dtype=w.dtype,
                                scale=w.scale, is_causal=w.is_causal,
                                q64=f64(w.q), k64=f64(w.k), v64=f64(w.v))
    m = w.attn_mask
    msub = m[bi, [h % m.shape[1] for h in hi]][None]
    _check(sub, [g[bi, hi][None] for g in got], do[bi, hi][None], msub, kind, w.dtype,
           grad_f32=False)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add_f32"])
def test_bwd_masked_one_group_grid(d, causal, kind):
    """The small grids above run the masked dQ and dK/dV kernels (dQ only at
    d = 128) with two groups of waves; 130 units of two tiles (N = 300) run
    the one-group ones, checked on four units against the oracle."""
    B, H, n = 1, 130, 300
    assert B * H * -(-n // 256) > 256
    mk = "bool" if kind == "bool" else "add"
    mdt = "f32" if kind == "add_f32" else "f16"
    w = inputs.make_dense(B, H, n, n, d, "f16", "normal", causal, seed=d + causal, cfg=138)
    do = inputs.make_grad_out(w, seed=d, cfg=138)
    m = inputs.make_attn_mask((B, H, n, n), mk, keep=0.85, seed=d + 3 * causal, cfg=139,
                              dtype=mdt)
    got = _run(w, do, _mask_t(m, mk, mdt))
    sub = dataclasses.replace(w, H=4, q=w.q[:, :4].copy(), k=w.k[:, :4].copy(),
                              v=w.v[:, :4].copy())
    _check(sub, [g[:, :4] for g in got], do[:, :4].copy(), m[:, :4].copy(), mk, mdt)


@pytest.mark.parametrize("shape", [(2, 1, 1, 256), (1, 3, 200, 256), (200, 256)])
def test_bwd_masked_broadcast(shape):
    B, H, Nq, Nk, d = 2, 3, 200, 256, 64
    w = inputs.make_dense(B, H, Nq, Nk, d, "f16", "normal", False, seed=2, cfg=132)
    do = inputs.make_grad_out(w, seed=2, cfg=132)
    m = inputs.make_attn_mask(shape, "bool", keep=0.7, seed=len(shape), cfg=133)
    m[..., 0] = 1
    got = _run(w, do, _mask_t(m, "bool", "f16"))
    _check(w, got, do, m.reshape((1,) * (4 - m.ndim) + m.shape), "bool", "f16")


def test_bwd_masked_empty_rows():
    # rows with no visible key: zero gradients, no NaN anywhere
    B, H, N, d = 1, 2, 130, 64
    w = inputs.make_dense(B, H, N, N, d, "f16", "normal", True, seed=5, cfg=134)
    do = inputs.make_grad_out(w, seed=5, cfg=134)
    m = np.ones((B, H, N, N), np.uint8)
    m[:, :, 7] = 0
    m[:, 1, 100:110, :90] = 0
    got = _run(w, do, _mask_t(m, "bool", "f16"))
    assert np.all(got[0][:, :, 7] == 0)
    _check(w, got, do, m, "bool", "f16")


def test_autograd_with_mask_matches_explicit():
    B, H, N, d = 2, 2, 100, 64
    w = inputs.make_dense(B, H, N, N, d, "f16", "normal", False, seed=6, cfg=135)
    do = inputs.make_grad_out(w, seed=6, cfg=135)
    m = inputs.make_attn_mask((B, 1, N, N), "add", keep=0.9, seed=6, cfg=136, dtype="f16")
    mt = _mask_t(m, "add", "f16")
    q, k, v = (to_device(x, "f16").requires_grad_() for x in (w.q, w.k, w.v))
    out = sdpa.attention(q, k, v, scale=float(w.scale), attn_mask=mt)
    out.backward(to_device(do, "f16"))
    torch.cuda.synchronize()
    ref = _run(w, do, mt)
    for t, r in zip((q.grad, k.grad, v.grad), ref):
        np.testing.assert_allclose(t.double().cpu().numpy(), r, rtol=2e-3, atol=2e-3)


def test_all_true_mask_matches_plain_backward():
    B, H, N, d = 1, 2, 200, 64
    w = inputs.make_dense(B, H, N, N, d, "f16", "normal", True, seed=7, cfg=137)
    do = inputs.make_grad_out(w, seed=7, cfg=137)
    q, k, v = (to_device(x, "f16") for x in (w.q, w.k, w.v))
    g = to_device(do, "f16")
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, is_causal=True, return_lse=True)
    plain = sdpa.scaled_dot_product_attention_backward(q, k, v, out, lse, g, is_causal=True,
                                                       grad_dtype=torch.float32)
    ones = torch.ones((N, N), dtype=torch.bool, device="cuda")
    masked = sdpa.scaled_dot_product_attention_backward(q, k, v, out, lse, g, is_causal=True,
                                                        grad_dtype=torch.float32,
                                                        attn_mask=ones)
    torch.cuda.synchronize()
    for a, b in zip(plain, masked):
        np.testing.assert_allclose(a.double().cpu().numpy(), b.double().cpu().numpy(),
                                   rtol=1e-3, atol=1e-3)

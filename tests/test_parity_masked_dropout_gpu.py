"""GPU parity of an elementwise mask together with dropout
(sdpa_fwd_masked_dropout, sdpa_bwd_masked_dropout) against the fp64
oracles of oracle/dropout.py and oracle/grad.py, through the C ABI.

The mask decides which pairs enter the softmax; dropout then keeps each
resulting weight with the Philox contract's draws (which depend only on the
pair's position) and divides kept weights by the keep probability.

* Forward: every head dim, both input types, causal on and off, boolean,
  16-bit and f32 additive masks, at the tolerances of tests/gpu_util.py;
  rows with no finite score give zeros and lse = -inf.
* With q = 0 and V the identity, O_ij = m_ij z_ij / (kappa sum_j m_ij):
  the output exposes every mask and keep decision, compared exactly.
* p = 0 is the masked kernel, bit for bit.
* Backward: the elementwise bound of tests/test_parity_bwd_dropout_gpu.py
  with P the masked softmax.
"""
import dataclasses

import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from oracle import dropout as odrop
from oracle import grad as ograd
from oracle import masked as omask
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

P_DROP, SEED, OFF = 0.2, 0x1234ABCD5678, 6


def _mask(kind, dtype, shape, seed, cfg, keep=0.75):
    """(device tensor, f64 bias-or-bool for the oracle, oracle kind)."""
    if kind == "bool":
        m = inputs.make_attn_mask(shape, "bool", keep=keep, seed=seed, cfg=cfg)
        return torch.from_numpy(m).cuda().bool(), m, "bool"
    mdt = "f32" if kind == "add_f32" else dtype
    m = inputs.make_attn_mask(shape, "add", keep=keep, bias_std=1.0, seed=seed, cfg=cfg, dtype=mdt)
    return G.to_device(m, mdt), inputs.storage_to_f64(m, mdt), "add"


def _fwd(w, mt, p=P_DROP, out_f32=False, q=None, k=None, v=None):
    q, k, v = (G.to_device(x, w.dtype) if t is None else t
               for x, t in ((w.q, q), (w.k, k), (w.v, v)))
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, attn_mask=mt, is_causal=w.is_causal, scale=float(w.scale), dropout_p=p,
        dropout_seed=SEED, dropout_offset=OFF, out_dtype=torch.float32 if out_f32 else None,
        return_lse=True)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add", "add_f32"])
def test_forward(dtype, d, causal, kind):
    B, H, Nq, Nk = 2, 2, 200, 333
    w = inputs.make_dense(B, H, Nq, Nk, d, dtype, "normal", causal, seed=d, cfg=150)
    mt, m64, mk = _mask(kind, dtype, (B, H, Nq, Nk), seed=d, cfg=150)
    out, lse = _fwd(w, mt, out_f32=True)
    ref, lref = odrop.sdpa_fwd_masked_dropout(w.q64, w.k64, w.v64, m64, mk, w.scale, causal,
                                              P_DROP, SEED, OFF)
    o, l = out.double().cpu().numpy(), lse.double().cpu().numpy()
    dead = np.isneginf(lref)
    assert np.array_equal(np.isneginf(l), dead)
    assert np.all(o[dead] == 0.0)
    G.assert_parity(o, ref, dtype, f"{dtype} d{d} causal={causal} {kind}",
                    np.where(dead, 0.0, l), np.where(dead, 0.0, lref))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_forward_one_group_grid(d, causal, kind):
    """The small grids above run the kernels that split each workgroup's
    keys over two wave groups; 130 units of two query tiles (N = 300) run
    the one-group ones, checked on the first four units (their keep
    decisions are those of units 0..3)."""
    B, H, n = 1, 130, 300
    assert B * H * -(-n // 256) > 256
    w = inputs.make_dense(B, H, n, n, d, "f16", "normal", causal, seed=d + causal, cfg=155)
    mt, m64, mk = _mask(kind, "f16", (B, H, n, n), seed=d, cfg=155, keep=0.85)
    out, lse = _fwd(w, mt, out_f32=True)
    sl = lambda x: x[:, :4]
    ref, lref = odrop.sdpa_fwd_masked_dropout(sl(w.q64), sl(w.k64), sl(w.v64), sl(m64), mk,
                                              w.scale, causal, P_DROP, SEED, OFF)
    o, l = sl(out.double().cpu().numpy()), sl(lse.double().cpu().numpy())
    dead = np.isneginf(lref)
    assert np.array_equal(np.isneginf(l), dead)
    assert np.all(o[dead] == 0.0)
    G.assert_parity(o, ref, "f16", f"one group d{d} causal={causal} {kind}",
                    np.where(dead, 0.0, l), np.where(dead, 0.0, lref))


@pytest.mark.parametrize("causal", [False, True])
def test_mask_and_keep_decisions_are_exact(causal):
    """q = 0, V = identity, a boolean mask: O_ij = m_ij z_ij / (kappa |A_i|)."""
    B, H, n = 1, 2, 128
    m = inputs.make_attn_mask((B, H, n, n), "bool", keep=0.6, seed=3, cfg=151)
    m[..., 0] = 1   # every row keeps a key
    q = torch.zeros(B, H, n, n, dtype=torch.float16, device="cuda")
    v = torch.eye(n, dtype=torch.float16, device="cuda").expand(B, H, n, n).contiguous()
    out = sdpa.scaled_dot_product_attention(
        q, q, v, attn_mask=torch.from_numpy(m).cuda().bool(), is_causal=causal,
        dropout_p=0.3, dropout_seed=SEED, dropout_offset=OFF, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    kappa = odrop.keep_probability(0.3)
    for h in range(H):
        vis = m[0, h].astype(bool)
        if causal:
            vis &= np.tri(n, dtype=bool)
        z = odrop.keep_mask(n, n, h, 0.3, SEED, OFF)
        assert np.array_equal(o[0, h] > 0, vis & z), f"head {h}"
        want = np.where(vis & z, 1.0 / (kappa * vis.sum(1, keepdims=True)), 0.0)
        np.testing.assert_allclose(o[0, h], want, rtol=2e-3)


def test_no_dropout_is_the_masked_kernel():
    w = inputs.make_dense(2, 2, 150, 260, 64, "f16", "normal", True, seed=4, cfg=152)
    mt, _, _ = _mask("add", "f16", (2, 2, 150, 260), seed=4, cfg=152)
    a, la = _fwd(w, mt, p=0.0)
    b, lb = sdpa.scaled_dot_product_attention(
        G.to_device(w.q, "f16"), G.to_device(w.k, "f16"), G.to_device(w.v, "f16"), attn_mask=mt,
        is_causal=True, scale=float(w.scale), return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


# ---- backward: the bound of tests/test_parity_bwd_dropout_gpu.py, P masked
U = 2.0 ** -11
U_P = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
U_SUBP = {"f16": 2.0 ** -25, "bf16": 0.0}
E_LSE = 1e-4
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -24}


def _bwd_check(w, do, mt, m64, mk, what, first_heads=None):
    """With first_heads = n (B = 1), the GPU runs every unit and the oracle
    checks units 0..n-1 (whose keep decisions are those of units 0..n-1 of a
    workload of n heads)."""
    q, k, v = (G.to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    g = G.to_device(do, w.dtype)
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, attn_mask=mt, is_causal=w.is_causal, scale=float(w.scale), dropout_p=P_DROP,
        dropout_seed=SEED, dropout_offset=OFF,
        out_dtype=torch.float32 if w.dtype == "bf16" else None, return_lse=True)
    got = sdpa.scaled_dot_product_attention_backward(
        q, k, v, out, lse, g, is_causal=w.is_causal, scale=float(w.scale),
        grad_dtype=torch.float32, dropout_p=P_DROP, dropout_seed=SEED, dropout_offset=OFF,
        attn_mask=mt)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in got]
    if first_heads is not None:
        n = first_heads
        got = [t[:, :n] for t in got]
        do, m64 = do[:, :n], m64[:, :n]
        w = dataclasses.replace(w, H=n, q=w.q[:, :n].copy(), k=w.k[:, :n].copy(),
                                v=w.v[:, :n].copy())
    do64 = inputs.storage_to_f64(do, w.dtype)
    sc = float(w.scale)
    ref = ograd.sdpa_bwd_masked_dropout(w.q64, w.k64, w.v64, do64, m64, mk, sc, w.is_causal,
                                        P_DROP, SEED, OFF)
    o64, _ = odrop.sdpa_fwd_masked_dropout(w.q64, w.k64, w.v64, m64, mk, sc, w.is_causal, P_DROP,
                                           SEED, OFF)
    rp = 1.0 / odrop.keep_probability(P_DROP)
    bounds = [np.zeros_like(r) for r in ref]
    for b in range(w.B):
        for h in range(w.H):
            mu = np.broadcast_to(m64[b % m64.shape[0], h % m64.shape[1]], (w.Nq, w.Nk))
            bias = omask.bias_of(mu, mk)
            qq, kk, vv, gg = w.q64[b, h], w.k64[b, h], w.v64[b, h], do64[b, h]
            s = sc * (qq @ kk.T) + bias
            if w.is_causal:
                s = np.where(np.arange(w.Nk)[None, :] <= np.arange(w.Nq)[:, None], s, -np.inf)
            P = np.zeros_like(s)
            live = np.any(s > -np.inf, axis=1)
            e = np.exp(s[live] - np.max(s[live], axis=1, keepdims=True))
            P[live] = e / np.sum(e, axis=1, keepdims=True)
            zr = odrop.keep_mask(w.Nq, w.Nk, b * w.H + h, P_DROP, SEED, OFF) * rp
            W = P * zr
            dp = (gg @ vv.T) * zr
            dd = np.sum(gg * o64[b, h], axis=1, keepdims=True)
            e_d = np.sum(np.abs(gg) * (U * (W @ np.abs(vv)) + U_OUT[w.dtype] * np.abs(o64[b, h])),
                         axis=1, keepdims=True)
            up, us = U_P[w.dtype], U_SUBP[w.dtype]
            vis = (P > 0).astype(np.float64)
            t = up * np.abs(P * (dp - dd)) + us * vis + P * (e_d + E_LSE * np.abs(dp - dd))
            bounds[2][b, h] = ((up + E_LSE) * W + us * vis).T @ np.abs(gg)
            bounds[0][b, h] = sc * (t @ np.abs(kk))
            bounds[1][b, h] = sc * (t.T @ np.abs(qq))
    for name, gv, r, bd in zip(("dq", "dk", "dv"), got, ref, bounds):
        assert np.all(np.isfinite(gv)), f"{what} {name}: non-finite"
        ratio = np.abs(gv - r) / (2.0 * bd + 1e-30)
        assert float(np.max(ratio)) <= 1.0, f"{what} {name}: {float(np.max(ratio)):.3f} x bound"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_backward(dtype, d, causal, kind):
    B, H, Nq, Nk = 1, 2, 160, 200
    w = inputs.make_dense(B, H, Nq, Nk, d, dtype, "normal", causal, seed=d, cfg=153)
    do = inputs.make_grad_out(w, seed=d, cfg=153)
    mt, m64, mk = _mask(kind, dtype, (B, H, Nq, Nk), seed=d, cfg=153)
    _bwd_check(w, do, mt, m64, mk, f"{dtype} d{d} causal={causal} {kind}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_backward_one_group_grid(d, causal, kind):
    """The small grids above run the backward kernels split over two groups
    of waves (dQ only at d = 128); 130 units of two tiles (N = 300) run the
    one-group ones, checked on the first four units."""
    B, H, n = 1, 130, 300
    assert B * H * -(-n // 256) > 256
    w = inputs.make_dense(B, H, n, n, d, "f16", "normal", causal, seed=d + causal, cfg=156)
    do = inputs.make_grad_out(w, seed=d, cfg=156)
    mt, m64, mk = _mask(kind, "f16", (B, H, n, n), seed=d, cfg=156, keep=0.85)
    _bwd_check(w, do, mt, m64, mk, f"one group d{d} causal={causal} {kind}", first_heads=4)


def test_backward_f32_mask_and_autograd():
    w = inputs.make_dense(1, 2, 130, 170, 64, "f16", "normal", False, seed=9, cfg=154)
    do = inputs.make_grad_out(w, seed=9, cfg=154)
    mt, m64, mk = _mask("add_f32", "f16", (1, 2, 130, 170), seed=9, cfg=154)
    _bwd_check(w, do, mt, m64, mk, "f32 mask")
    # the differentiable wrapper runs the same two entry points
    q, k, v = (G.to_device(x, "f16").requires_grad_() for x in (w.q, w.k, w.v))
    out = sdpa.attention(q, k, v, scale=float(w.scale), dropout_p=P_DROP, dropout_seed=SEED,
                         dropout_offset=OFF, attn_mask=mt)
    out.backward(G.to_device(do, "f16"))
    ref = sdpa.scaled_dot_product_attention_backward(
        q.detach(), k.detach(), v.detach(), out.detach(),
        sdpa.scaled_dot_product_attention(q.detach(), k.detach(), v.detach(), attn_mask=mt,
                                          scale=float(w.scale), dropout_p=P_DROP,
                                          dropout_seed=SEED, dropout_offset=OFF,
                                          return_lse=True)[1],
        G.to_device(do, "f16"), scale=float(w.scale), dropout_p=P_DROP, dropout_seed=SEED,
        dropout_offset=OFF, attn_mask=mt)
    torch.cuda.synchronize()
    for a, b in zip((q.grad, k.grad, v.grad), ref):
        assert torch.equal(a, b)

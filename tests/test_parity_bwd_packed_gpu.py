"""GPU parity of the packed-batch backward (sdpa_bwd_packed) against the fp64
gradient oracle, through the C ABI.

Each (sequence, head) unit of a packed batch is an independent attention
problem (the tutorial's NestedTensor batches, "NestedTensor and dense tensor
support"), so the oracle is the dense gradient oracle applied to each unit,
with the dropout unit index s*H + h of the packed forward.  The elementwise
error bound is the one derived for the dense backward (P and dS rounded to
f16, the forward's O inside D_i = <dO_i, O_i>, the forward's lse error, the
output rounding), allowed twice over for fp32 accumulation and exp2.
"""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from oracle import dropout as odrop
from oracle import grad as ograd
from oracle import sdpa as ofwd
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu

U = 2.0 ** -11
# rounding of P and dS before the dV, dK, dQ products: f16 for f16 inputs,
# bf16 (relative 2^-8, no subnormal range in play) for bf16 inputs
U_P = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
U_SUBP = {"f16": 2.0 ** -25, "bf16": 0.0}
E_LSE = 1e-4
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -24}   # bf16 runs keep O in f32


def _run(w, do, p=0.0, seed=0, offset=0):
    q, k, v = (to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    g = to_device(do, w.dtype)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    odt = torch.float32 if w.dtype == "bf16" else None
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, is_causal=w.is_causal, scale=float(w.scale), cu_seqlens=cu, max_seqlen=w.Nq,
        out_dtype=odt, return_lse=True, dropout_p=p, dropout_seed=seed, dropout_offset=offset)
    dq, dk, dv = sdpa.scaled_dot_product_attention_backward(
        q, k, v, out, lse, g, is_causal=w.is_causal, scale=float(w.scale),
        grad_dtype=torch.float32, dropout_p=p, dropout_seed=seed, dropout_offset=offset,
        cu_seqlens=cu, max_seqlen=w.Nq)
    torch.cuda.synchronize()
    return [t.to(torch.float64).cpu().numpy() for t in (dq, dk, dv)]


def _unit_ref_and_bound(q, k, v, g, scale, causal, dtype, p, seed, offset, unit):
    """Oracle gradients of one unit and their elementwise bound."""
    if p > 0.0:
        ref = ograd.attention_grads_dropout(q, k, v, g, scale, causal, p, seed, offset, unit)
        o, _ = odrop.attend_dropout(q, k, v, scale, causal, p, seed, offset, unit)
        zr = odrop.keep_mask(q.shape[0], k.shape[0], unit, p, seed, offset) / (
            1.0 - float(np.float32(p)))
    else:
        ref = ograd.attention_grads(q, k, v, g, scale, causal)
        o, _ = ofwd.sdpa_fwd(q[None, None], k[None, None], v[None, None], scale, causal)
        o = o[0, 0]
        zr = 1.0
    P = ograd._probs(q, k, scale, causal)
    W = P * zr
    dp = (g @ v.T) * zr
    dd = np.sum(g * o, axis=1, keepdims=True)
    e_d = np.sum(np.abs(g) * (U * (W @ np.abs(v)) + U_OUT[dtype] * np.abs(o)), axis=1,
                 keepdims=True)
    up, us = U_P[dtype], U_SUBP[dtype]
    vis = (P > 0).astype(np.float64)
    t = up * np.abs(P * (dp - dd)) + us * vis + P * (e_d + E_LSE * np.abs(dp - dd))
    bounds = (scale * (t @ np.abs(k)), scale * (t.T @ np.abs(q)),
              ((up + E_LSE) * W + us * vis).T @ np.abs(g))
    return ref, [2.0 * b + 1e-30 for b in bounds]


def _check(w, got, do, p=0.0, seed=0, offset=0, seqs=None):
    do64 = inputs.storage_to_f64(do, w.dtype)
    q64, k64, v64 = w.q64, w.k64, w.v64
    cu = w.cu_seqlens
    for s in (range(len(cu) - 1) if seqs is None else seqs):
        s0, s1 = int(cu[s]), int(cu[s + 1])
        if s1 == s0:
            continue
        for h in range(w.H):
            ref, bounds = _unit_ref_and_bound(q64[s0:s1, h], k64[s0:s1, h], v64[s0:s1, h],
                                              do64[s0:s1, h], float(w.scale), w.is_causal,
                                              w.dtype, p, seed, offset, s * w.H + h)
            for name, gt, r, bd in zip(("dq", "dk", "dv"), got, ref, bounds):
                gu = gt[s0:s1, h]
                assert np.all(np.isfinite(gu)), f"seq {s} head {h} {name}: non-finite"
                worst = float(np.max(np.abs(gu - r) / bd))
                assert worst <= 1.0, f"seq {s} head {h} {name}: error {worst:.3f} x bound"


LENS = np.array([37, 128, 1, 200, 0, 64, 129])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_packed_ragged(dtype, d, causal):
    w = inputs.make_varlen(LENS, 2, d, dtype, "normal", causal, seed=d, cfg=120)
    do = inputs.make_grad_out(w, seed=d, cfg=120)
    _check(w, _run(w, do), do)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_packed_dropout(causal):
    w = inputs.make_varlen(LENS, 3, 64, "f16", "normal", causal, seed=4, cfg=121)
    do = inputs.make_grad_out(w, seed=4, cfg=121)
    p, seed, off = 0.2, 0x1234567890ABCDEF, 3
    _check(w, _run(w, do, p, seed, off), do, p, seed, off)


def test_bwd_packed_matches_dense_per_sequence():
    # one sequence of a packed batch gives the dense backward's gradients bit
    # for bit: the same tiles, the same arithmetic
    lens = np.array([150, 96])
    w = inputs.make_varlen(lens, 2, 64, "f16", "normal", True, seed=6, cfg=122)
    do = inputs.make_grad_out(w, seed=6, cfg=122)
    got = _run(w, do)
    s0, s1 = 0, 150
    q, k, v, g = (to_device(np.ascontiguousarray(x[s0:s1].transpose(1, 0, 2))[None], "f16")
                  for x in (w.q, w.k, w.v, do))
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, is_causal=True, scale=float(w.scale),
                                                 return_lse=True)
    dq, dk, dv = sdpa.scaled_dot_product_attention_backward(
        q, k, v, out, lse, g, is_causal=True, scale=float(w.scale), grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in zip(got, (dq, dk, dv)):
        dense = b[0].double().cpu().numpy().transpose(1, 0, 2)
        assert np.array_equal(a[s0:s1], dense)


def test_autograd_packed_matches_explicit():
    w = inputs.make_varlen(LENS, 2, 64, "f16", "normal", True, seed=8, cfg=123)
    do = inputs.make_grad_out(w, seed=8, cfg=123)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    q, k, v = (to_device(x, "f16").requires_grad_() for x in (w.q, w.k, w.v))
    out = sdpa.attention(q, k, v, is_causal=True, scale=float(w.scale), cu_seqlens=cu,
                         max_seqlen=w.Nq)
    out.backward(to_device(do, "f16"))
    torch.cuda.synchronize()
    ref = _run(w, do)
    for t, r in zip((q.grad, k.grad, v.grad), ref):
        # the autograd path keeps the input dtype for the gradients
        np.testing.assert_allclose(t.double().cpu().numpy(), r, rtol=2e-3, atol=2e-3)


def test_bwd_packed_nested_workload_sampled():
    # the NestedTensor workload at full size (32 sequences, max 512, H8 d64),
    # sampled sequences against the oracle (its longest one included)
    w = inputs.make_config(4)
    do = inputs.make_grad_out(w, seed=0, cfg=4)
    got = _run(w, do)
    lens = np.diff(w.cu_seqlens)
    seqs = sorted({int(np.argmax(lens)), 0, len(lens) - 1, 7})
    _check(w, got, do, seqs=seqs)

"""fp64 CPU oracle for the gradients of exact attention (the backward pass).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares
no code with the GPU path and imports nothing from it.

What it computes:

* The FlashAttention article (method paragraph) names two techniques: tiling
  the forward pass, and recomputing attention in the backward pass instead
  of keeping the N x N matrix.  The pages print no backward formulas.  What a
  backward pass computes is fixed by calculus: for an upstream gradient dO
  of the forward output O (oracle/sdpa.py), the gradients of
  L = sum(dO * O) with respect to q, k and v.  The logsumexp output is an
  auxiliary statistic and is not differentiated.
* Written out by the chain rule, per (batch, head) unit, with
  S = scale * q k^T (masked entries excluded) and P = softmax_rows(S):
      dV    = P^T dO
      dP    = dO V^T
      dS_ij = P_ij * (dP_ij - sum_j' P_ij' dP_ij')     (Jacobian of softmax)
      dQ    = scale * dS K
      dK    = scale * dS^T Q
  Masked entries have P = 0 and so contribute nothing.

Inputs are upcast to float64 exactly; numpy matmul is the only library
primitive used.  The row-maximum shift inside the softmax only guards
against overflow.
"""
from __future__ import annotations

import numpy as np


def _probs(q, k, scale, is_causal):
    """P = softmax_rows(scale * q k^T), keys j > i excluded when causal."""
    s = float(scale) * (q @ k.T)
    if is_causal:
        allowed = np.arange(k.shape[0])[None, :] <= np.arange(q.shape[0])[:, None]
        s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)  # overflow guard only
    e = np.exp(s - m)
    return e / np.sum(e, axis=1, keepdims=True)


def attention_grads(q, k, v, do, scale, is_causal=False):
    """One unit: q [nq,d], k/v [nk,d], do [nq,dv] -> (dq, dk, dv) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    p = _probs(q, k, scale, is_causal)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def sdpa_bwd(q, k, v, do, scale, is_causal=False):
    """Dense: q/do [B,H,Nq,d], k/v [B,H,Nk,d] -> dq, dk, dv (float64)."""
    q = np.asarray(q)
    B, H, Nq, _ = q.shape
    if Nq == 0 or k.shape[2] == 0:
        raise ValueError("empty query or key set")
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = attention_grads(q[b, h], k[b, h], v[b, h], do[b, h],
                                                           scale, is_causal)
    return dq, dk, dv


def attention_grads_dropout(q, k, v, do, scale, is_causal, p, seed, offset, unit):
    """Gradients of L = sum(dO * O) for the dropout forward of
    oracle/dropout.py, whose mask z (fixed by seed, offset and the unit
    index) is a constant: O = (P * z / kappa) V, kappa the keep probability
    T / 65536 of that module.  By the chain rule, with W = P * z / kappa:
        dV    = W^T dO
        dW    = dO V^T,  dP = dW * z / kappa
        dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
        dQ    = scale dS K,  dK = scale dS^T Q
    (sum_j' P_ij' dP_ij' = <dO_i, O_i>, as without dropout.)"""
    from .dropout import keep_mask, keep_probability
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    P = _probs(q, k, scale, is_causal)
    zr = keep_mask(q.shape[0], k.shape[0], unit, p, seed, offset) / keep_probability(p)
    dv = (P * zr).T @ do
    dp = (do @ v.T) * zr
    ds = P * (dp - np.sum(P * dp, axis=1, keepdims=True))
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv


def sdpa_bwd_dropout(q, k, v, do, scale, is_causal, p, seed, offset=0):
    """Dense layouts, unit u = b*H + h (as the dropout forward)."""
    q = np.asarray(q)
    B, H = q.shape[:2]
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(np.shape(k), dtype=np.float64)
    dv = np.empty(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = attention_grads_dropout(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, is_causal, p, seed, offset, b * H + h)
    return dq, dk, dv


def attention_grads_biased(q, k, v, do, scale, bias, is_causal=False):
    """Gradients of L = sum(dO * O) for attention with an elementwise
    additive bias (oracle/masked.py: s = scale q k^T + bias, bias -inf for
    pairs a boolean mask drops).  The bias is a constant, so the chain rule
    is that of the plain case with P = softmax_rows(s):
        dV = P^T dO,  dP = dO V^T,  dS = P (dP - rowsum(P dP)),
        dQ = scale dS K,  dK = scale dS^T Q.
    Rows with no finite score have P = 0 and contribute nothing (their
    output is the constant 0).  The bias itself is not differentiated."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    s = float(scale) * (q @ k.T) + np.asarray(bias, dtype=np.float64)
    nq, nk = s.shape
    if is_causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    P = np.zeros_like(s)
    live = np.any(s > -np.inf, axis=1)
    if np.any(live):
        sl = s[live]
        e = np.exp(sl - np.max(sl, axis=1, keepdims=True))  # overflow guard only
        P[live] = e / np.sum(e, axis=1, keepdims=True)
    dv = P.T @ do
    dp = do @ v.T
    ds = P * (dp - np.sum(P * dp, axis=1, keepdims=True))
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv


def sdpa_bwd_masked(q, k, v, do, mask, kind, scale, is_causal=False):
    """Dense q/do [B,H,Nq,d], k/v [B,H,Nk,d]; mask [Bm,Hm,Nq,Nk] (Bm in
    {1, B}, Hm in {1, H}), kind "bool" (nonzero = attend) or "add"."""
    q = np.asarray(q)
    B, H = q.shape[:2]
    m = np.asarray(mask)
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(np.shape(k), dtype=np.float64)
    dv = np.empty(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            mu = m[b % m.shape[0], h % m.shape[1]]
            bias = np.where(mu != 0, 0.0, -np.inf) if kind == "bool" else mu.astype(np.float64)
            dq[b, h], dk[b, h], dv[b, h] = attention_grads_biased(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, bias, is_causal)
    return dq, dk, dv


def attention_grads_masked_dropout(q, k, v, do, scale, bias, is_causal, p, seed, offset, unit):
    """Gradients of L = sum(dO * O) for the masked forward with dropout of
    oracle/dropout.py (attend_masked_dropout): P the softmax of the biased,
    causally masked scores, z the unit's keep mask, kappa the keep
    probability.  Both the bias and z are constants, so with W = P z / kappa:
        dV = W^T dO,  dP = (dO V^T) z / kappa,
        dS = P (dP - rowsum(P dP)),  dQ = scale dS K,  dK = scale dS^T Q.
    Rows with no finite score have P = 0 and contribute nothing."""
    from .dropout import keep_mask, keep_probability
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    s = float(scale) * (q @ k.T) + np.asarray(bias, dtype=np.float64)
    nq, nk = s.shape
    if is_causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    P = np.zeros_like(s)
    live = np.any(s > -np.inf, axis=1)
    if np.any(live):
        sl = s[live]
        e = np.exp(sl - np.max(sl, axis=1, keepdims=True))  # overflow guard only
        P[live] = e / np.sum(e, axis=1, keepdims=True)
    zr = keep_mask(nq, nk, unit, p, seed, offset) / keep_probability(p)
    dv = (P * zr).T @ do
    dp = (do @ v.T) * zr
    ds = P * (dp - np.sum(P * dp, axis=1, keepdims=True))
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv


def sdpa_bwd_masked_dropout(q, k, v, do, mask, kind, scale, is_causal, p, seed, offset=0):
    """Dense layouts; mask as sdpa_bwd_masked; unit u = b*H + h (as the
    forward)."""
    q = np.asarray(q)
    B, H = q.shape[:2]
    m = np.asarray(mask)
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(np.shape(k), dtype=np.float64)
    dv = np.empty(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            mu = m[b % m.shape[0], h % m.shape[1]]
            bias = np.where(mu != 0, 0.0, -np.inf) if kind == "bool" else mu.astype(np.float64)
            dq[b, h], dk[b, h], dv[b, h] = attention_grads_masked_dropout(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, bias, is_causal, p, seed, offset,
                b * H + h)
    return dq, dk, dv

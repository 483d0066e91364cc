"""fp64 CPU oracle for attention with an elementwise attention mask.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares
no code with the GPU path and imports nothing from it.

What it computes.  The SDPA tutorial's functional call takes an
``attn_mask`` argument (its CausalSelfAttention passes None); the pages do
not define it.  The reading taken, the functional API's convention: a
boolean mask says which (query, key) pairs take part (True = attend); an
additive mask is added to the scaled scores before the softmax:

    s_ij = scale <q_i, k_j> + a_ij          (a_ij = 0 or -inf for a boolean mask)
    O_i  = sum_j softmax_j(s_i.) v_j,  lse_i = ln sum_j exp(s_ij)

over the keys the causal rule leaves (j <= i when causal).  A row whose
every score is -inf has O = 0 and lse = -inf (as block-sparse rows that see
no key).  Masks broadcast over batch and heads as given: a_ij of unit
(b, h) is mask[b % Bm, h % Hm] for a [Bm, Hm, Nq, Nk] mask.
"""
from __future__ import annotations

import numpy as np


def attend_biased(q, k, v, scale, bias, is_causal=False):
    """One unit with an explicit [nq, nk] additive bias (may hold -inf)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = float(scale) * (q @ k.T) + np.asarray(bias, dtype=np.float64)
    nq, nk = s.shape
    if is_causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    live = np.any(s > -np.inf, axis=1)
    out = np.zeros((nq, v.shape[1]))
    lse = np.full(nq, -np.inf)
    if np.any(live):
        sl = s[live]
        m = np.max(sl, axis=1, keepdims=True)   # overflow guard only
        e = np.exp(sl - m)
        l = np.sum(e, axis=1, keepdims=True)
        out[live] = (e @ v) / l
        lse[live] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def bias_of(mask, kind):
    """The additive bias of a mask: 'bool' -> 0 / -inf, 'add' -> the values."""
    mask = np.asarray(mask)
    if kind == "bool":
        return np.where(mask != 0, 0.0, -np.inf)
    return mask.astype(np.float64)


def sdpa_fwd_masked(q, k, v, mask, kind, scale, is_causal=False):
    """Dense q [B,H,Nq,d], k/v [B,H,Nk,d]; mask [Bm,Hm,Nq,Nk] with Bm in
    {1, B} and Hm in {1, H} -> O, lse in float64."""
    B, H, Nq, _ = np.shape(q)
    m = np.asarray(mask)
    O = np.empty((B, H, Nq, np.shape(v)[3]))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            bias = bias_of(m[b % m.shape[0], h % m.shape[1]], kind)
            O[b, h], L[b, h] = attend_biased(q[b, h], k[b, h], v[b, h], scale, bias, is_causal)
    return O, L

"""fp64 CPU oracle for block-sparse exact attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares
no code with the GPU path and imports nothing from it.

What it computes: the FlashAttention article (results paragraph) benchmarks
a block-sparse FlashAttention next to the dense one but gives no mask
format.  The reading taken here: exact attention in which query i may attend
key j only if the block mask entry (i // block, j // block) is nonzero (and
j <= i when causal); within the allowed set it is the plain definition of
oracle/sdpa.py.  A row that sees no key has O = 0 and lse = -inf.

The mask is [Hm, ceil(Nq/block), ceil(Nk/block)] with Hm = 1 (shared by all
heads) or Hm = H.  Inputs are upcast to float64; numpy matmul is the only
library primitive used.
"""
from __future__ import annotations

import numpy as np


def attend_masked(q, k, v, scale, allowed):
    """One unit with an explicit [nq, nk] boolean visibility matrix."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = np.where(allowed, float(scale) * (q @ k.T), -np.inf)
    any_key = np.any(allowed, axis=1)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.full(q.shape[0], -np.inf, dtype=np.float64)
    if np.any(any_key):
        s = s[any_key]
        m = np.max(s, axis=1, keepdims=True)  # overflow guard only
        e = np.exp(s - m)
        l = np.sum(e, axis=1, keepdims=True)
        out[any_key] = (e @ v) / l
        lse[any_key] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def visibility(nq, nk, mask2d, block, is_causal, rows=None):
    """[nq, nk] boolean: mask entry of (i // block, j // block), and j <= i
    when causal.  With ``rows``, only those query rows ([len(rows), nk])."""
    i = (np.arange(nq) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(nk)[None, :]
    vis = np.asarray(mask2d)[i // block, j // block] != 0
    if is_causal:
        vis = vis & (j <= i)
    return vis


def sdpa_fwd_block_sparse(q, k, v, block_mask, scale, is_causal=False, block=128):
    """Dense layouts q [B,H,Nq,d], k/v [B,H,Nk,d]; block_mask
    [Hm, ceil(Nq/block), ceil(Nk/block)].  Returns O [B,H,Nq,d] and lse
    [B,H,Nq] in float64."""
    q = np.asarray(q)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    bm = np.asarray(block_mask)
    if bm.ndim != 3 or bm.shape[0] not in (1, H) or bm.shape[1] * block < Nq or \
            bm.shape[2] * block < Nk:
        raise ValueError("block mask shape")
    O = np.empty((B, H, Nq, v.shape[3]), dtype=np.float64)
    L = np.empty((B, H, Nq), dtype=np.float64)
    for h in range(H):
        vis = visibility(Nq, Nk, bm[h if bm.shape[0] == H else 0], block, is_causal)
        for b in range(B):
            O[b, h], L[b, h] = attend_masked(q[b, h], k[b, h], v[b, h], scale, vis)
    return O, L

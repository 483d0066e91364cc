"""fp64 CPU oracle for attention with dropout on the attention weights.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares
no code with the GPU path and imports nothing from it.

What it computes.  The SDPA tutorial's CausalSelfAttention ("Causal
self-attention" section) passes its dropout rate to the functional call in
training.  Dropout on the attention weights: with P the softmax of the
visible scores (as in oracle/sdpa.py), each weight is kept with probability
1 - p and kept weights are divided by the keep probability (inverted
dropout, so that the expected output is the undropped one):

    O_i   = sum_j P_ij z_ij / kappa v_j,   z_ij in {0, 1}
    lse_i = the logsumexp of the (undropped) visible scores

The pages fix no random-number contract; this is the one taken (the GPU
kernel implements it independently):

    generator  Philox4x32-10 (oracle/philox.py)
    key        (seed mod 2^32, seed >> 32)
    counter    (n(j), i, u, offset), u = b*H + h (dense) or s*H + h (packed,
               i counted from the sequence start)
    n(j)       2*(j >> 4) + ((j >> 2) & 1)       which call
    e(j)       4*((j >> 3) & 1) + (j & 3)        which 16-bit half of its
               output: word e >> 1, bits 16*(e & 1) .. +15
    keep       r < T with r that 16-bit number and
               T = floor((1 - p) * 65536 + 1/2), p taken as a float32

so each call decides 8 keys of one query row, and (n, e) runs over every
key exactly once.  The keep probability is kappa = T / 65536, within 2^-17
of 1 - p, and kept weights are divided by that kappa (reading: the scale is
the inverse of the keep probability actually drawn, which leaves the
expected output unbiased).  A p that rounds T to 0 would keep nothing; it
is outside the contract.
"""
from __future__ import annotations

import numpy as np

from .philox import philox4


def keep_threshold(p) -> int:
    return int(np.floor((1.0 - float(np.float32(p))) * 65536.0 + 0.5))


def keep_probability(p) -> float:
    """kappa = T / 65536, the probability that a weight is kept."""
    return keep_threshold(p) / 65536.0


def draw16(nq, nk, unit, seed, offset, row0=0):
    """The 16-bit number r of every (query row, key) of one unit: [nq, nk]
    uint32 (query rows row0 .. row0 + nq - 1)."""
    seed = int(seed)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    n_calls = 2 * ((nk + 15) // 16)
    i = np.arange(row0, row0 + nq, dtype=np.uint64)[:, None]
    n = np.arange(n_calls, dtype=np.uint64)[None, :]
    out = philox4((n, i, np.uint64(unit), np.uint64(offset)), key, 32, 10)
    words = np.stack([np.broadcast_to(w, (nq, n_calls)) for w in out])   # [4, nq, calls]
    j = np.arange(nk)
    nj = 2 * (j >> 4) + ((j >> 2) & 1)
    ej = 4 * ((j >> 3) & 1) + (j & 3)
    w = words[ej >> 1, :, nj].T                                            # [nq, nk]
    return ((w >> (16 * (ej & 1)).astype(np.uint64)) & np.uint64(0xFFFF)).astype(np.uint32)


def keep_mask(nq, nk, unit, p, seed, offset, row0=0):
    """z of one unit, [nq, nk] bool."""
    return draw16(nq, nk, unit, seed, offset, row0) < keep_threshold(p)


def attend_dropout(q, k, v, scale, is_causal, p, seed, offset, unit):
    """One unit: q [nq, d], k/v [nk, d] -> O [nq, d], lse [nq] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    s = float(scale) * (q @ k.T)
    if is_causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)    # overflow guard only
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    P = e / l
    z = keep_mask(nq, nk, unit, p, seed, offset)
    O = ((P * z) / keep_probability(p)) @ v
    return O, m[:, 0] + np.log(l[:, 0])


def sdpa_fwd_dropout(q, k, v, scale, is_causal, p, seed, offset=0):
    """Dense q [B,H,Nq,d], k/v [B,H,Nk,d] -> O, lse in float64."""
    B, H, Nq, _ = np.shape(q)
    O = np.empty((B, H, Nq, np.shape(v)[3]))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = attend_dropout(q[b, h], k[b, h], v[b, h], scale, is_causal, p,
                                              seed, offset, b * H + h)
    return O, L


def sdpa_fwd_dropout_varlen(q, k, v, cu_seqlens, scale, is_causal, p, seed, offset=0):
    """Packed q/k/v [T,H,d] with sequences at cu_seqlens -> O [T,H,d], lse [T,H]."""
    T, H, _ = np.shape(q)
    O = np.zeros((T, H, np.shape(v)[2]))
    L = np.zeros((T, H))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(H):
            O[a:b, h], L[a:b, h] = attend_dropout(q[a:b, h], k[a:b, h], v[a:b, h], scale,
                                                  is_causal, p, seed, offset, s * H + h)
    return O, L


def attend_masked_dropout(q, k, v, scale, bias, is_causal, p, seed, offset, unit):
    """One unit with an elementwise additive bias (the reading of
    oracle/masked.py: s = scale q k^T + bias, -inf where a boolean mask
    drops a pair, and the causal rule on top) and dropout on the resulting
    softmax weights, with the keep mask z of this module for the unit:

        O_i = sum_j P_ij z_ij / kappa v_j,  lse_i = ln sum_j exp(s_ij)

    The mask decides which pairs take part in the softmax; dropout then
    acts on the weights of the pairs that do, with the same draws as
    without a mask (they depend on the pair's position only).  A row with
    no finite score has O = 0 and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = float(scale) * (q @ k.T) + np.asarray(bias, dtype=np.float64)
    nq, nk = s.shape
    if is_causal:
        s = np.where(np.arange(nk)[None, :] <= np.arange(nq)[:, None], s, -np.inf)
    live = np.any(s > -np.inf, axis=1)
    P = np.zeros_like(s)
    lse = np.full(nq, -np.inf)
    if np.any(live):
        sl = s[live]
        m = np.max(sl, axis=1, keepdims=True)   # overflow guard only
        e = np.exp(sl - m)
        l = np.sum(e, axis=1, keepdims=True)
        P[live] = e / l
        lse[live] = m[:, 0] + np.log(l[:, 0])
    z = keep_mask(nq, nk, unit, p, seed, offset)
    return ((P * z) / keep_probability(p)) @ v, lse


def sdpa_fwd_masked_dropout(q, k, v, mask, kind, scale, is_causal, p, seed, offset=0):
    """Dense q [B,H,Nq,d], k/v [B,H,Nk,d]; mask [Bm,Hm,Nq,Nk] (Bm in {1, B},
    Hm in {1, H}), kind "bool" (nonzero = attend) or "add"; unit u = b*H + h
    -> O, lse in float64."""
    B, H, Nq, _ = np.shape(q)
    m = np.asarray(mask)
    O = np.empty((B, H, Nq, np.shape(v)[3]))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            mu = m[b % m.shape[0], h % m.shape[1]]
            bias = np.where(mu != 0, 0.0, -np.inf) if kind == "bool" else mu.astype(np.float64)
            O[b, h], L[b, h] = attend_masked_dropout(q[b, h], k[b, h], v[b, h], scale, bias,
                                                     is_causal, p, seed, offset, b * H + h)
    return O, L

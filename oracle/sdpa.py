"""fp64 CPU oracle for the exact scaled dot-product attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares
no code with the GPU path and imports nothing from it.

What it computes (the plain definition, written out):

* The PyTorch SDPA tutorial ("Overview") says the function computes scaled
  dot-product attention as defined in *Attention is all you need*; the
  kuaisou snippet page (last snippet) describes it as weighting the values
  by how well the query matches each key, and its formal definition is cut
  off.  The reading taken here is the standard one:
      s_ij  = scale * <q_i, k_j>                      for j in A_i
      O_i   = sum_j softmax_j(s_i.) v_j
      lse_i = log sum_{j in A_i} exp(s_ij)            (natural log)
* A_i is every key, or with ``is_causal`` (the tutorial's CausalSelfAttention
  block) the keys j <= i (lower-triangular, aligned at the top-left corner,
  so a row is never empty).
* FlashAttention is exact attention ("IO-aware exact attention", the
  FlashAttention article's method paragraph; the tutorial's list of fused
  implementations), so the fused kernel is held to this plain result.
* Variable-length (NestedTensor) batches: each packed sequence attends only
  to itself (tutorial, "NestedTensor and dense tensor support").

Implementation notes: inputs are upcast to float64 exactly; each (batch,
head) or (sequence, head) unit materialises its score block in row chunks
(numpy matmul is the only library primitive used); subtracting the row
maximum before exponentiating only guards against overflow and leaves the
result unchanged, since softmax is invariant to a per-row shift.
"""
from __future__ import annotations

import numpy as np

_CHUNK_ELEMS = 1 << 24  # score entries per chunk (128 MiB of float64)


def _attend_unit(q, k, v, scale, is_causal, row_ids=None):
    """One (batch, head) unit.

    q [nq, d] rows with query indices ``row_ids`` (default 0..nq-1),
    k/v [nk, d].  Returns O [nq, d], lse [nq] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if row_ids is None:
        row_ids = np.arange(nq, dtype=np.int64)
    out = np.empty((nq, v.shape[1]), dtype=np.float64)
    lse = np.empty(nq, dtype=np.float64)
    step = max(1, _CHUNK_ELEMS // max(nk, 1))
    cols = np.arange(nk, dtype=np.int64)
    for r0 in range(0, nq, step):
        r1 = min(nq, r0 + step)
        s = float(scale) * (q[r0:r1] @ k.T)  # s_ij = scale * <q_i, k_j>
        if is_causal:
            allowed = cols[None, :] <= row_ids[r0:r1, None]
            s = np.where(allowed, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)  # overflow guard only
        e = np.exp(s - m)
        l = np.sum(e, axis=1, keepdims=True)
        out[r0:r1] = (e @ v) / l
        lse[r0:r1] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def sdpa_fwd(q, k, v, scale, is_causal=False):
    """Dense attention.  q [B,H,Nq,d], k/v [B,H,Nk,d] (any real dtype).

    Returns O [B,H,Nq,d] and lse [B,H,Nq], float64."""
    q = np.asarray(q)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if Nq == 0 or Nk == 0:
        raise ValueError("empty query or key set")
    O = np.empty((B, H, Nq, v.shape[3]), dtype=np.float64)
    L = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = _attend_unit(q[b, h], k[b, h], v[b, h], scale, is_causal)
    return O, L


def sdpa_fwd_rows(q, k, v, scale, is_causal, rows):
    """Dense attention on selected query rows only (every batch and head).

    Returns O [B,H,len(rows),d] and lse [B,H,len(rows)], float64."""
    rows = np.asarray(rows, dtype=np.int64)
    B, H = q.shape[0], q.shape[1]
    O = np.empty((B, H, len(rows), v.shape[3]), dtype=np.float64)
    L = np.empty((B, H, len(rows)), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = _attend_unit(q[b, h][rows], k[b, h], v[b, h], scale,
                                            is_causal, row_ids=rows)
    return O, L


def sdpa_fwd_varlen(q, k, v, cu_seqlens, scale, is_causal=False):
    """Packed variable-length self-attention.

    q/k/v [T,H,d]; sequence s owns rows cu_seqlens[s]:cu_seqlens[s+1] and
    attends only to itself.  Returns O [T,H,d] and lse [T,H], float64.
    Zero-length sequences contribute nothing."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d = q.shape
    O = np.zeros((T, H, v.shape[2]), dtype=np.float64)
    L = np.zeros((T, H), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        for h in range(H):
            O[a:b, h], L[a:b, h] = _attend_unit(q[a:b, h], k[a:b, h], v[a:b, h], scale,
                                                is_causal)
    return O, L


def attention_weights(q, k, scale, is_causal=False):
    """The softmax matrix P of one unit, q [nq,d], k [nk,d] -> [nq,nk].

    Exposed for the normalisation pin (rows of P sum to 1)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = float(scale) * (q @ k.T)
    if is_causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= np.arange(q.shape[0])[:, None],
                     s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=1, keepdims=True)

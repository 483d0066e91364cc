"""Seeded synthetic inputs for the attention forward and backward passes.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to the storage dtype, and decodes stored values back to float64
exactly.  The oracle and the GPU path both consume what it produces.

Every tensor comes from ``numpy.random.default_rng(SeedSequence([seed, cfg,
tensor_id]))`` with tensor ids q=0, k=1, v=2, lengths=3, forced index=4,
sampled rows=5, upstream gradient dO=6, block mask=7, elementwise mask values=8
and drops=9, so a workload is reproducible on any
machine with no torch
RNG involved.  Values are drawn in float32 and rounded to the storage dtype
with round-to-nearest-even (bf16 rounding is done on the bit pattern).

Workloads (each stands in for a workload printed on the pages):

1. tiny      -- the 2x3x8 ``torch.randn`` example of the PyTorch SDPA tutorial
                ("Fused implementations" section): B=2, H=1, N=3, d=8, f32.
2. noncausal -- the tutorial's dispatcher benchmark ("Explicit dispatcher
                control"): B=32, H=32, N=1024, d=32, f16, ``torch.rand``.
3. causal    -- the attention core of the tutorial's CausalSelfAttention
                module (embed 512, 8 heads, head dim 64) with causal masking
                switched on: B=32, H=8, N=1024, d=64, f16, N(0,1).
4. varlen    -- the NestedTensor batch recipe ("NestedTensor and dense tensor
                support"): 32 sequences of length int(512*(1-g)), g~N(0.5,
                0.01), one random entry forced to 512; H=8, d=64, f16, packed.
5. long      -- the 64k-token regime of the FlashAttention article's
                benchmark paragraph on one GPU: B=1, H=16, N=65536, d=64,
                bf16, causal; checked on 256 sampled query rows per head.
6. block_sparse -- the block-sparse FlashAttention of the same benchmark
                paragraph, at the same 64k-token size: B=1, H=16, N=65536,
                d=64, bf16, non-causal, one mask per head over 128x128
                blocks, each block kept with probability 1/4 and the
                diagonal blocks always kept (the pages give no mask).
7. masked    -- the tutorial's functional call with an ``attn_mask`` (its
                module passes None; the pages give no mask): the causal
                workload's shape, non-causal, with an additive f16 bias per
                (batch, head, query, key) ~ N(0, 2), a quarter of the pairs
                set to -inf.
8. padded    -- the dense side of the tutorial's NestedTensor comparison:
                workload 4's lengths in a dense [32, 8, 512, 64] f16 batch
                padded to 512, keys past each length masked by a boolean
                key-padding mask [32, 1, 1, 512] (padding rows hold random
                values: the kernel computes them like any other row).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# tensor ids for SeedSequence
_TID_Q, _TID_K, _TID_V, _TID_LEN, _TID_FORCE, _TID_ROWS, _TID_DO, _TID_MASK = range(8)
_TID_AMASK, _TID_AMASK_DROP = 8, 9

# largest float16 strictly below 1.0; uniform draws are clamped here so that
# rounding to f16 never produces 1.0 (the pages' torch.rand is [0, 1)).
_F16_BELOW_ONE = np.float32(0.99951171875)

DTYPES = ("f16", "bf16", "f32")


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs must be finite (the generator never produces NaN/Inf)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to float64."""
    u32 = (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16)
    return u32.view(np.float32).astype(np.float64)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype.

    Returns float32 / float16 arrays, or uint16 bit patterns for bf16."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == "bf16":
        return round_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a).astype(np.float64)


def _rng(seed: int, cfg: int, tid: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(cfg), int(tid)]))


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(size=shape, dtype=np.float32)
    if dist == "uniform":
        u = rng.random(size=shape, dtype=np.float32)
        return np.minimum(u, _F16_BELOW_ONE)
    raise ValueError(f"unknown distribution {dist!r}")


@dataclasses.dataclass
class Workload:
    """One seeded problem instance.

    Dense: q [B,H,Nq,d], k/v [B,H,Nk,d].  Varlen (cu_seqlens set): q/k/v
    packed [T,H,d] with sequence s in rows cu_seqlens[s]:cu_seqlens[s+1].
    ``q``/``k``/``v`` hold the stored values (f32/f16 arrays, or uint16 bf16
    bit patterns); ``q64`` etc. are their exact float64 values."""

    name: str
    dtype: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    is_causal: bool
    scale: np.float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: Optional[np.ndarray] = None
    rows: Optional[np.ndarray] = None  # sampled query rows (dense only)
    block_mask: Optional[np.ndarray] = None  # uint8 [Hm, nqb, nkb] (dense only)
    attn_mask: Optional[np.ndarray] = None   # elementwise mask, broadcast to [B,H,Nq,Nk]
    mask_kind: Optional[str] = None          # "bool" or "add" (stored in ``dtype``)

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens is not None

    @property
    def q64(self) -> np.ndarray:
        return storage_to_f64(self.q, self.dtype)

    @property
    def k64(self) -> np.ndarray:
        return storage_to_f64(self.k, self.dtype)

    @property
    def v64(self) -> np.ndarray:
        return storage_to_f64(self.v, self.dtype)

    def flops(self) -> float:
        """Metric FLOPs: 4*B*H*Nq*Nk*d, halved when causal; varlen sums
        4*H*len^2*d over sequences (halved when causal); with a block mask,
        4*d per (query, key) pair the mask leaves visible."""
        if self.block_mask is not None:
            return 4.0 * self.d * self.B * visible_pairs(self.block_mask, self.Nq, self.Nk,
                                                         self.is_causal, self.H)
        if self.varlen:
            lens = np.diff(self.cu_seqlens.astype(np.int64))
            f = float(np.sum(4.0 * self.H * lens.astype(np.float64) ** 2 * self.d))
        else:
            f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.is_causal else f


def default_scale(d: int) -> np.float32:
    return np.float32(1.0 / math.sqrt(d))


def make_dense(B, H, Nq, Nk, d, dtype="f16", dist="normal", is_causal=False,
               seed=0, cfg=0, scale=None, name="dense") -> Workload:
    q32 = _draw(_rng(seed, cfg, _TID_Q), (B, H, Nq, d), dist)
    k32 = _draw(_rng(seed, cfg, _TID_K), (B, H, Nk, d), dist)
    v32 = _draw(_rng(seed, cfg, _TID_V), (B, H, Nk, d), dist)
    sc = default_scale(d) if scale is None else np.float32(scale)
    return Workload(name=name, dtype=dtype, B=B, H=H, Nq=Nq, Nk=Nk, d=d,
                    is_causal=is_causal, scale=sc,
                    q=to_storage(q32, dtype), k=to_storage(k32, dtype),
                    v=to_storage(v32, dtype))


def make_grad_out(w: Workload, seed=0, cfg=0, dist="normal", scale=1.0) -> np.ndarray:
    """Upstream gradient dO for workload ``w`` (the shape of its output), in
    its storage dtype; ``scale`` multiplies the float32 draws before the
    rounding (e.g. 1e-6 for the small gradients of bf16 training)."""
    shape = (w.q.shape[0], w.q.shape[1], w.q.shape[2], w.d) if not w.varlen else w.q.shape
    g = _draw(_rng(seed, cfg, _TID_DO), shape, dist)
    if scale != 1.0:
        g = (g * np.float32(scale)).astype(np.float32)
    return to_storage(g, w.dtype)


def nested_lengths(batch: int, max_len: int, pad_fraction: float, seed=0, cfg=4) -> np.ndarray:
    """The NestedTensor batch recipe: len_i = int(max_len*(1-g_i)) with
    g_i ~ N(pad_fraction, 0.01), then one uniformly chosen entry is set to
    max_len.  Lengths are clamped to [1, max_len]."""
    g = _rng(seed, cfg, _TID_LEN).normal(loc=pad_fraction, scale=0.01, size=batch)
    lens = np.array([int(max_len * (1.0 - gi)) for gi in g], dtype=np.int64)
    forced = int(_rng(seed, cfg, _TID_FORCE).integers(0, batch))
    lens[forced] = max_len
    return np.clip(lens, 1, max_len)


def cu_seqlens_from_lengths(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    assert cu[-1] < 2 ** 31
    return cu.astype(np.int32)


def make_varlen(lens, H, d, dtype="f16", dist="normal", is_causal=False, seed=0,
                cfg=0, scale=None, name="varlen") -> Workload:
    lens = np.asarray(lens, dtype=np.int64)
    cu = cu_seqlens_from_lengths(lens)
    T = int(cu[-1])
    q32 = _draw(_rng(seed, cfg, _TID_Q), (T, H, d), dist)
    k32 = _draw(_rng(seed, cfg, _TID_K), (T, H, d), dist)
    v32 = _draw(_rng(seed, cfg, _TID_V), (T, H, d), dist)
    sc = default_scale(d) if scale is None else np.float32(scale)
    mx = int(lens.max()) if len(lens) else 0
    return Workload(name=name, dtype=dtype, B=len(lens), H=H, Nq=mx, Nk=mx, d=d,
                    is_causal=is_causal, scale=sc,
                    q=to_storage(q32, dtype), k=to_storage(k32, dtype),
                    v=to_storage(v32, dtype), cu_seqlens=cu)


def sample_rows(n: int, count: int, seed=0, cfg=5) -> np.ndarray:
    """``count`` distinct query rows of [0, n), sorted."""
    rng = _rng(seed, cfg, _TID_ROWS)
    return np.sort(rng.choice(n, size=min(count, n), replace=False)).astype(np.int64)


def visible_pairs(mask: np.ndarray, nq: int, nk: int, is_causal: bool, heads: int,
                  block: int = 128) -> float:
    """Number of (query, key) pairs a block mask leaves visible, summed over
    ``heads`` heads (a one-head mask counts once per head); causal pairs
    need key <= query.  Bookkeeping for the FLOP count only."""
    m = np.asarray(mask) != 0
    rq = np.minimum(block, nq - block * np.arange(m.shape[1]))      # rows per block row
    rk = np.minimum(block, nk - block * np.arange(m.shape[2]))      # keys per block column
    if is_causal:
        per = np.zeros((m.shape[1], m.shape[2]))
        for i in range(m.shape[1]):
            r = block * i + np.arange(rq[i])                        # query indices
            for j in range(m.shape[2]):
                per[i, j] = np.sum(np.clip(r - block * j + 1, 0, rk[j]))
    else:
        per = np.outer(rq, rk).astype(np.float64)
    tot = float(np.sum(m * per[None]))
    return tot * heads if m.shape[0] == 1 else tot


def make_block_mask(heads: int, nq: int, nk: int, density: float, diagonal=False, seed=0,
                    cfg=0, block=128) -> np.ndarray:
    """uint8 block mask [heads, ceil(nq/block), ceil(nk/block)]: each entry
    is 1 with probability ``density``, independently; with ``diagonal`` the
    entries (i, i) are forced to 1, so every query block sees its own key
    block."""
    shape = (heads, -(-nq // block), -(-nk // block))
    m = (_rng(seed, cfg, _TID_MASK).random(shape) < density).astype(np.uint8)
    if diagonal:
        n = min(shape[1], shape[2])
        m[:, np.arange(n), np.arange(n)] = 1
    return m


# --- score structures that move the softmax's row maximum late -------------
#
# Random N(0,1) inputs keep every score within a few units of the first
# block's maximum, so a kernel that fixes its softmax reference early is
# never made to move it.  These families build q and k (v stays N(0,1)) so
# that the maximum of a row arrives after its first block of keys:
#
#   late      keys are scaled to length sqrt(d), and each query row is
#             aligned with one key of the row's last key tile (its own key
#             when causal, else one of the last 64 keys):
#             q_i = 0.25 z_i + beta * k_j / (scale d) puts that key's score
#             beta = 48 natural-log units above a typical score.
#   rising    scores climb steadily along the keys: q_i[0] = 8 and
#             k_j[0] = rate * pos_j with rate chosen so that 2048 keys add
#             120 log2 units (pos_j counts from the start of the key's own
#             sequence).
#   low_first the first 32 keys of every unit sit 25 log2 units below the
#             rest: q_i[0] = 8, k_j[0] = -drop for pos_j < 32.
#
# Offsets are applied in float32 before the rounding to the storage dtype;
# the oracle sees the stored values, whatever the rounding did to them.

RESCALE_FAMILIES = ("late", "rising", "low_first")
_RISE_LOG2_PER_KEY = 120.0 / 2048.0
_LATE_MARGIN = 48.0
_LOW_FIRST_LOG2 = 25.0
_LOG2E = 1.4426950408889634


def _shape_unit(q: np.ndarray, k: np.ndarray, family: str, causal: bool, scale: float) -> None:
    """Apply ``family`` in place to one unit's q [nq, d] and k [nk, d]
    (float32, rows in sequence order)."""
    nq, nk = q.shape[0], k.shape[0]
    if nq == 0 or nk == 0:
        return
    if family == "late":
        # keys on the sphere of radius sqrt(d), so that a row's margin does
        # not depend on its key's length
        d = k.shape[1]
        k64 = k.astype(np.float64)
        k64 *= math.sqrt(d) / np.maximum(np.linalg.norm(k64, axis=1, keepdims=True), 1e-6)
        k[:] = k64.astype(np.float32)
        i = np.arange(nq)
        j = np.minimum(i, nk - 1) if causal else nk - 1 - (i % min(64, nk))
        q[:] = (0.25 * q + _LATE_MARGIN * k64[j] / (scale * d)).astype(np.float32)
        return
    a = np.float32(8.0)
    q[:, 0] = a
    if family == "rising":
        rate = _RISE_LOG2_PER_KEY / (scale * _LOG2E * float(a))
        k[:, 0] = (rate * np.arange(nk)).astype(np.float32)
    elif family == "low_first":
        drop = _LOW_FIRST_LOG2 / (scale * _LOG2E * float(a))
        k[:, 0] = 0.0
        k[:min(32, nk), 0] = np.float32(-drop)
    else:
        raise ValueError(f"unknown family {family!r}")


def make_rescale(family: str, B, H, Nq, Nk, d, dtype="f16", is_causal=False, seed=0, cfg=0,
                 lens=None, name=None) -> Workload:
    """A dense (or, with ``lens``, packed) workload whose row maxima arrive
    late (see the family list above); N(0,1) values otherwise."""
    if lens is not None:
        w = make_varlen(lens, H, d, "f32", "normal", is_causal, seed, cfg)
        q32, k32 = w.q.copy(), w.k.copy()
        cu = w.cu_seqlens
        for s in range(len(cu) - 1):
            for h in range(H):
                sl = slice(int(cu[s]), int(cu[s + 1]))
                qs, ks = q32[sl, h].copy(), k32[sl, h].copy()
                _shape_unit(qs, ks, family, is_causal, float(w.scale))
                q32[sl, h], k32[sl, h] = qs, ks
    else:
        w = make_dense(B, H, Nq, Nk, d, "f32", "normal", is_causal, seed, cfg)
        q32, k32 = w.q.copy(), w.k.copy()
        for b in range(B):
            for h in range(H):
                _shape_unit(q32[b, h], k32[b, h], family, is_causal, float(w.scale))
    w.q = to_storage(q32, dtype)
    w.k = to_storage(k32, dtype)
    w.v = to_storage(w.v, dtype)
    w.dtype = dtype
    w.name = name or f"rescale-{family}"
    return w


CONFIG_NAMES = {1: "tiny", 2: "noncausal", 3: "causal", 4: "varlen", 5: "long", 7: "masked",
                8: "padded",
                6: "block_sparse"}


def make_attn_mask(shape, kind: str, keep: float = 0.75, bias_std: float = 2.0, seed=0,
                   cfg=0, dtype="f16") -> np.ndarray:
    """A seeded elementwise attention mask of ``shape``.

    kind "bool": uint8 0/1, each pair kept (1) with probability ``keep``.
    kind "add":  additive values ~ N(0, bias_std) rounded to ``dtype``
                 ("f16", "bf16" as uint16 bits, or "f32"), and -inf where an
                 independent draw drops the pair (probability 1 - keep)."""
    drop = _rng(seed, cfg, _TID_AMASK_DROP).random(shape, dtype=np.float32) >= keep
    if kind == "bool":
        return (~drop).astype(np.uint8)
    a = _rng(seed, cfg, _TID_AMASK).standard_normal(shape, dtype=np.float32) * np.float32(bias_std)
    a[drop] = -np.inf
    return to_storage(a, dtype)


def key_padding_mask(lens, max_len: int) -> np.ndarray:
    """uint8 [B, 1, 1, max_len]: key j of batch b is kept iff j < lens[b]
    (a padded dense batch of the NestedTensor recipe's sequences)."""
    lens = np.asarray(lens)
    return (np.arange(max_len)[None, :] < lens[:, None]).astype(np.uint8)[:, None, None, :]


def make_config(i: int, seed: int = 0) -> Workload:
    """The five workloads (see module docstring)."""
    if i == 1:
        return make_dense(2, 1, 3, 3, 8, "f32", "normal", False, seed, 1, name="tiny")
    if i == 2:
        return make_dense(32, 32, 1024, 1024, 32, "f16", "uniform", False, seed, 2,
                          name="noncausal")
    if i == 3:
        return make_dense(32, 8, 1024, 1024, 64, "f16", "normal", True, seed, 3,
                          name="causal")
    if i == 4:
        lens = nested_lengths(32, 512, 0.5, seed, 4)
        return make_varlen(lens, 8, 64, "f16", "normal", False, seed, 4, name="varlen")
    if i == 5:
        w = make_dense(1, 16, 65536, 65536, 64, "bf16", "normal", True, seed, 5,
                       name="long")
        w.rows = sample_rows(65536, 256, seed, 5)
        return w
    if i == 6:
        w = make_dense(1, 16, 65536, 65536, 64, "bf16", "normal", False, seed, 6,
                       name="block_sparse")
        w.block_mask = make_block_mask(16, 65536, 65536, 0.25, diagonal=True, seed=seed, cfg=6)
        w.rows = sample_rows(65536, 256, seed, 6)
        return w
    if i == 7:
        # an additive f16 bias per (batch, head, query, key), a quarter of
        # the pairs dropped with -inf, on the causal workload's shape
        w = make_dense(32, 8, 1024, 1024, 64, "f16", "normal", False, seed, 7, name="masked")
        w.attn_mask = make_attn_mask((32, 8, 1024, 1024), "add", keep=0.75, bias_std=2.0,
                                     seed=seed, cfg=7, dtype="f16")
        w.mask_kind = "add"
        return w
    if i == 8:
        # the NestedTensor recipe's sequences as a padded dense batch with a
        # key-padding mask (the dense side of the tutorial's comparison)
        lens = nested_lengths(32, 512, 0.5, seed, 4)
        w = make_dense(32, 8, 512, 512, 64, "f16", "normal", False, seed, 8, name="padded")
        w.attn_mask = key_padding_mask(lens, 512)
        w.mask_kind = "bool"
        return w
    raise ValueError(f"no config {i}")

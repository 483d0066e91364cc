"""GPU parity of the dropout forward (sdpa_fwd_dropout) against the fp64
dropout oracle, through the C ABI.

Tolerances are those of the dense forward (tests/gpu_util.py).  The keep
decisions are integer work, so they are compared bit for bit: with q = 0
and V the identity (d = Nk), O_ij = z_ij / ((1 - p) |A_i|), which exposes
the kernel's whole mask.
"""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from oracle import dropout as odrop
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _run(w, p, seed, offset=0, out_f32=False, q=None, k=None, v=None):
    q, k, v = (G.to_device(x, w.dtype) if t is None else t
               for x, t in ((w.q, q), (w.k, k), (w.v, v)))
    cu = torch.from_numpy(w.cu_seqlens).to("cuda") if w.varlen else None
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, is_causal=w.is_causal, scale=float(w.scale), cu_seqlens=cu,
        max_seqlen=w.Nq if w.varlen else None, dropout_p=p, dropout_seed=seed,
        dropout_offset=offset, out_dtype=torch.float32 if out_f32 else None, return_lse=True)
    torch.cuda.synchronize()
    return out.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def _ref(w, p, seed, offset=0):
    if w.varlen:
        return odrop.sdpa_fwd_dropout_varlen(w.q64, w.k64, w.v64, w.cu_seqlens, w.scale,
                                             w.is_causal, p, seed, offset)
    return odrop.sdpa_fwd_dropout(w.q64, w.k64, w.v64, w.scale, w.is_causal, p, seed, offset)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_sweep(dtype, d, causal):
    w = inputs.make_dense(2, 3, 300, 300, d, dtype, "normal", causal, seed=d, cfg=100)
    o, lse = _run(w, 0.2, seed=1234 + d, offset=3, out_f32=dtype == "bf16")
    ref, lref = _ref(w, 0.2, 1234 + d, 3)
    G.assert_parity(o, ref, dtype, f"dropout {dtype} d{d} causal={causal}", lse, lref)


@pytest.mark.parametrize("p", [0.05, 0.5, 0.9])
@pytest.mark.parametrize("nq,nk", [(1, 300), (300, 1), (129, 700), (700, 129)])
def test_dropout_rates_and_shapes(p, nq, nk):
    w = inputs.make_dense(1, 2, nq, nk, 64, "f16", "normal", True, seed=nq + nk, cfg=101)
    o, lse = _run(w, p, seed=7, offset=0, out_f32=True)
    ref, lref = _ref(w, p, 7, 0)
    # kept weights are scaled by 1/(1-p): so is the error of the f16 P
    G.assert_parity(o * (1 - p), ref * (1 - p), "f16", f"p={p} nq{nq} nk{nk}", lse, lref)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_packed(causal):
    lens = [1, 31, 32, 33, 0, 64, 127, 128, 129, 300, 5]
    w = inputs.make_varlen(lens, 2, 64, "bf16", "normal", causal, seed=5, cfg=102)
    o, lse = _run(w, 0.3, seed=99, offset=11, out_f32=True)
    ref, lref = _ref(w, 0.3, 99, 11)
    G.assert_parity(o, ref, "bf16", f"packed causal={causal}", lse, lref)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("varlen", [False, True])
def test_keep_mask_is_bit_exact(causal, varlen):
    """q = 0, V = identity: the output exposes every keep decision."""
    nk, p, seed, off = 128, 0.3, 0x0123456789ABCDEF, 5
    eye = np.eye(nk, dtype=np.float16)
    if varlen:
        lens = [128, 57, 128]
        cu = inputs.cu_seqlens_from_lengths(lens)
        T, H = int(cu[-1]), 2
        q = torch.zeros(T, H, nk, dtype=torch.float16, device="cuda")
        vv = np.zeros((T, H, nk), np.float16)
        for s, n in enumerate(lens):
            vv[cu[s]:cu[s] + n] = eye[:n, None, :]
        v = torch.from_numpy(vv).to("cuda")
        out = sdpa.scaled_dot_product_attention(
            q, q, v, is_causal=causal, cu_seqlens=torch.from_numpy(cu).to("cuda"),
            max_seqlen=128, dropout_p=p, dropout_seed=seed, dropout_offset=off,
            out_dtype=torch.float32)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        for s, n in enumerate(lens):
            for h in range(H):
                z = o[cu[s]:cu[s] + n, h, :n] > 0
                want = odrop.keep_mask(n, n, s * H + h, p, seed, off)
                if causal:
                    want = want & np.tri(n, dtype=bool)
                assert np.array_equal(z, want), f"sequence {s} head {h}"
    else:
        B, H, nq = 2, 2, 300
        q = torch.zeros(B, H, nq, nk, dtype=torch.float16, device="cuda")
        k = torch.zeros(B, H, nk, nk, dtype=torch.float16, device="cuda")
        v = torch.from_numpy(np.broadcast_to(eye, (B, H, nk, nk)).copy()).to("cuda")
        out = sdpa.scaled_dot_product_attention(
            q, k, v, is_causal=causal, dropout_p=p, dropout_seed=seed, dropout_offset=off,
            out_dtype=torch.float32)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        for b in range(B):
            for h in range(H):
                z = o[b, h] > 0
                want = odrop.keep_mask(nq, nk, b * H + h, p, seed, off)
                if causal:
                    want = want & (np.arange(nk)[None, :] <= np.arange(nq)[:, None])
                assert np.array_equal(z, want), f"unit {b * H + h}"
                # the kept values are exactly 1 / ((1 - p) |A_i|)
                cnt = np.minimum(np.arange(nq) + 1, nk) if causal else np.full(nq, nk)
                kept = np.where(want, 1.0 / ((1 - np.float32(p)) * cnt[:, None]), 0.0)
                np.testing.assert_allclose(o[b, h], kept, rtol=2e-3)


def test_same_seed_same_output_and_lse_matches_plain():
    # 2 x 136 units of one query tile: above the tile count under which plain
    # launches split each workgroup's keys over two wave groups, so the plain
    # kernel adds the keys in the dropout kernel's order
    w = inputs.make_dense(2, 136, 200, 200, 64, "f16", "normal", True, seed=9, cfg=103)
    a = _run(w, 0.1, seed=5, offset=1)
    b = _run(w, 0.1, seed=5, offset=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = _run(w, 0.1, seed=6, offset=1)
    d = _run(w, 0.1, seed=5, offset=2)
    assert not np.array_equal(a[0], c[0]) and not np.array_equal(a[0], d[0])
    # the row sums keep the undropped weights: lse is the plain kernel's
    plain = G.run(w)
    assert np.array_equal(a[1], plain[1])
    # p = 0 is the plain kernel
    z = _run(w, 0.0, seed=5)
    assert np.array_equal(z[0], plain[0])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_one_group_grid(dtype, d, causal):
    """The small grids above run the dropout kernels that split each
    workgroup's keys over two wave groups; 130 units of two query tiles
    (N = 300) run the one-group ones, checked on sampled units plus the
    first and last."""
    B, H, n, p, seed, off = 1, 130, 300, 0.2, 77 + d, 4
    assert B * H * -(-n // 256) > 256
    w = inputs.make_dense(B, H, n, n, d, dtype, "normal", causal, seed=d + causal, cfg=104)
    o, lse = _run(w, p, seed=seed, offset=off, out_f32=dtype == "bf16")
    for h in (0, 17, 64, H - 1):
        ref, lref = odrop.attend_dropout(w.q64[0, h], w.k64[0, h], w.v64[0, h], w.scale, causal,
                                         p, seed, off, h)
        G.assert_parity(o[0, h] * (1 - p), ref * (1 - p), dtype, f"one group {dtype} d{d} head {h}",
                        lse[0, h], lref)


def test_module_training_workload_full_size():
    """The tutorial's CausalSelfAttention core in training (dropout 0.1,
    causal; B32 H8 N1024 d64 f16), checked on sampled (batch, head) units."""
    w = inputs.make_config(3)
    o, lse = _run(w, 0.1, seed=2023, offset=0)
    rng = np.random.default_rng(0)
    q64, k64, v64 = w.q64, w.k64, w.v64
    for u in rng.choice(w.B * w.H, size=6, replace=False):
        b, h = divmod(int(u), w.H)
        ref, lref = odrop.attend_dropout(q64[b, h], k64[b, h], v64[b, h], w.scale, True, 0.1,
                                         2023, 0, b * w.H + h)
        G.assert_parity(o[b, h], ref, "f16", f"unit {b},{h}", lse[b, h], lref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d32_wide_grid_dropout(dtype, causal):
    """d = 32 grids of at least 2048 query tiles of 256 rows run the dropout
    kernels with two query blocks per wave: B32 H32 N1024 (the headline
    shape in training) and a ragged N = 600 grid, on sampled units plus the
    first and last."""
    for B, H, n in ((32, 32, 1024), (22, 32, 600)):
        assert B * H * -(-n // 256) >= 2048
        w = inputs.make_dense(B, H, n, n, 32, dtype, "normal", causal, seed=n + 5 * causal,
                              cfg=103)
        o, lse = _run(w, 0.15, seed=77, offset=4, out_f32=dtype == "bf16")
        q64, k64, v64 = w.q64, w.k64, w.v64
        rng = np.random.default_rng(n)
        units = [0, B * H - 1] + [int(u) for u in rng.choice(B * H, size=6, replace=False)]
        for u in units:
            b, h = divmod(u, H)
            ref, lref = odrop.attend_dropout(q64[b, h], k64[b, h], v64[b, h], w.scale, causal,
                                             0.15, 77, 4, u)
            G.assert_parity(o[b, h] * 0.85, ref * 0.85, dtype,
                            f"wide dropout N{n} unit {b},{h}", lse[b, h], lref)

"""Parity of the HIP path against the fp64 oracle, through the C ABI.

Tolerances are in tests/gpu_util.py.  Small shapes are compared in full;
the large workloads are compared on whole sampled (batch, head) units or on
sampled query rows that the oracle computes one by one.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_sdpa_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _dense_ref(w, rows=None):
    if rows is None:
        return oracle.sdpa_fwd(w.q64, w.k64, w.v64, w.scale, w.is_causal)
    return oracle.sdpa_fwd_rows(w.q64, w.k64, w.v64, w.scale, w.is_causal, rows)


# --- the tiny f32 workload of the tutorial's example -------------------------

def test_config1_tiny_f32():
    w = inputs.make_config(1)
    o, lse = G.run(w)
    ref, lref = _dense_ref(w)
    G.assert_parity(o, ref, "f32", "config1", lse, lref)


# --- shape sweeps on the matrix-core path ------------------------------------

SWEEP_N = [1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 257]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_sweep(dtype, d, causal):
    for n in SWEEP_N:
        w = inputs.make_dense(1, 2, n, n, d, dtype, "normal", causal, seed=n, cfg=40 + d)
        out_f32 = dtype == "bf16"
        o, lse = G.run(w, out_f32=out_f32)
        ref, lref = _dense_ref(w)
        G.assert_parity(o, ref, dtype, f"{dtype} d{d} causal{causal} N{n}", lse, lref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [250, 600])
def test_d32_wide_grid(dtype, causal, n):
    """d = 32 grids of at least 2048 query tiles of 256 rows run the kernels
    with two query blocks per wave: distinct random units, full sequences
    and ragged tails, every unit compared with the oracle."""
    B = 64 if n <= 256 else 22      # 64 x 32 x 1 or 22 x 32 x 3 >= 2048 tiles
    w = inputs.make_dense(B, 32, n, n, 32, dtype, "normal", causal, seed=n + causal, cfg=45)
    assert w.B * w.H * -(-n // 256) >= 2048
    ref, lref = _dense_ref(w)
    for out_f32 in ((True,) if dtype == "bf16" else (False, True)):
        o, lse = G.run(w, out_f32=out_f32)
        G.assert_parity(o, ref, dtype, f"wide {dtype} N{n} causal{causal} f32out{out_f32}",
                        lse, lref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_split_threshold_both_sides(dtype, d, causal):
    """Plain grids of at most 128 query tiles of 256 rows (256 at d = 32 and
    when causal) split each workgroup's keys over two wave groups that merge
    their states; one tile more runs the one-group kernels.  The same ragged
    units (N = 300, two tiles each) on both sides of the threshold, every
    unit against the oracle, and the two results against each other."""
    limit = 256 if (d == 32 or causal) else 128
    H = limit // 2 + 1       # H x 2 tiles: one group; (H - 1) x 2 = limit: two
    w = inputs.make_dense(1, H, 300, 300, d, dtype, "normal", causal, seed=d + causal, cfg=46)
    ws = dataclasses.replace(w, H=H - 1, q=w.q[:, : H - 1].copy(), k=w.k[:, : H - 1].copy(),
                             v=w.v[:, : H - 1].copy())
    ref, lref = _dense_ref(w)
    out_f32 = dtype == "bf16"
    o1, l1 = G.run(w, out_f32=out_f32)
    G.assert_parity(o1, ref, dtype, f"one group {dtype} d{d} causal{causal}", l1, lref)
    o2, l2 = G.run(ws, out_f32=out_f32)
    G.assert_parity(o2, ref[:, : H - 1], dtype, f"two groups {dtype} d{d} causal{causal}", l2,
                    lref[:, : H - 1])
    # the two orders of additions agree to fp32 rounding of O and lse
    G.assert_parity(o2, o1[:, : H - 1], dtype, "two groups vs one", l2, l1[:, : H - 1])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 300), (130, 70), (70, 130), (256, 1000), (1000, 256)])
def test_dense_nq_ne_nk(dtype, causal, nq, nk):
    w = inputs.make_dense(2, 3, nq, nk, 64, dtype, "normal", causal, seed=nq * 7 + nk, cfg=50)
    o, lse = G.run(w, out_f32=dtype == "bf16")
    ref, lref = _dense_ref(w)
    G.assert_parity(o, ref, dtype, f"nq{nq} nk{nk}", lse, lref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_sweep(dtype, d, causal):
    lens = [1, 31, 32, 33, 0, 64, 127, 128, 129, 300, 5]
    w = inputs.make_varlen(lens, 2, d, dtype, "normal", causal, seed=d, cfg=60)
    o, lse = G.run(w, out_f32=dtype == "bf16")
    ref, lref = oracle.sdpa_fwd_varlen(w.q64, w.k64, w.v64, w.cu_seqlens, w.scale, causal)
    G.assert_parity(o, ref, dtype, f"varlen {dtype} d{d} causal{causal}", lse, lref)


def test_output_dtypes():
    """f16 in -> f16 or f32 out; bf16 in -> bf16 (one extra rounding) or f32."""
    for dtype in ("f16", "bf16"):
        w = inputs.make_dense(2, 2, 150, 150, 64, dtype, "normal", True, seed=3, cfg=70)
        ref, lref = _dense_ref(w)
        o, lse = G.run(w, out_f32=True)
        G.assert_parity(o, ref, dtype, f"{dtype}->f32", lse, lref)
        o, lse = G.run(w, out_f32=False)
        G.assert_parity(o, ref, dtype, f"{dtype}->same", lse, lref, bf16_out=dtype == "bf16")


@pytest.mark.parametrize("d", [1, 3, 8, 16, 33, 64, 100, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_sweep(d, causal):
    for nq, nk in [(1, 1), (5, 5), (64, 64), (65, 65), (100, 37), (37, 100), (200, 200)]:
        w = inputs.make_dense(2, 2, nq, nk, d, "f32", "normal", causal, seed=d + nq, cfg=80)
        o, lse = G.run(w)
        ref, lref = _dense_ref(w)
        G.assert_parity(o, ref, "f32", f"f32 d{d} {nq}x{nk} causal{causal}", lse, lref)


def test_f32_varlen():
    w = inputs.make_varlen([3, 0, 70, 1, 129], 3, 24, "f32", "normal", True, seed=1, cfg=81)
    o, lse = G.run(w)
    ref, lref = oracle.sdpa_fwd_varlen(w.q64, w.k64, w.v64, w.cu_seqlens, w.scale, True)
    G.assert_parity(o, ref, "f32", "f32 varlen", lse, lref)


def test_grid_not_multiple_of_eight():
    """B*H*tiles not divisible by 8 takes the plain block order."""
    w = inputs.make_dense(1, 3, 200, 200, 64, "f16", "normal", False, seed=2, cfg=90)
    o, lse = G.run(w)
    ref, lref = _dense_ref(w)
    G.assert_parity(o, ref, "f16", "odd grid", lse, lref)


# --- the workloads at full size ----------------------------------------------

def _sampled_units(w, n_units, seed):
    rng = np.random.default_rng(seed)
    units = rng.choice(w.B * w.H, size=min(n_units, w.B * w.H), replace=False)
    return [(int(u) // w.H, int(u) % w.H) for u in units]


def _unit_ref(w, b, h):
    """Oracle on one (batch, head) unit, decoding only that unit's values."""
    dec = lambda a: inputs.storage_to_f64(a[b:b + 1, h:h + 1], w.dtype)
    return oracle.sdpa_fwd(dec(w.q), dec(w.k), dec(w.v), w.scale, w.is_causal)


def _check_units(w, o, lse, units, dtype, what):
    O_g, L_g, O_r, L_r = [], [], [], []
    for b, h in units:
        ref, lref = _unit_ref(w, b, h)
        O_g.append(o[b, h]); L_g.append(lse[b, h]); O_r.append(ref[0, 0]); L_r.append(lref[0, 0])
    return G.assert_parity(np.stack(O_g), np.stack(O_r), dtype, what, np.stack(L_g),
                           np.stack(L_r))


def test_config2_noncausal_full_size():
    w = inputs.make_config(2)
    o, lse = G.run(w)
    units = _sampled_units(w, 48, 2)
    m = _check_units(w, o, lse, units, "f16", "config2")
    # centered metric: the uniform inputs make attention nearly flat, so also
    # compare the deviation from the column mean of V (bound 0.15 with an
    # f16 output, whose rounding dominates the deviation).
    num = den = 0.0
    for b, h in units:
        ref, _ = _unit_ref(w, b, h)
        mu = inputs.storage_to_f64(w.v[b, h], w.dtype).mean(axis=0)
        num += np.sum(((o[b, h] - mu) - (ref[0, 0] - mu)) ** 2)
        den += np.sum((ref[0, 0] - mu) ** 2)
    assert math.sqrt(num / den) <= 0.15, f"centered rel-L2 {math.sqrt(num / den):.3f}"
    assert m["rel_l2"] <= 1e-3


def test_config2_centered_f32_output():
    """Diagnostic run with an f32 output: the centered error must be small
    (<= 1e-2), which rules out kernels that ignore Q.K or misapply the scale."""
    w = inputs.make_config(2)
    o, _ = G.run(w, out_f32=True, with_lse=False)
    num = den = 0.0
    for b, h in _sampled_units(w, 24, 3):
        ref, _ = _unit_ref(w, b, h)
        mu = inputs.storage_to_f64(w.v[b, h], w.dtype).mean(axis=0)
        num += np.sum(((o[b, h] - mu) - (ref[0, 0] - mu)) ** 2)
        den += np.sum((ref[0, 0] - mu) ** 2)
    assert math.sqrt(num / den) <= 1e-2, f"centered rel-L2 {math.sqrt(num / den):.4f}"


def test_config3_causal_full_size():
    w = inputs.make_config(3)
    o, lse = G.run(w)
    _check_units(w, o, lse, _sampled_units(w, 32, 3), "f16", "config3")


def test_config4_varlen_full():
    w = inputs.make_config(4)
    o, lse = G.run(w)
    ref, lref = oracle.sdpa_fwd_varlen(w.q64, w.k64, w.v64, w.cu_seqlens, w.scale, False)
    G.assert_parity(o, ref, "f16", "config4", lse, lref)


def test_config5_long_sampled_rows():
    w = inputs.make_config(5)
    o, lse = G.run(w, out_f32=True)
    ref, lref = _dense_ref(w, w.rows)
    G.assert_parity(o[:, :, w.rows], ref, "bf16", "config5 sampled rows",
                    lse[:, :, w.rows], lref)
    edge = np.array([0, 1, 2, 3, 63, 64, 127, 128, 65535])
    eref, elref = _dense_ref(w, edge)
    err = float(np.max(np.abs(o[:, :, edge] - eref)))
    assert err <= 2e-3, f"config5 edge rows max-abs {err:.3e}"
    assert float(np.max(np.abs(lse[:, :, edge] - elref))) <= 1e-4


# --- invariants on GPU outputs -----------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_row0_is_v0(dtype):
    w = inputs.make_dense(2, 2, 300, 300, 64, dtype, "normal", True, seed=5, cfg=100)
    o, lse = G.run(w, out_f32=False)
    assert np.array_equal(o[:, :, 0], w.v64[:, :, 0])
    lref = w.scale * np.einsum("bhd,bhd->bh", w.q64[:, :, 0], w.k64[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - lref)) <= 1e-4


def test_identical_keys_give_mean_of_v():
    w = inputs.make_dense(1, 2, 100, 257, 64, "f16", "normal", False, seed=6, cfg=101)
    w.k = np.broadcast_to(w.k[:, :, :1], w.k.shape).copy()
    o, lse = G.run(w, out_f32=True)
    mean = w.v64.mean(axis=2, keepdims=True)
    assert np.max(np.abs(o - mean)) <= 1e-3
    lref = w.scale * np.einsum("bhid,bhd->bhi", w.q64, w.k64[:, :, 0]) + math.log(257)
    assert np.max(np.abs(lse - lref)) <= 1e-4


def test_scale_zero_is_mean_and_log_n():
    w = inputs.make_dense(1, 1, 70, 70, 32, "f16", "normal", True, seed=7, cfg=102, scale=0.0)
    o, lse = G.run(w, out_f32=True)
    for i in (0, 1, 33, 69):
        assert np.max(np.abs(o[0, 0, i] - w.v64[0, 0, :i + 1].mean(axis=0))) <= 1e-3
        assert abs(lse[0, 0, i] - math.log(i + 1)) <= 1e-5


def test_one_hot_key_selects_value_row():
    w = inputs.make_dense(1, 1, 64, 64, 64, "f16", "normal", False, seed=8, cfg=103)
    q = np.zeros((1, 1, 64, 64), np.float32)
    k = np.zeros((1, 1, 64, 64), np.float32)
    perm = np.random.default_rng(0).permutation(64)
    for i in range(64):
        q[0, 0, i, i] = 8.0
        k[0, 0, perm[i], i] = 8.0   # score 64 * 0.125 = 8 vs 0 elsewhere
    w.q, w.k = q.astype(np.float16), k.astype(np.float16)
    w.scale = np.float32(1.0)
    o, _ = G.run(w, out_f32=True)
    assert np.max(np.abs(o[0, 0] - w.v64[0, 0, perm])) <= 1e-5


# --- memory safety, determinism, streams, errors -----------------------------

@pytest.mark.parametrize("dtype,d,varlen", [("f16", 64, False), ("bf16", 32, True),
                                            ("f16", 128, True), ("f32", 24, False)])
def test_guard_bands_untouched(dtype, d, varlen):
    """Outputs live inside larger buffers filled with a sentinel: the kernel
    must write exactly its rows and nothing around them."""
    if varlen:
        w = inputs.make_varlen([33, 1, 130], 2, d, dtype, "normal", True, seed=9, cfg=110)
        T = int(w.cu_seqlens[-1])
        oshape, lshape = (T, 2, d), (T, 2)
    else:
        w = inputs.make_dense(2, 2, 77, 77, d, dtype, "normal", True, seed=9, cfg=110)
        oshape, lshape = (2, 2, 77, d), (2, 2, 77)
    tdt = G.TORCH_DTYPE[dtype]
    pad = 4096
    n_o, n_l = int(np.prod(oshape)), int(np.prod(lshape))
    obuf = torch.full((pad + n_o + pad,), 7.0, dtype=tdt, device="cuda")
    lbuf = torch.full((pad + n_l + pad,), 7.0, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n_o].view(oshape)
    lse = lbuf[pad:pad + n_l].view(lshape)
    q, k, v = (G.to_device(x, dtype) for x in (w.q, w.k, w.v))
    import exact_attention_sdpa_amd as S
    code = {"f16": S.SDPA_F16, "bf16": S.SDPA_BF16, "f32": S.SDPA_F32}[dtype]
    cu = torch.from_numpy(w.cu_seqlens).cuda() if varlen else None
    S.sdpa_fwd(q, k, v, out, lse, w.B, 2, w.Nq, w.Nk, d, float(w.scale), 1, cu, code,
               S.SDPA_SAME, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for buf in (obuf, lbuf):
        assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0)
    assert torch.all(torch.isfinite(out.float())) and torch.all(torch.isfinite(lse))


def test_deterministic():
    w = inputs.make_dense(2, 4, 700, 700, 64, "bf16", "normal", True, seed=11, cfg=111)
    o1, l1 = G.run(w)
    o2, l2 = G.run(w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_side_stream_and_no_lse():
    w = inputs.make_dense(2, 2, 300, 300, 64, "f16", "normal", False, seed=12, cfg=112)
    s = torch.cuda.Stream()
    o, lse = G.run(w, with_lse=False, stream=s)
    assert lse is None
    ref, _ = _dense_ref(w)
    G.assert_parity(o, ref, "f16", "side stream")


def test_unsupported_raises():
    import exact_attention_sdpa_amd as S
    q = torch.zeros(1, 1, 8, 48, dtype=torch.float16, device="cuda")
    with pytest.raises(S.SdpaError):
        S.scaled_dot_product_attention(q, q, q)
    with pytest.raises(S.SdpaError):     # p must be below 1
        S.scaled_dot_product_attention(q[..., :32], q[..., :32], q[..., :32], dropout_p=1.0)
    with pytest.raises(S.SdpaError):     # dropout needs f16/bf16 inputs
        q32 = q[..., :32].float()
        S.scaled_dot_product_attention(q32, q32, q32, dropout_p=0.1)
    q32h = q[..., :32].contiguous()
    with pytest.raises(S.SdpaError):     # masks: bool, the input dtype or f32 only
        S.scaled_dot_product_attention(q32h, q32h, q32h,
                                       attn_mask=torch.ones(8, 8, dtype=torch.float64,
                                                            device="cuda"))
    with pytest.raises(S.SdpaError):     # a mask with dropout needs f16/bf16 inputs too
        q32 = q[..., :32].float()
        S.scaled_dot_product_attention(q32, q32, q32, dropout_p=0.1,
                                       attn_mask=torch.ones(8, 8, dtype=torch.bool,
                                                            device="cuda"))
    with pytest.raises(S.SdpaError):     # a mask that does not broadcast to [B,H,Nq,Nk]
        S.scaled_dot_product_attention(q32h, q32h, q32h,
                                       attn_mask=torch.ones(7, 8, dtype=torch.bool,
                                                            device="cuda"))


def test_out_buffer_is_written_or_refused():
    """out= on the general path (here f32 inputs, a 3-D tensor and a packed
    batch): a matching contiguous buffer is written and returned; any other
    buffer is refused rather than silently replaced."""
    import exact_attention_sdpa_amd as S
    w = inputs.make_dense(2, 1, 40, 40, 16, "f32", "normal", True, seed=13, cfg=113)
    q, k, v = (G.to_device(x, "f32")[:, 0] for x in (w.q, w.k, w.v))   # [B, N, d]
    buf = torch.full(q.shape, 9.0, device="cuda")
    res = S.scaled_dot_product_attention(q, k, v, is_causal=True, scale=float(w.scale), out=buf)
    torch.cuda.synchronize()
    assert res.data_ptr() == buf.data_ptr()
    ref, _ = _dense_ref(w)
    G.assert_parity(buf.double().cpu().numpy(), ref[:, 0], "f32", "out= f32 3-D")
    wv = inputs.make_varlen([5, 0, 33], 2, 32, "f16", "normal", False, seed=14, cfg=113)
    qv, kv, vv = (G.to_device(x, "f16") for x in (wv.q, wv.k, wv.v))
    cu = torch.from_numpy(wv.cu_seqlens).cuda()
    pbuf = torch.zeros(qv.shape, dtype=torch.float16, device="cuda")
    S.scaled_dot_product_attention(qv, kv, vv, cu_seqlens=cu, max_seqlen=33, out=pbuf)
    torch.cuda.synchronize()
    pref, _ = oracle.sdpa_fwd_varlen(wv.q64, wv.k64, wv.v64, wv.cu_seqlens, wv.scale, False)
    G.assert_parity(pbuf.double().cpu().numpy(), pref, "f16", "out= packed")
    for bad in (torch.empty(q.shape, dtype=torch.float16, device="cuda"),          # dtype
                torch.empty((2, 41, 16), device="cuda"),                           # shape
                torch.empty((2, 16, 40), device="cuda").transpose(1, 2)):          # layout
        with pytest.raises(S.SdpaError):
            S.scaled_dot_product_attention(q, k, v, is_causal=True, out=bad)

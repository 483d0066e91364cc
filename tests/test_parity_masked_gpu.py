"""GPU parity of the elementwise-mask forward (sdpa_fwd_masked) through the
C ABI, against the fp64 masked oracle (tolerances of tests/gpu_util.py).

The SDPA tutorial's functional call takes an ``attn_mask`` argument
("Fused implementations"; its CausalSelfAttention passes None); the reading
is the functional API's convention: a boolean mask selects the pairs that
take part, an additive one is added to the scaled scores.  Rows with no
finite score give zeros and lse = -inf.
"""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
import oracle
from exact_attention_sdpa_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _mask_tensor(m, kind, dtype):
    """Upload a generated mask: bool -> torch.bool, add -> its storage dtype."""
    if kind == "bool":
        return torch.from_numpy(m).cuda().bool()
    return G.to_device(m, dtype)


def _mask64(m, kind, dtype):
    if kind == "bool":
        return m, "bool"
    return inputs.storage_to_f64(m, dtype), "add"


def _check(w, m, kind, mdt, out_f32, what, mask_t=None, q=None, k=None, v=None, lse_rel=0.0):
    q = G.to_device(w.q, w.dtype) if q is None else q
    k = G.to_device(w.k, w.dtype) if k is None else k
    v = G.to_device(w.v, w.dtype) if v is None else v
    mt = _mask_tensor(m, kind, mdt) if mask_t is None else mask_t
    out, lse = sdpa.scaled_dot_product_attention(
        q, k, v, attn_mask=mt, is_causal=w.is_causal, scale=float(w.scale),
        out_dtype=torch.float32 if out_f32 else None, return_lse=True)
    torch.cuda.synchronize()
    m64, mk = _mask64(m, kind, mdt)
    ref, lref = oracle.sdpa_fwd_masked(w.q64, w.k64, w.v64, m64, mk, w.scale, w.is_causal)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    dead = np.isneginf(lref)
    assert np.array_equal(np.isneginf(l), dead), f"{what}: empty rows differ"
    assert np.all(o[dead] == 0.0), f"{what}: empty rows not zero"
    G.assert_parity(o, ref, w.dtype, what)
    lref0 = np.where(dead, 0.0, lref)
    err = np.abs(np.where(dead, 0.0, l) - lref0)
    bound = G.TOL[w.dtype][2] + lse_rel * np.abs(lref0)
    assert np.all(err <= bound), f"{what}: lse err {float(np.max(err / bound)):.3f} x bound"
    return out, lse


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add", "add_f32"])
def test_full_mask(dtype, d, causal, kind):
    # several query and key tiles, ragged tails, Nk not a multiple of 4
    B, H, Nq, Nk = 2, 3, 200, 333
    w = inputs.make_dense(B, H, Nq, Nk, d, dtype, "normal", causal, seed=d, cfg=40)
    mdt = "f32" if kind == "add_f32" else dtype
    m = inputs.make_attn_mask((B, H, Nq, Nk), "bool" if kind == "bool" else "add", keep=0.8,
                              seed=d + 7 * causal, cfg=41, dtype=mdt)
    _check(w, m, "bool" if kind == "bool" else "add", mdt, dtype == "bf16",
           f"{dtype} d{d} causal={causal} {kind}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add", "add_f32"])
def test_masked_one_group_grid(d, causal, kind):
    """The small grids above run the masked kernels with two key groups that
    merge their states; 130 units of two query tiles (N = 300) run the
    one-group ones, checked on sampled units (with their empty rows).  The
    output is f32: mask biases put a row's weight on few keys, so |O| reaches
    about 4.7, where one f16 rounding of the output alone is 2.3e-3, above
    the max-abs bound; f32 leaves the kernel's own arithmetic measured."""
    B, H, n = 1, 130, 300
    assert B * H * -(-n // 256) > 256
    w = inputs.make_dense(B, H, n, n, d, "f16", "normal", causal, seed=d + causal, cfg=53)
    mk = "bool" if kind == "bool" else "add"
    mdt = "f32" if kind == "add_f32" else "f16"
    m = inputs.make_attn_mask((B, H, n, n), mk, keep=0.8, seed=d + 5 * causal, cfg=54, dtype=mdt)
    q, k, v = (G.to_device(x, "f16") for x in (w.q, w.k, w.v))
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, attn_mask=_mask_tensor(m, kind, mdt),
                                                 is_causal=causal, scale=float(w.scale),
                                                 out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    o, l = out.double().cpu().numpy(), lse.double().cpu().numpy()
    for h in (0, 17, 64, H - 1):
        sl = lambda x: x[:, h:h + 1]
        m64, _ = _mask64(sl(m), kind, mdt)
        ref, lref = oracle.sdpa_fwd_masked(sl(w.q64), sl(w.k64), sl(w.v64), m64, mk, w.scale,
                                           causal)
        what = f"one group d{d} causal={causal} {kind} head {h}"
        dead = np.isneginf(lref)
        assert np.array_equal(np.isneginf(sl(l)), dead), f"{what}: empty rows differ"
        assert np.all(sl(o)[dead] == 0.0), f"{what}: empty rows not zero"
        G.assert_parity(sl(o), ref, "f16", what, np.where(dead, 0.0, sl(l)),
                        np.where(dead, 0.0, lref))


@pytest.mark.parametrize("shape", [(1, 1, 260, 256), (2, 1, 1, 256), (1, 3, 260, 256),
                                   (2, 3, 1, 256), (260, 256), (256,)])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_broadcast_masks(shape, kind):
    # Nk a multiple of 4: broadcast dims are read in place at stride 0
    B, H, Nq, Nk, d = 2, 3, 260, 256, 64
    w = inputs.make_dense(B, H, Nq, Nk, d, "f16", "normal", False, seed=3, cfg=42)
    m = inputs.make_attn_mask(shape, kind, keep=0.7, seed=len(shape), cfg=43, dtype="f16")
    full = np.broadcast_to(m.reshape((1,) * (4 - m.ndim) + m.shape), (B, H, Nq, Nk))
    _check(w, full, kind, "f16", False, f"broadcast {shape} {kind}",
           mask_t=_mask_tensor(m, kind, "f16"))


def test_key_padding_mask_matches_packed_sequences():
    # a padded dense batch with a key-padding mask: its valid rows equal the
    # packed (varlen) result of the same sequences
    lens = np.array([37, 128, 1, 200, 64])
    N, H, d = 200, 2, 64
    wv = inputs.make_varlen(lens, H, d, "f16", "normal", False, seed=5, cfg=44)
    B = len(lens)
    cu = wv.cu_seqlens
    qd = np.zeros((B, H, N, d), np.float16)
    kd, vd = qd.copy(), qd.copy()
    for b in range(B):
        s0, s1 = cu[b], cu[b + 1]
        qd[b, :, : s1 - s0] = wv.q[s0:s1].transpose(1, 0, 2)
        kd[b, :, : s1 - s0] = wv.k[s0:s1].transpose(1, 0, 2)
        vd[b, :, : s1 - s0] = wv.v[s0:s1].transpose(1, 0, 2)
    kp = torch.from_numpy(inputs.key_padding_mask(lens, N)).cuda().bool()
    out, lse = sdpa.scaled_dot_product_attention(
        *(torch.from_numpy(x).cuda() for x in (qd, kd, vd)), attn_mask=kp,
        return_lse=True)
    packed, plse = G.run(wv)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    for b in range(B):
        s0, s1 = cu[b], cu[b + 1]
        ref = packed[s0:s1].transpose(1, 0, 2)
        G.assert_parity(o[b, :, : s1 - s0], ref, "f16", f"seq {b}", l[b, :, : s1 - s0],
                        plse[s0:s1].T)


@pytest.mark.parametrize("causal", [False, True])
def test_empty_and_late_rows(causal):
    # rows whose every key is dropped (O = 0, lse = -inf); rows whose first
    # visible key is far into the sequence (the softmax reference is set
    # late); rows seeing a single key
    B, H, Nq, Nk, d = 1, 2, 300, 300, 64
    w = inputs.make_dense(B, H, Nq, Nk, d, "f16", "normal", causal, seed=9, cfg=45)
    m = np.ones((B, H, Nq, Nk), np.uint8)
    m[:, :, 5] = 0                      # empty row
    m[:, :, 250:260, :200] = 0          # first visible key at 200
    m[:, :, 100, :] = 0
    m[:, :, 100, 37] = 1                # one key only
    m[:, 1, 299, :] = 0                 # last row of one head empty
    _check(w, m, "bool", "f16", False, f"empty/late rows causal={causal}")


def test_large_additive_offsets():
    # a soft mask with large finite offsets per row: the result depends only
    # on differences within a row
    B, H, Nq, Nk, d = 1, 2, 130, 257, 32
    w = inputs.make_dense(B, H, Nq, Nk, d, "f16", "normal", False, seed=11, cfg=46)
    rng = np.random.default_rng(0)
    a = (rng.standard_normal((B, H, Nq, Nk)) * 3).astype(np.float32)
    a += (rng.integers(-3, 4, (B, H, Nq, 1)) * 1000).astype(np.float32)
    a[:, :, :, ::3] = -1.0e4            # soft-masked keys
    # lse ~ 3000 here, where one fp32 ulp is 2.4e-4: the kernel's lse passes
    # through two fp32 roundings at that magnitude (the row reference in
    # log2 units and the final product), so its bound grows by 2^-21 |lse|
    _check(w, a, "add", "f32", False, "large offsets", lse_rel=2.0 ** -21)


def test_cross_attention_and_module_layout():
    # Nq != Nk, and q/k/v as views of one packed projection (read in place)
    B, H, Nq, d = 2, 4, 150, 64
    E = H * d
    g = torch.Generator().manual_seed(3)
    x = torch.randn(B, Nq, 3 * E, generator=g).half().cuda()
    qv, kv_, vv = (t.view(B, Nq, H, d).transpose(1, 2) for t in x.chunk(3, -1))
    m = inputs.make_attn_mask((B, 1, Nq, Nq), "bool", keep=0.6, seed=1, cfg=47)
    mt = torch.from_numpy(m).cuda().bool()
    out, lse = sdpa.scaled_dot_product_attention(qv, kv_, vv, attn_mask=mt, is_causal=True,
                                                 return_lse=True)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    ref, lref = oracle.sdpa_fwd_masked(f(qv), f(kv_), f(vv), m, "bool", 1.0 / np.sqrt(d), True)
    dead = np.isneginf(lref)
    G.assert_parity(f(out), ref, "f16", "module layout", np.where(dead, 0, f(lse)),
                    np.where(dead, 0, lref))
    # cross-attention: fewer keys than queries
    Nk = 77
    w = inputs.make_dense(B, H, Nq, Nk, d, "bf16", "normal", False, seed=4, cfg=48)
    mm = inputs.make_attn_mask((B, H, Nq, Nk), "add", keep=0.9, seed=2, cfg=49, dtype="bf16")
    _check(w, mm, "add", "bf16", True, "cross bf16")


def test_three_dim_inputs():
    # [B, N, d] inputs (one head) with a [B, Nq, Nk] mask
    B, Nq, Nk, d = 3, 70, 90, 32
    w = inputs.make_dense(B, 1, Nq, Nk, d, "f16", "normal", False, seed=6, cfg=50)
    m = inputs.make_attn_mask((B, Nq, Nk), "bool", keep=0.5, seed=6, cfg=51)
    q, k, v = (G.to_device(x[:, 0], "f16") for x in (w.q, w.k, w.v))
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(m).cuda()
                                                 .bool(), return_lse=True)
    torch.cuda.synchronize()
    ref, lref = oracle.sdpa_fwd_masked(w.q64, w.k64, w.v64, m[:, None], "bool", w.scale, False)
    dead = np.isneginf(lref[:, 0])
    G.assert_parity(out.double().cpu().numpy(), ref[:, 0], "f16", "3-D",
                    np.where(dead, 0, lse.double().cpu().numpy()), np.where(dead, 0, lref[:, 0]))


def test_all_true_mask_matches_plain_kernel():
    B, H, N, d = 2, 2, 300, 64
    w = inputs.make_dense(B, H, N, N, d, "f16", "normal", True, seed=8, cfg=52)
    q, k, v = (G.to_device(x, "f16") for x in (w.q, w.k, w.v))
    ones = torch.ones((N, N), dtype=torch.bool, device="cuda")
    a, la = sdpa.scaled_dot_product_attention(q, k, v, attn_mask=ones, is_causal=True,
                                              return_lse=True)
    b, lb = sdpa.scaled_dot_product_attention(q, k, v, is_causal=True, return_lse=True)
    torch.cuda.synchronize()
    G.assert_parity(a.double().cpu().numpy(), b.double().cpu().numpy(), "f16", "all-true",
                    la.double().cpu().numpy(), lb.double().cpu().numpy())


@pytest.mark.parametrize("cfg", [7, 8])
def test_bench_workloads_sampled_units(cfg):
    # the masked and padded workloads at full size, in the launch the
    # benchmark times (sdpa_fwd_masked, same mask layout and output type);
    # whole (batch, head) units sampled against the fp64 oracle
    w = inputs.make_config(cfg)
    q, k, v = (G.to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    m = w.attn_mask
    mt = (torch.from_numpy(m).cuda().bool() if w.mask_kind == "bool"
          else G.to_device(m, w.dtype))
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, attn_mask=mt, is_causal=w.is_causal,
                                                 scale=float(w.scale), return_lse=True)
    torch.cuda.synchronize()
    m4 = m.reshape((1,) * (4 - m.ndim) + m.shape)
    rng = np.random.default_rng(cfg)
    units = [(0, 0), (w.B - 1, w.H - 1)] + [tuple(x) for x in
                                           zip(rng.integers(0, w.B, 4), rng.integers(0, w.H, 4))]
    for b, h in units:
        mu = m4[b % m4.shape[0], h % m4.shape[1]]
        mu = mu if w.mask_kind == "bool" else inputs.storage_to_f64(mu, w.dtype)
        mu = np.broadcast_to(mu, (w.Nq, w.Nk))[None, None]
        sl = lambda x: x[b:b + 1, h:h + 1]
        ref, lref = oracle.sdpa_fwd_masked(sl(w.q64), sl(w.k64), sl(w.v64), mu, w.mask_kind,
                                           w.scale, w.is_causal)
        G.assert_parity(out[b:b + 1, h:h + 1].double().cpu().numpy(), ref, w.dtype,
                        f"{w.name} unit ({b}, {h})", lse[b:b + 1, h:h + 1].double().cpu().numpy(),
                        lref)

"""GPU parity of the strided forward (sdpa_fwd_strided) through the C ABI.

The SDPA tutorial's CausalSelfAttention ("Causal self-attention") takes q,
k, v as views of one packed projection: c_attn(x) [B, N, 3E], chunked in
three along the last dim and viewed as [B, H, N, d] (strides (3NE, d, 3E,
1)); its output is transposed back to [B, N, E].  These tests read such
views in place and write the output straight into a [B, N, E] buffer, and
check against the fp64 oracle on contiguous copies (tolerances of
tests/gpu_util.py) and bit for bit against the contiguous path, which runs
the same arithmetic.
"""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
import oracle
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16}


def _packed_qkv(B, N, H, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    E = H * d
    x = torch.randn(B, N, 3 * E, generator=g).to(TD[dtype]).cuda()
    q, k, v = x.chunk(3, -1)
    view = lambda t: t.view(B, N, H, d).transpose(1, 2)
    return x, view(q), view(k), view(v)


def _ref(q, k, v, scale, causal):
    f = lambda t: t.double().cpu().numpy()
    return oracle.sdpa_fwd(f(q), f(k), f(v), scale, causal)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_module_layout_in_place(dtype, d, causal):
    B, N, H = 2, 200, 4
    x, q, k, v = _packed_qkv(B, N, H, d, dtype, seed=d + causal)
    assert not q.is_contiguous() and q.stride() == (N * 3 * H * d, d, 3 * H * d, 1)
    odt = torch.float32 if dtype == "bf16" else TD[dtype]
    y = torch.full((B, N, H * d), float("nan"), dtype=odt, device="cuda")
    yv = y.view(B, N, H, d).transpose(1, 2)
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, is_causal=causal, out=yv,
                                                 out_dtype=odt, return_lse=True)
    torch.cuda.synchronize()
    assert out.data_ptr() == y.data_ptr()
    ref, lref = _ref(q, k, v, 1.0 / np.sqrt(d), causal)
    # y holds the module's y.transpose(1, 2).view(B, N, E) directly
    got = y.double().cpu().numpy().reshape(B, N, H, d).transpose(0, 2, 1, 3)
    G.assert_parity(got, ref, dtype, f"{dtype} d{d} causal={causal}", lse.double().cpu().numpy(),
                    lref)
    # the same bits as the contiguous path
    oc, lc = sdpa.scaled_dot_product_attention(q.contiguous(), k.contiguous(), v.contiguous(),
                                               is_causal=causal, out_dtype=odt, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, oc) and torch.equal(lse, lc)


@pytest.mark.parametrize("causal", [False, True])
def test_padded_rows_and_separate_kv_strides(causal):
    B, H, Nq, Nk, d = 2, 3, 130, 257, 64
    g = torch.Generator().manual_seed(6 + causal)
    base_q = torch.randn(B, H, Nq, d + 24, generator=g).half().cuda()     # row stride 88
    base_kv = torch.randn(H, B, Nk, 2, d + 8, generator=g).half().cuda()  # k, v interleaved per row
    q = base_q[..., :d]
    k = base_kv[:, :, :, 0, :d].transpose(0, 1)
    v = base_kv[:, :, :, 1, :d].transpose(0, 1)
    assert k.stride() == v.stride() and q.stride()[2] == d + 24
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, is_causal=causal,
                                                 out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ref, lref = _ref(q, k, v, 1.0 / np.sqrt(d), causal)
    G.assert_parity(out.double().cpu().numpy(), ref, "f16", f"padded causal={causal}",
                    lse.double().cpu().numpy(), lref)


def test_unaligned_views_are_copied_not_misread():
    # seeded; an f32 output, so that the check is of the reading, not of one
    # f16 rounding of |O| up to ~8 (q = k makes one key dominate each row)
    B, H, N, d = 1, 2, 64, 64
    g = torch.Generator().manual_seed(5)
    base = torch.randn(B, H, N, d + 4, generator=g).half().cuda()   # row stride 68: not a multiple of 8
    q = base[..., :d]
    out = sdpa.scaled_dot_product_attention(q, q, q, out_dtype=torch.float32)
    ref, _ = _ref(q, q, q, 1.0 / np.sqrt(d), False)
    torch.cuda.synchronize()
    G.assert_parity(out.double().cpu().numpy(), ref, "f16", "copied view")


def test_bad_out_view_raises():
    q = torch.randn(1, 2, 64, 64).half().cuda()
    with pytest.raises(sdpa.SdpaError):   # overlapping output rows
        o = torch.empty(1, 2, 64, 64, dtype=torch.float16, device="cuda").as_strided(
            (1, 2, 64, 64), (0, 8, 8, 1))
        sdpa.scaled_dot_product_attention(q, q, q, out=o)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_out_rows_at_eight_byte_alignment(dtype, d):
    """A 16-bit output whose row stride is a multiple of 4 elements but not
    of 8 (the ABI's minimum): its rows start 8 bytes off a 16-byte boundary.
    The kernel's row-segment stores must land exactly in the view, leaving
    the padding columns between the rows untouched, and give the bits of the
    contiguous path."""
    B, H, N = 2, 3, 300
    g = torch.Generator().manual_seed(d)
    q, k, v = (torch.randn(B, H, N, d, generator=g).to(TD[dtype]).cuda() for _ in range(3))
    base = torch.full((B, H, N, d + 4), float("nan"), dtype=TD[dtype], device="cuda")
    yv = base[..., :d]
    assert yv.stride()[2] % 8 == 4
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, out=yv, return_lse=True)
    oc, lc = sdpa.scaled_dot_product_attention(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    assert out.data_ptr() == base.data_ptr()
    assert torch.equal(yv, oc) and torch.equal(lse, lc)
    assert torch.isnan(base[..., d:]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_wide_d32_grid_in_place_and_cross(causal):
    """d = 32 grids of at least 2048 query tiles (the kernels with two query
    blocks per wave) read the packed-QKV views in place and write the
    module's layout, with the same bits as the contiguous path; and a
    cross-attention grid (Nq != Nk) of that size matches the oracle on
    sampled units."""
    B, N, H, d = 64, 250, 32, 32
    x, q, k, v = _packed_qkv(B, N, H, d, "f16", seed=11 + causal)
    assert B * H * -(-N // 256) >= 2048
    y = torch.full((B, N, H * d), float("nan"), dtype=torch.float16, device="cuda")
    yv = y.view(B, N, H, d).transpose(1, 2)
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, is_causal=causal, out=yv,
                                                 return_lse=True)
    oc, lc = sdpa.scaled_dot_product_attention(q.contiguous(), k.contiguous(), v.contiguous(),
                                               is_causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, oc) and torch.equal(lse, lc)
    units = [(0, 0), (B - 1, H - 1), (17, 5), (40, 30)]
    for b, h in units:
        ref, lref = _ref(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                         1.0 / np.sqrt(d), causal)
        G.assert_parity(out[b:b + 1, h:h + 1].double().cpu().numpy(), ref, "f16",
                        f"wide in place unit {b},{h}", lse[b:b + 1, h:h + 1].double().cpu().numpy(),
                        lref)
    # cross attention: 250 queries, 600 keys
    g = torch.Generator().manual_seed(21 + causal)
    qx = torch.randn(B, H, 250, d, generator=g).half().cuda()
    kx = torch.randn(B, H, 600, d, generator=g).half().cuda()
    vx = torch.randn(B, H, 600, d, generator=g).half().cuda()
    ox, lx = sdpa.scaled_dot_product_attention(qx, kx, vx, is_causal=causal, return_lse=True)
    torch.cuda.synchronize()
    for b, h in units:
        ref, lref = _ref(qx[b:b + 1, h:h + 1], kx[b:b + 1, h:h + 1], vx[b:b + 1, h:h + 1],
                         1.0 / np.sqrt(d), causal)
        G.assert_parity(ox[b:b + 1, h:h + 1].double().cpu().numpy(), ref, "f16",
                        f"wide cross unit {b},{h}", lx[b:b + 1, h:h + 1].double().cpu().numpy(),
                        lref)

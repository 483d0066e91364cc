"""The allocation-free backward (sdpa_bwd_noalloc) through the C ABI: the
same gradients, bit for bit, as sdpa_bwd with a caller workspace, on two
calls in a row, the second smaller than the first (the library's device
array keeps the first call's row dots, which the second must not read)."""
import numpy as np
import pytest
import torch

import exact_attention_sdpa_amd as sdpa
from exact_attention_sdpa_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CODE = {"f16": sdpa.SDPA_F16, "bf16": sdpa.SDPA_BF16}


def _grads(w, do, noalloc, grad_f32):
    dt = CODE[w.dtype]
    q, k, v = (G.to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    out, lse = sdpa.scaled_dot_product_attention(q, k, v, is_causal=w.is_causal,
                                                 scale=float(w.scale), return_lse=True)
    dout = G.to_device(do, w.dtype)
    gdt = torch.float32 if grad_f32 else q.dtype
    dq = torch.full(q.shape, float("nan"), dtype=gdt, device="cuda")
    dk = torch.full(k.shape, float("nan"), dtype=gdt, device="cuda")
    dv = torch.full(v.shape, float("nan"), dtype=gdt, device="cuda")
    gcode = sdpa.SDPA_F32 if grad_f32 else sdpa.SDPA_SAME
    stream = torch.cuda.current_stream()
    args = (w.B, w.H, w.Nq, w.Nk, w.d, float(w.scale), int(w.is_causal), dt, sdpa.SDPA_SAME,
            gcode, stream)
    if noalloc:
        sdpa.sdpa_bwd_noalloc(q, k, v, out, dout, lse, dq, dk, dv, *args)
    else:
        ws = torch.empty(sdpa.sdpa_bwd_workspace_bytes(w.B, w.H, w.Nq) // 4,
                         dtype=torch.float32, device="cuda")
        sdpa.sdpa_bwd(q, k, v, out, dout, lse, dq, dk, dv, ws, *args)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (dq, dk, dv)]


def test_noalloc_backward_matches_sdpa_bwd_on_two_calls():
    cases = [  # the second call is smaller than the first
        (inputs.make_dense(2, 3, 300, 300, 64, "f16", "normal", True, seed=1, cfg=130), False),
        (inputs.make_dense(1, 2, 77, 77, 32, "bf16", "normal", False, seed=2, cfg=130), True),
    ]
    for w, gf32 in cases:
        print(f"noalloc case {w.dtype} B{w.B} H{w.H} N{w.Nq} d{w.d} causal={w.is_causal}",
              flush=True)
        do = inputs.make_grad_out(w, seed=3, cfg=130)
        want = _grads(w, do, noalloc=False, grad_f32=gf32)
        got = _grads(w, do, noalloc=True, grad_f32=gf32)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert np.all(np.isfinite(a)), name
            assert np.array_equal(a, b), f"{name}: max diff {float(np.max(np.abs(a - b)))}"


def test_noalloc_backward_refuses_oversized_calls():
    z = torch.zeros(16, dtype=torch.float16, device="cuda")
    rows = sdpa._lib.SDPA_BWD_NOALLOC_MAX_ROWS
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.sdpa_bwd_noalloc(z, z, z, z, z, z.float(), z, z, z, 1, 1, rows + 1, 16, 64, 0.125,
                              0, sdpa.SDPA_F16, sdpa.SDPA_SAME, sdpa.SDPA_SAME, None)
    assert e.value.status == sdpa.SDPA_ERR_UNSUPPORTED

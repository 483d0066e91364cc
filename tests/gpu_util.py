"""Helpers shared by the GPU tests: moving seeded workloads to the device,
running the HIP path through the binding, and the parity metrics.

Tolerances (written here once, used by every parity test):
  f16/bf16 inputs, f16/f32 output: max-abs <= 2e-3 and rel-L2 <= 1e-3
      against the fp64 oracle (fp32 accumulation on the matrix cores).
  f32 inputs: max-abs <= 1e-5 and rel-L2 <= 1e-5.
  lse: |err| <= 1e-4 (f16/bf16), 1e-5 (f32).
  bf16 output: one bf16 rounding of the result on top of the f16/bf16
      bound, i.e. |err| <= 2e-3 + 2^-8 |O_ref| elementwise.
rel-L2 = ||O_gpu - O_ref||_2 / ||O_ref||_2 over all compared elements.
"""
from __future__ import annotations

import numpy as np
import torch

import exact_attention_sdpa_amd as sdpa

TOL = {"f16": (2e-3, 1e-3, 1e-4), "bf16": (2e-3, 1e-3, 1e-4), "f32": (1e-5, 1e-5, 1e-5)}

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Upload stored values bit for bit (bf16 arrives as uint16 patterns)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def run(w, out_f32=False, with_lse=True, stream=None):
    """Run the HIP path on workload ``w``; returns (out, lse) as float64 numpy."""
    q, k, v = (to_device(x, w.dtype) for x in (w.q, w.k, w.v))
    cu = None
    if w.varlen:
        cu = torch.from_numpy(w.cu_seqlens).to("cuda")
    res = sdpa.scaled_dot_product_attention(
        q, k, v, is_causal=w.is_causal, scale=float(w.scale), cu_seqlens=cu,
        max_seqlen=w.Nq if w.varlen else None,
        out_dtype=torch.float32 if out_f32 else None, return_lse=with_lse, stream=stream)
    if stream is not None:
        stream.synchronize()
    else:
        torch.cuda.synchronize()
    out, lse = res if with_lse else (res, None)
    o64 = out.to(torch.float64).cpu().numpy()
    l64 = lse.to(torch.float64).cpu().numpy() if lse is not None else None
    return o64, l64


def metrics(o, ref):
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = o - ref
    nref = np.linalg.norm(ref)
    return {"max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
            "rel_l2": float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff)),
            "finite": bool(np.all(np.isfinite(o)))}


def assert_parity(o, ref, dtype, what="", lse=None, lse_ref=None, bf16_out=False):
    max_abs_tol, rel_tol, lse_tol = TOL[dtype]
    m = metrics(o, ref)
    assert m["finite"], f"{what}: non-finite output"
    if bf16_out:
        bound = 2e-3 + 2.0 ** -8 * np.abs(ref)
        worst = float(np.max(np.abs(np.asarray(o) - ref) / bound))
        assert worst <= 1.0, f"{what}: bf16 output error {worst:.3f} x bound"
    else:
        assert m["max_abs"] <= max_abs_tol, f"{what}: max-abs {m['max_abs']:.3e} > {max_abs_tol}"
        assert m["rel_l2"] <= rel_tol, f"{what}: rel-L2 {m['rel_l2']:.3e} > {rel_tol}"
    if lse is not None:
        e = float(np.max(np.abs(lse - lse_ref)))
        assert e <= lse_tol, f"{what}: lse err {e:.3e} > {lse_tol}"
    return m

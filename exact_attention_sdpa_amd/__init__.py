"""MI355X-native fused exact attention forward.

Thin Python binding of the C ABI in include/sdpa.h: argument marshalling
only.  Every step of the computation runs in the HIP kernels of
libsdpa.so; PyTorch supplies device memory and the current stream.

``sdpa_fwd`` mirrors the C entry point one to one.  ``scaled_dot_product_
attention`` is the functional form of the PyTorch SDPA tutorial ("Fused
implementations"): it allocates the output (and optionally the logsumexp)
and calls ``sdpa_fwd`` on the current stream.
"""
from __future__ import annotations

import math
import warnings

from . import _lib
from ._lib import (SDPA_BF16, SDPA_ERR_DEVICE, SDPA_ERR_INVALID, SDPA_ERR_LAUNCH,  # noqa: F401
                   SDPA_ERR_UNSUPPORTED, SDPA_F16, SDPA_F32, SDPA_OK, SDPA_SAME)

__all__ = ["sdpa_fwd", "sdpa_supports", "sdpa_status_str", "sdpa_abi_version",
           "scaled_dot_product_attention", "SdpaError"]


class SdpaError(RuntimeError):
    """A non-OK status from the C ABI (message names the status)."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(f"sdpa_fwd: {sdpa_status_str(status)} (status {status})")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def sdpa_fwd(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal, cu_seqlens, dtype,
             out_dtype, stream):
    """Call the C entry point.  Pointer arguments may be torch tensors or
    integers (device addresses); ``stream`` a torch stream, an integer
    handle or None.  Raises SdpaError on a non-OK status."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H),
                             int(Nq), int(Nk), int(d), float(scale), int(is_causal),
                             _ptr(cu_seqlens), int(dtype), int(out_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_supports(dtype: int, d: int, is_causal: bool = False, varlen: bool = False) -> int:
    return _lib.lib().sdpa_supports(int(dtype), int(d), int(is_causal), int(varlen))


def sdpa_status_str(status: int) -> str:
    return _lib.lib().sdpa_status_str(int(status)).decode()


def sdpa_abi_version() -> int:
    return _lib.lib().sdpa_abi_version()


def _code(dt):
    import torch
    codes = {torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16, torch.float32: SDPA_F32}
    if dt not in codes:
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    return codes[dt]


_warned_copy = False


def _contig(t):
    global _warned_copy
    if t.is_contiguous():
        return t
    if not _warned_copy:
        warnings.warn("sdpa: non-contiguous input copied to a contiguous buffer")
        _warned_copy = True
    return t.contiguous()


def scaled_dot_product_attention(query, key, value, attn_mask=None, dropout_p=0.0,
                                 is_causal=False, scale=None, cu_seqlens=None,
                                 max_seqlen=None, out_dtype=None, return_lse=False,
                                 stream=None):
    """Attention forward on device tensors.

    Dense: query [B,H,Nq,d] (or [B,Nq,d], read as H=1), key/value
    [B,H,Nk,d].  Packed (cu_seqlens, an int32 device tensor of B+1 offsets,
    with max_seqlen): query/key/value [T,H,d].  ``out_dtype`` None keeps the
    input dtype; torch.float32 requests an f32 output.  Returns out, or
    (out, lse) with ``return_lse``.  A mask or dropout is not supported and
    raises, as the tutorial's backends do for inputs they cannot serve."""
    import torch
    if attn_mask is not None:
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if dropout_p != 0.0:
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if not (query.dtype == key.dtype == value.dtype):
        raise SdpaError(SDPA_ERR_INVALID)
    if not (query.is_cuda and key.is_cuda and value.is_cuda):
        raise SdpaError(SDPA_ERR_INVALID)
    q, k, v = _contig(query), _contig(key), _contig(value)
    dt = _code(q.dtype)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in (q.dtype, torch.float32):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    out = torch.empty(q.shape, dtype=odt, device=q.device)
    squeeze = False
    if cu_seqlens is not None:
        if q.dim() != 3 or max_seqlen is None:
            raise SdpaError(SDPA_ERR_INVALID)
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
            raise SdpaError(SDPA_ERR_INVALID)
        T, H, _ = q.shape
        B = cu_seqlens.numel() - 1
        Nq = Nk = int(max_seqlen)
        if k.shape != q.shape or v.shape != q.shape:
            raise SdpaError(SDPA_ERR_INVALID)
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if return_lse else None
    else:
        if q.dim() == 3:
            q, k, v, out = q[:, None], k[:, None], v[:, None], out[:, None]
            squeeze = True
        if q.dim() != 4:
            raise SdpaError(SDPA_ERR_INVALID)
        B, H, Nq, _ = q.shape
        Nk = k.shape[2]
        if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
            raise SdpaError(SDPA_ERR_INVALID)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if return_lse else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        sdpa_fwd(q, k, v, out, lse, B, H, Nq, Nk, d, scale, bool(is_causal), cu_seqlens, dt,
                 _code(odt) if odt != q.dtype else SDPA_SAME, stream)
    if squeeze:
        out = out[:, 0]
        if lse is not None:
            lse = lse[:, 0]
    return (out, lse) if return_lse else out

"""MI355X-native fused exact attention, forward and backward.

Thin Python binding of the C ABI in include/sdpa.h: argument marshalling
only.  Every step of the computation runs in the HIP kernels of
libsdpa.so; PyTorch supplies device memory and the current stream.

``sdpa_fwd`` and ``sdpa_bwd`` mirror the C entry points one to one.
``scaled_dot_product_attention`` is the functional form of the PyTorch SDPA
tutorial ("Fused implementations"): it allocates the output (and optionally
the logsumexp) and calls ``sdpa_fwd`` on the current stream.
``scaled_dot_product_attention_backward`` allocates the gradients and calls
``sdpa_bwd``; ``attention`` wraps both in a torch.autograd.Function.
"""
from __future__ import annotations

import math
import warnings

from . import _lib
from ._lib import (SDPA_BF16, SDPA_BLOCK_SPARSE_BLOCK, SDPA_ERR_DEVICE,  # noqa: F401
                   SDPA_ERR_INVALID, SDPA_ERR_LAUNCH, SDPA_ERR_UNSUPPORTED, SDPA_F16, SDPA_F32,
                   SDPA_MASK_ADD, SDPA_MASK_ADD_F32, SDPA_MASK_BOOL, SDPA_OK, SDPA_SAME)

__all__ = ["sdpa_fwd", "sdpa_fwd_strided", "sdpa_fwd_masked", "sdpa_fwd_masked_dropout", "sdpa_fwd_block_sparse", "sdpa_fwd_dropout", "sdpa_bwd", "sdpa_bwd_dropout", "sdpa_bwd_packed", "sdpa_bwd_masked", "sdpa_bwd_masked_dropout", "sdpa_bwd_block_sparse", "sdpa_bwd_noalloc", "sdpa_bwd_workspace_bytes", "sdpa_supports",
           "sdpa_status_str", "sdpa_abi_version", "scaled_dot_product_attention",
           "scaled_dot_product_attention_backward", "attention", "SdpaError"]


class SdpaError(RuntimeError):
    """A non-OK status from the C ABI (message names the status)."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(f"sdpa: {sdpa_status_str(status)} (status {status})")


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


def sdpa_fwd_strided(q, k, v, out, lse, B, H, Nq, Nk, d, q_strides, kv_strides, out_strides,
                     scale, is_causal, dtype, out_dtype, stream):
    """Call the strided C entry point; strides are 3-sequences of element
    strides (batch, head, row)."""
    import ctypes
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    arr = lambda s: (ctypes.c_int64 * 3)(*[int(x) for x in s])
    qs, ks, os_ = arr(q_strides), arr(kv_strides), arr(out_strides)
    st = _lib.lib().sdpa_fwd_strided(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
        int(d), ctypes.cast(qs, ctypes.c_void_p), ctypes.cast(ks, ctypes.c_void_p),
        ctypes.cast(os_, ctypes.c_void_p), float(scale), int(is_causal), int(dtype),
        int(out_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_fwd_masked(q, k, v, out, lse, B, H, Nq, Nk, d, q_strides, kv_strides, out_strides,
                    scale, is_causal, mask, mask_kind, mask_strides, dtype, out_dtype, stream):
    """Call the masked C entry point.  q/kv/out strides: all None
    (contiguous) or 3-sequences of element strides; mask_strides a
    3-sequence (batch, head, row)."""
    import ctypes
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    keep = []

    def arr(s):
        if s is None:
            return None
        a = (ctypes.c_int64 * 3)(*[int(x) for x in s])
        keep.append(a)
        return ctypes.cast(a, ctypes.c_void_p)

    st = _lib.lib().sdpa_fwd_masked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
        int(d), arr(q_strides), arr(kv_strides), arr(out_strides), float(scale),
        int(is_causal), _ptr(mask), int(mask_kind), arr(mask_strides), int(dtype),
        int(out_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_fwd_masked_dropout(q, k, v, out, lse, B, H, Nq, Nk, d, q_strides, kv_strides,
                            out_strides, scale, is_causal, mask, mask_kind, mask_strides,
                            dropout_p, seed, offset, dtype, out_dtype, stream):
    """Call the masked-dropout C entry point (arguments as sdpa_fwd_masked
    and sdpa_fwd_dropout)."""
    import ctypes
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    keep = []

    def arr(s):
        if s is None:
            return None
        a = (ctypes.c_int64 * 3)(*[int(x) for x in s])
        keep.append(a)
        return ctypes.cast(a, ctypes.c_void_p)

    st = _lib.lib().sdpa_fwd_masked_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
        int(d), arr(q_strides), arr(kv_strides), arr(out_strides), float(scale),
        int(is_causal), _ptr(mask), int(mask_kind), arr(mask_strides), float(dropout_p),
        int(seed), int(offset), int(dtype), int(out_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_fwd_block_sparse(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal, block_mask,
                          mask_heads, dtype, out_dtype, stream):
    """Call the block-sparse C entry point (same conventions as sdpa_fwd)."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_fwd_block_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
        int(d), float(scale), int(is_causal), _ptr(block_mask), int(mask_heads), int(dtype),
        int(out_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_fwd_dropout(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal, cu_seqlens,
                     dropout_p, seed, offset, dtype, out_dtype, stream):
    """Call the dropout C entry point (same conventions as sdpa_fwd)."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_fwd_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
        int(d), float(scale), int(is_causal), _ptr(cu_seqlens), float(dropout_p), int(seed),
        int(offset), int(dtype), int(out_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
             is_causal, dtype, out_dtype, grad_dtype, stream):
    """Call the C backward entry point (same conventions as sdpa_fwd)."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), int(B), int(H),
                             int(Nq), int(Nk), int(d), float(scale), int(is_causal), int(dtype),
                             int(out_dtype), int(grad_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd_noalloc(q, k, v, out, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, is_causal,
                     dtype, out_dtype, grad_dtype, stream):
    """Call the allocation-free backward entry point (sdpa_bwd without a
    workspace: the row dots live in the library's per-device array)."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), int(B), int(H), int(Nq),
                                     int(Nk), int(d), float(scale), int(is_causal), int(dtype),
                                     int(out_dtype), int(grad_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd_dropout(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                     is_causal, dropout_p, seed, offset, dtype, out_dtype, grad_dtype, stream):
    """Call the dropout backward C entry point (same conventions as sdpa_fwd)."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_bwd_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), int(B), int(H), int(Nq), int(Nk), int(d), float(scale),
        int(is_causal), float(dropout_p), int(seed), int(offset), int(dtype), int(out_dtype),
        int(grad_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd_packed(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, T, max_seqlen, d,
                    scale, is_causal, cu_seqlens, dropout_p, seed, offset, dtype, out_dtype,
                    grad_dtype, stream):
    """Call the packed-batch backward C entry point (same conventions as
    sdpa_fwd; dropout_p 0 for none)."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_bwd_packed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), int(B), int(H), int(T), int(max_seqlen), int(d), float(scale),
        int(is_causal), _ptr(cu_seqlens), float(dropout_p), int(seed), int(offset), int(dtype),
        int(out_dtype), int(grad_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd_masked(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                    is_causal, mask, mask_kind, mask_strides, dtype, out_dtype, grad_dtype,
                    stream):
    """Call the masked backward C entry point (mask_strides a 3-sequence:
    batch, head, row)."""
    import ctypes
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    ms = (ctypes.c_int64 * 3)(*[int(x) for x in mask_strides])
    st = _lib.lib().sdpa_bwd_masked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), int(B), int(H), int(Nq), int(Nk), int(d), float(scale),
        int(is_causal), _ptr(mask), int(mask_kind), ctypes.cast(ms, ctypes.c_void_p), int(dtype),
        int(out_dtype), int(grad_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd_masked_dropout(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d,
                            scale, is_causal, mask, mask_kind, mask_strides, dropout_p, seed,
                            offset, dtype, out_dtype, grad_dtype, stream):
    """Call the masked-dropout backward C entry point."""
    import ctypes
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    ms = (ctypes.c_int64 * 3)(*[int(x) for x in mask_strides])
    st = _lib.lib().sdpa_bwd_masked_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), int(B), int(H), int(Nq), int(Nk), int(d), float(scale),
        int(is_causal), _ptr(mask), int(mask_kind), ctypes.cast(ms, ctypes.c_void_p),
        float(dropout_p), int(seed), int(offset), int(dtype), int(out_dtype), int(grad_dtype),
        stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd_block_sparse(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d,
                          scale, is_causal, block_mask, mask_heads, dtype, out_dtype,
                          grad_dtype, stream):
    """Call the block-sparse backward C entry point."""
    if stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    st = _lib.lib().sdpa_bwd_block_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), int(B), int(H), int(Nq), int(Nk), int(d), float(scale),
        int(is_causal), _ptr(block_mask), int(mask_heads), int(dtype), int(out_dtype),
        int(grad_dtype), stream)
    if st != SDPA_OK:
        raise SdpaError(st)


def sdpa_bwd_workspace_bytes(B: int, H: int, Nq: int) -> int:
    return int(_lib.lib().sdpa_bwd_workspace_bytes(int(B), int(H), int(Nq)))


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
                                 stream=None, block_mask=None, dropout_seed=None,
                                 dropout_offset=0, out=None):
    """Attention forward on device tensors.

    Dense: query [B,H,Nq,d] (or [B,Nq,d], read as H=1), key/value
    [B,H,Nk,d].  Packed (cu_seqlens, an int32 device tensor of B+1 offsets,
    with max_seqlen): query/key/value [T,H,d].  ``out_dtype`` None keeps the
    input dtype; torch.float32 requests an f32 output.  Returns out, or
    (out, lse) with ``return_lse``.  ``block_mask`` (dense layouts only) is
    a uint8 device tensor [Hm, ceil(Nq/128), ceil(Nk/128)] with Hm 1 or H (or
    2-D, shared by every head): query i sees key j only where the entry of
    (i // 128, j // 128) is nonzero; rows that see no key give zeros and
    lse = -inf.  ``dropout_p`` > 0 drops attention weights with the Philox
    contract of sdpa_fwd_dropout, keyed by ``dropout_seed`` (drawn from
    torch's CPU generator when None) and ``dropout_offset``.  ``attn_mask``
    (dense layouts only) is a device tensor broadcastable to [B,H,Nq,Nk]:
    torch.bool (True = attend), or additive in the input dtype or float32;
    it runs through sdpa_fwd_masked (sdpa_fwd_masked_dropout with
    ``dropout_p`` > 0), and rows with no finite score give zeros and
    lse = -inf.  A mask together with packed batches or a block mask, or
    dropout together with a block mask, is not supported and raises, as the
    tutorial's backends do for inputs they cannot serve.

    Dense f16/bf16 inputs that are strided views (for instance the q, k, v
    of a packed QKV projection, ``c_attn(x).chunk(3, -1)`` viewed as
    [B,H,N,d]) are read in place through sdpa_fwd_strided when their strides
    allow it, and ``out`` may be a strided [B,H,Nq,d] view to write into
    (for instance a [B,N,H*d] buffer viewed as [B,H,N,d]); other inputs are
    copied to contiguous buffers first."""
    import torch
    if not 0.0 <= float(dropout_p) < 1.0:
        raise SdpaError(SDPA_ERR_INVALID)
    if dropout_p > 0.0 and block_mask is not None:
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if not (query.dtype == key.dtype == value.dtype):
        raise SdpaError(SDPA_ERR_INVALID)
    if not (query.is_cuda and key.is_cuda and value.is_cuda):
        raise SdpaError(SDPA_ERR_INVALID)
    if attn_mask is not None:
        if cu_seqlens is not None or block_mask is not None:
            raise SdpaError(SDPA_ERR_UNSUPPORTED)
        return _masked_forward(query, key, value, attn_mask, is_causal, scale, out_dtype,
                               return_lse, stream, out, dropout_p, dropout_seed, dropout_offset)
    plain = cu_seqlens is None and block_mask is None and dropout_p == 0.0
    if (plain and query.dim() == 4 and key.dim() == 4 and value.dim() == 4
            and query.dtype in (torch.float16, torch.bfloat16)
            and (out is not None or not (query.is_contiguous() and key.is_contiguous()
                                         and value.is_contiguous()))):
        return _strided_forward(query, key, value, is_causal, scale, out_dtype, return_lse,
                                stream, out)
    q, k, v = _contig(query), _contig(key), _contig(value)
    dt = _code(q.dtype)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in (q.dtype, torch.float32):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    elif (tuple(out.shape) != tuple(q.shape) or out.dtype != odt or out.device != q.device
          or not out.is_contiguous() or out.data_ptr() % 16 != 0):
        # packed, 3-D, f32, block-sparse and dropout calls write a contiguous
        # output of the query's shape; any other buffer is refused
        raise SdpaError(SDPA_ERR_INVALID)
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
    odc = _code(odt) if odt != q.dtype else SDPA_SAME
    with torch.cuda.device(q.device):
        if block_mask is not None:
            if cu_seqlens is not None:
                raise SdpaError(SDPA_ERR_UNSUPPORTED)
            bm = block_mask[None] if block_mask.dim() == 2 else block_mask
            blk = SDPA_BLOCK_SPARSE_BLOCK
            shape = (-(-Nq // blk), -(-Nk // blk))
            if (bm.dim() != 3 or bm.dtype != torch.uint8 or not bm.is_cuda
                    or bm.shape[0] not in (1, H) or tuple(bm.shape[1:]) != shape):
                raise SdpaError(SDPA_ERR_INVALID)
            bm = bm.contiguous()
            sdpa_fwd_block_sparse(q, k, v, out, lse, B, H, Nq, Nk, d, scale, bool(is_causal),
                                  bm, bm.shape[0], dt, odc, stream)
        elif dropout_p > 0.0:
            if dropout_seed is None:
                dropout_seed = int(torch.randint(0, 2 ** 62, (1,)).item())
            sdpa_fwd_dropout(q, k, v, out, lse, B, H, Nq, Nk, d, scale, bool(is_causal),
                             cu_seqlens, dropout_p, dropout_seed, dropout_offset, dt, odc, stream)
        else:
            sdpa_fwd(q, k, v, out, lse, B, H, Nq, Nk, d, scale, bool(is_causal), cu_seqlens,
                     dt, odc, stream)
    if squeeze:
        out = out[:, 0]
        if lse is not None:
            lse = lse[:, 0]
    return (out, lse) if return_lse else out


def _strided_ok(t, mult):
    s = t.stride()
    return s[3] == 1 and all(x >= 0 and x % mult == 0 for x in s[:3]) and t.data_ptr() % 16 == 0


def _strided_forward(query, key, value, is_causal, scale, out_dtype, return_lse, stream, out):
    import torch
    q = query if _strided_ok(query, 8) else query.contiguous()
    if key.stride() == value.stride() and _strided_ok(key, 8) and _strided_ok(value, 8):
        k, v = key, value
    else:
        k, v = key.contiguous(), value.contiguous()
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise SdpaError(SDPA_ERR_INVALID)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in (q.dtype, torch.float32):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=odt, device=q.device)
    elif (tuple(out.shape) != (B, H, Nq, d) or out.dtype != odt or out.device != q.device
          or not _strided_ok(out, 4)):
        raise SdpaError(SDPA_ERR_INVALID)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if return_lse else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        sdpa_fwd_strided(q, k, v, out, lse, B, H, Nq, Nk, d, q.stride()[:3], k.stride()[:3],
                         out.stride()[:3], scale, bool(is_causal), _code(q.dtype),
                         _code(odt) if odt != q.dtype else SDPA_SAME, stream)
    return (out, lse) if return_lse else out


def _mask_operand(attn_mask, q, B, H, Nq, Nk, no_heads=False):
    """(tensor, kind, strides) for sdpa_fwd_masked: the mask viewed as
    [B,H,Nq,Nk] with broadcast dimensions at stride 0.  A mask whose layout
    the kernel cannot read in place (key stride not 1, other strides not
    multiples of 4, misaligned base, or Nk not a multiple of 16: rows are
    read in blocks of 16) is copied into rows padded to a multiple of 16
    elements."""
    import torch
    if attn_mask.dtype == torch.bool:
        kind, m = SDPA_MASK_BOOL, attn_mask.view(torch.uint8)
    elif attn_mask.dtype == q.dtype:
        kind, m = SDPA_MASK_ADD, attn_mask
    elif attn_mask.dtype == torch.float32:
        kind, m = SDPA_MASK_ADD_F32, attn_mask
    else:
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if not m.is_cuda or m.device != q.device or not 1 <= m.dim() <= (3 if no_heads else 4):
        raise SdpaError(SDPA_ERR_INVALID)
    if no_heads and m.dim() == 3:   # [B, Nq, Nk] for 3-D inputs: insert the head dim
        m = m[:, None]
    m = m.reshape((1,) * (4 - m.dim()) + tuple(m.shape)) if m.dim() < 4 else m
    try:
        m4 = m.expand(B, H, Nq, Nk)
    except RuntimeError:
        raise SdpaError(SDPA_ERR_INVALID) from None
    eb = m.element_size()

    def eff(t):   # strides with size-1 dimensions read at stride 0
        return tuple(x if n > 1 else 0 for x, n in zip(t.stride()[:3], t.shape[:3]))

    st = eff(m4)
    if not (Nk % 16 == 0 and m4.stride(3) == 1 and all(x % 4 == 0 for x in st)
            and m4.data_ptr() % (4 * eb) == 0):
        nk16 = -(-Nk // 16) * 16
        pad = torch.zeros(tuple(m.shape[:3]) + (nk16,), dtype=m.dtype, device=m.device)
        pad[..., :Nk] = m.expand(tuple(m.shape[:3]) + (Nk,))
        m4 = pad.expand(B, H, Nq, nk16)
        st = eff(m4)
    return m4, kind, st


def _masked_forward(query, key, value, attn_mask, is_causal, scale, out_dtype, return_lse,
                    stream, out, dropout_p=0.0, dropout_seed=None, dropout_offset=0):
    import torch
    squeeze = query.dim() == 3
    q, k, v = (query[:, None], key[:, None], value[:, None]) if squeeze else (query, key, value)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise SdpaError(SDPA_ERR_INVALID)
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise SdpaError(SDPA_ERR_INVALID)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in (q.dtype, torch.float32):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if not _strided_ok(q, 8):
        q = q.contiguous()
    if not (k.stride() == v.stride() and _strided_ok(k, 8) and _strided_ok(v, 8)):
        k, v = k.contiguous(), v.contiguous()
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=odt, device=q.device)
    else:
        out = out[:, None] if squeeze else out
        if (tuple(out.shape) != (B, H, Nq, d) or out.dtype != odt or out.device != q.device
                or not _strided_ok(out, 4)):
            raise SdpaError(SDPA_ERR_INVALID)
    m4, kind, mst = _mask_operand(attn_mask, q, B, H, Nq, Nk, no_heads=squeeze)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if return_lse else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    odc = _code(odt) if odt != q.dtype else SDPA_SAME
    with torch.cuda.device(q.device):
        if dropout_p > 0.0:
            if dropout_seed is None:
                dropout_seed = int(torch.randint(0, 2 ** 62, (1,)).item())
            sdpa_fwd_masked_dropout(q, k, v, out, lse, B, H, Nq, Nk, d, q.stride()[:3],
                                    k.stride()[:3], out.stride()[:3], scale, bool(is_causal), m4,
                                    kind, mst, dropout_p, dropout_seed, dropout_offset,
                                    _code(q.dtype), odc, stream)
        else:
            sdpa_fwd_masked(q, k, v, out, lse, B, H, Nq, Nk, d, q.stride()[:3], k.stride()[:3],
                            out.stride()[:3], scale, bool(is_causal), m4, kind, mst,
                            _code(q.dtype), odc, stream)
    if squeeze:
        out = out[:, 0]
        if lse is not None:
            lse = lse[:, 0]
    return (out, lse) if return_lse else out


def scaled_dot_product_attention_backward(query, key, value, out, lse, grad_out,
                                          is_causal=False, scale=None, grad_dtype=None,
                                          stream=None, dropout_p=0.0, dropout_seed=None,
                                          dropout_offset=0, cu_seqlens=None, max_seqlen=None,
                                          attn_mask=None, block_mask=None):
    """Gradients (dq, dk, dv) of sum(grad_out * out) for dense inputs
    [B,H,N,d], or packed inputs [T,H,d] with ``cu_seqlens`` and
    ``max_seqlen`` (as the forward), given the forward's out and lse.
    ``grad_out`` is cast to the input dtype (the matrix cores consume it);
    ``grad_dtype`` None keeps the input dtype, torch.float32 requests f32
    gradients.  After a dropout forward, pass its ``dropout_p``,
    ``dropout_seed`` and ``dropout_offset``; after a masked or block-sparse
    forward, the same ``attn_mask`` or ``block_mask`` (dense inputs; a mask
    may come with dropout, a block mask may not)."""
    import torch
    if not (query.dtype == key.dtype == value.dtype):
        raise SdpaError(SDPA_ERR_INVALID)
    if (attn_mask is not None or block_mask is not None) and (
            cu_seqlens is not None or (block_mask is not None and dropout_p > 0.0)
            or (attn_mask is not None and block_mask is not None)):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if cu_seqlens is not None:
        return _packed_backward(query, key, value, out, lse, grad_out, is_causal, scale,
                                grad_dtype, stream, dropout_p, dropout_seed, dropout_offset,
                                cu_seqlens, max_seqlen)
    q, k, v, o = _contig(query), _contig(key), _contig(value), _contig(out)
    if q.dim() != 4 or k.dim() != 4 or o.shape != q.shape or grad_out.shape != q.shape:
        raise SdpaError(SDPA_ERR_INVALID)
    dt = _code(q.dtype)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise SdpaError(SDPA_ERR_INVALID)
    if lse is None or lse.shape != (B, H, Nq) or lse.dtype != torch.float32:
        raise SdpaError(SDPA_ERR_INVALID)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    if gdt not in (q.dtype, torch.float32) or o.dtype not in (q.dtype, torch.float32):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    do = _contig(grad_out.to(q.dtype))
    lse = _contig(lse)
    dq = torch.empty(q.shape, dtype=gdt, device=q.device)
    dk = torch.empty(k.shape, dtype=gdt, device=q.device)
    dv = torch.empty(v.shape, dtype=gdt, device=q.device)
    work = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    odc = SDPA_F32 if o.dtype != q.dtype else SDPA_SAME
    gdc = SDPA_F32 if gdt != q.dtype else SDPA_SAME
    with torch.cuda.device(q.device):
        if block_mask is not None:
            bm = block_mask[None] if block_mask.dim() == 2 else block_mask
            blk = SDPA_BLOCK_SPARSE_BLOCK
            if (bm.dim() != 3 or bm.dtype != torch.uint8 or not bm.is_cuda
                    or bm.shape[0] not in (1, H)
                    or tuple(bm.shape[1:]) != (-(-Nq // blk), -(-Nk // blk))):
                raise SdpaError(SDPA_ERR_INVALID)
            bm = bm.contiguous()
            sdpa_bwd_block_sparse(q, k, v, o, do, lse, dq, dk, dv, work, B, H, Nq, Nk, d, scale,
                                  bool(is_causal), bm, bm.shape[0], dt, odc, gdc, stream)
            return dq, dk, dv
        if attn_mask is not None:
            m4, kind, mst = _mask_operand(attn_mask, q, B, H, Nq, Nk)
            if dropout_p > 0.0:
                if dropout_seed is None:
                    raise SdpaError(SDPA_ERR_INVALID)   # the forward's seed is needed
                sdpa_bwd_masked_dropout(q, k, v, o, do, lse, dq, dk, dv, work, B, H, Nq, Nk, d,
                                        scale, bool(is_causal), m4, kind, mst, dropout_p,
                                        dropout_seed, dropout_offset, dt, odc, gdc, stream)
            else:
                sdpa_bwd_masked(q, k, v, o, do, lse, dq, dk, dv, work, B, H, Nq, Nk, d, scale,
                                bool(is_causal), m4, kind, mst, dt, odc, gdc, stream)
            return dq, dk, dv
        if dropout_p > 0.0:
            if dropout_seed is None:
                raise SdpaError(SDPA_ERR_INVALID)   # the forward's seed is needed
            sdpa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, work, B, H, Nq, Nk, d, scale,
                             bool(is_causal), dropout_p, dropout_seed, dropout_offset, dt, odc,
                             gdc, stream)
        else:
            sdpa_bwd(q, k, v, o, do, lse, dq, dk, dv, work, B, H, Nq, Nk, d, scale,
                     bool(is_causal), dt, odc, gdc, stream)
    return dq, dk, dv


def _packed_backward(query, key, value, out, lse, grad_out, is_causal, scale, grad_dtype,
                     stream, dropout_p, dropout_seed, dropout_offset, cu_seqlens, max_seqlen):
    import torch
    q, k, v, o = _contig(query), _contig(key), _contig(value), _contig(out)
    if (q.dim() != 3 or k.shape != q.shape or v.shape != q.shape or o.shape != q.shape
            or grad_out.shape != q.shape or max_seqlen is None):
        raise SdpaError(SDPA_ERR_INVALID)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise SdpaError(SDPA_ERR_INVALID)
    T, H, d = q.shape
    B = cu_seqlens.numel() - 1
    if lse is None or lse.shape != (T, H) or lse.dtype != torch.float32:
        raise SdpaError(SDPA_ERR_INVALID)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    if gdt not in (q.dtype, torch.float32) or o.dtype not in (q.dtype, torch.float32):
        raise SdpaError(SDPA_ERR_UNSUPPORTED)
    if dropout_p > 0.0 and dropout_seed is None:
        raise SdpaError(SDPA_ERR_INVALID)   # the forward's seed is needed
    do = _contig(grad_out.to(q.dtype))
    lse = _contig(lse)
    dq, dk, dv = (torch.zeros(q.shape, dtype=gdt, device=q.device) for _ in range(3))
    work = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        sdpa_bwd_packed(q, k, v, o, do, lse, dq, dk, dv, work, B, H, T, int(max_seqlen), d,
                        scale, bool(is_causal), cu_seqlens, float(dropout_p),
                        int(dropout_seed or 0), int(dropout_offset), _code(q.dtype),
                        SDPA_F32 if o.dtype != q.dtype else SDPA_SAME,
                        SDPA_F32 if gdt != q.dtype else SDPA_SAME, stream)
    return dq, dk, dv


def _autograd_function():
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, is_causal, scale, dropout_p, seed, offset, cu, max_seqlen,
                    attn_mask, block_mask):
            out, lse = scaled_dot_product_attention(q, k, v, is_causal=is_causal, scale=scale,
                                                    dropout_p=dropout_p, dropout_seed=seed,
                                                    dropout_offset=offset, return_lse=True,
                                                    cu_seqlens=cu, max_seqlen=max_seqlen,
                                                    attn_mask=attn_mask, block_mask=block_mask)
            ctx.attn_mask, ctx.block_mask = attn_mask, block_mask
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.is_causal, ctx.scale = is_causal, scale
            ctx.drop = (dropout_p, seed, offset)
            ctx.packed = (cu, max_seqlen)
            return out

        @staticmethod
        def backward(ctx, grad_out):
            q, k, v, out, lse = ctx.saved_tensors
            p, seed, offset = ctx.drop
            cu, max_seqlen = ctx.packed
            dq, dk, dv = scaled_dot_product_attention_backward(
                q, k, v, out, lse, grad_out, is_causal=ctx.is_causal, scale=ctx.scale,
                dropout_p=p, dropout_seed=seed, dropout_offset=offset, cu_seqlens=cu,
                max_seqlen=max_seqlen, attn_mask=ctx.attn_mask, block_mask=ctx.block_mask)
            return dq, dk, dv, None, None, None, None, None, None, None, None, None

    return _Attention


_ATTN = None


def attention(query, key, value, is_causal=False, scale=None, dropout_p=0.0, dropout_seed=None,
              dropout_offset=0, cu_seqlens=None, max_seqlen=None, attn_mask=None,
              block_mask=None):
    """Differentiable attention, dense [B,H,N,d] or packed [T,H,d] with
    ``cu_seqlens`` and ``max_seqlen``, optionally with an elementwise
    ``attn_mask`` or a ``block_mask`` (dense; masks are not differentiated):
    the forward and backward both run in the HIP kernels.  With ``dropout_p`` > 0 the backward
    regenerates the forward's mask from the same seed (drawn from torch's
    CPU generator when None) and offset."""
    global _ATTN
    if _ATTN is None:
        _ATTN = _autograd_function()
    if dropout_p > 0.0 and dropout_seed is None:
        import torch
        dropout_seed = int(torch.randint(0, 2 ** 62, (1,)).item())
    return _ATTN.apply(query, key, value, bool(is_causal), scale, float(dropout_p), dropout_seed,
                       int(dropout_offset), cu_seqlens,
                       None if max_seqlen is None else int(max_seqlen), attn_mask, block_mask)

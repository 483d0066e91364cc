"""ctypes loader for libsdpa.so (the gfx950 HIP library with the C ABI of
include/sdpa.h).  There is no fallback: if the library is missing, every
entry point raises."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

SDPA_F16, SDPA_BF16, SDPA_F32, SDPA_SAME = 0, 1, 2, 255
SDPA_OK, SDPA_ERR_INVALID, SDPA_ERR_UNSUPPORTED, SDPA_ERR_LAUNCH, SDPA_ERR_DEVICE = range(5)
SDPA_BLOCK_SPARSE_BLOCK = 128
SDPA_MASK_BOOL, SDPA_MASK_ADD, SDPA_MASK_ADD_F32 = 0, 1, 2
SDPA_BWD_NOALLOC_MAX_ROWS = 4 * 1024 * 1024

# every symbol include/sdpa.h declares
EXPORTS = ("sdpa_fwd", "sdpa_fwd_strided", "sdpa_fwd_masked", "sdpa_fwd_masked_dropout",
           "sdpa_fwd_block_sparse", "sdpa_fwd_dropout", "sdpa_bwd", "sdpa_bwd_dropout",
           "sdpa_bwd_packed", "sdpa_bwd_masked", "sdpa_bwd_masked_dropout",
           "sdpa_bwd_block_sparse", "sdpa_bwd_noalloc", "sdpa_bwd_workspace_bytes",
           "sdpa_supports", "sdpa_status_str", "sdpa_abi_version")

# the same library built with the LDS-poisoning debug option
LIB_DEBUG_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa_debug.so")

_lib = None
_lib_debug = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def lib_debug() -> ctypes.CDLL:
    """libsdpa_debug.so: the entry points of lib() with LDS poisoning on."""
    global _lib_debug
    if _lib_debug is None:
        _lib_debug = _load(LIB_DEBUG_PATH)
    return _lib_debug


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m exact_attention_sdpa_amd.build` "
            "(the HIP library is required, there is no fallback)")
    L = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.sdpa_fwd.restype = ctypes.c_int
    L.sdpa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                           ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp]
    L.sdpa_fwd_strided.restype = ctypes.c_int
    L.sdpa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp,
                                   ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.sdpa_fwd_masked.restype = ctypes.c_int
    L.sdpa_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp,
                                  ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp,
                                  ctypes.c_int, ctypes.c_int, vp]
    L.sdpa_fwd_masked_dropout.restype = ctypes.c_int
    L.sdpa_fwd_masked_dropout.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp,
                                          ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp,
                                          ctypes.c_float, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.c_int, ctypes.c_int, vp]
    L.sdpa_fwd_block_sparse.restype = ctypes.c_int
    L.sdpa_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                        ctypes.c_float, ctypes.c_int, vp, i64, ctypes.c_int,
                                        ctypes.c_int, vp]
    L.sdpa_fwd_dropout.restype = ctypes.c_int
    L.sdpa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                   ctypes.c_int, vp, ctypes.c_float, ctypes.c_uint64,
                                   ctypes.c_uint32, ctypes.c_int, ctypes.c_int, vp]
    L.sdpa_bwd.restype = ctypes.c_int
    L.sdpa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                           ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           ctypes.c_int, vp]
    L.sdpa_bwd_dropout.restype = ctypes.c_int
    L.sdpa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                   i64, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                   ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, vp]
    L.sdpa_bwd_packed.restype = ctypes.c_int
    L.sdpa_bwd_packed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                  i64, ctypes.c_float, ctypes.c_int, vp, ctypes.c_float,
                                  ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, vp]
    L.sdpa_bwd_masked.restype = ctypes.c_int
    L.sdpa_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                  i64, ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.sdpa_bwd_masked_dropout.restype = ctypes.c_int
    L.sdpa_bwd_masked_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                          i64, i64, ctypes.c_float, ctypes.c_int, vp,
                                          ctypes.c_int, vp, ctypes.c_float, ctypes.c_uint64,
                                          ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, vp]
    L.sdpa_bwd_block_sparse.restype = ctypes.c_int
    L.sdpa_bwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                        i64, i64, ctypes.c_float, ctypes.c_int, vp, i64,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    L.sdpa_bwd_noalloc.restype = ctypes.c_int
    L.sdpa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                   ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, vp]
    L.sdpa_bwd_workspace_bytes.restype = i64
    L.sdpa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    L.sdpa_supports.restype = ctypes.c_int
    L.sdpa_supports.argtypes = [ctypes.c_int, i64, ctypes.c_int, ctypes.c_int]
    L.sdpa_status_str.restype = ctypes.c_char_p
    L.sdpa_status_str.argtypes = [ctypes.c_int]
    L.sdpa_abi_version.restype = ctypes.c_int
    L.sdpa_abi_version.argtypes = []
    return L

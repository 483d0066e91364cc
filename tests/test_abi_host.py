"""The C-ABI library on the host: it loads, exports what include/sdpa.h
declares, and rejects malformed calls before touching any device."""
import ctypes
import os
import re

import pytest

from exact_attention_sdpa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")

OK, INVALID, UNSUPPORTED, LAUNCH, DEVICE = range(5)
F16, BF16, F32, SAME = 0, 1, 2, 255

# fake, 256-byte aligned, distinct addresses: only ever used on paths that
# return before any HIP call
Q, K, V, O, L = 0x10000, 0x20000000, 0x40000000, 0x60000000, 0x7F000000


def _declared():
    text = open(HEADER).read()
    return re.findall(r"SDPA_API\s+[\w\s\*]+?\b(sdpa_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_header_declares_expected_symbols():
    assert sorted(_declared()) == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+SDPA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.sdpa_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s in range(5):
        assert lib.sdpa_status_str(s)
    assert lib.sdpa_status_str(2) == b"not supported"
    assert lib.sdpa_status_str(99) == b"unknown status"


def test_supports_matrix(lib):
    for dt in (F16, BF16):
        for d in (32, 64, 128):
            assert lib.sdpa_supports(dt, d, 0, 0) == 1
            assert lib.sdpa_supports(dt, d, 1, 1) == 1
        for d in (8, 16, 48, 96, 256):
            assert lib.sdpa_supports(dt, d, 0, 0) == -1
    # the flags are booleans; anything else is refused
    assert lib.sdpa_supports(F16, 64, 2, 0) == -1
    assert lib.sdpa_supports(F16, 64, 0, -1) == -1
    assert lib.sdpa_supports(F32, 8, 1, 1) == 0
    for d in (1, 3, 8, 64, 128):
        assert lib.sdpa_supports(F32, d, 0, 0) == 0
    assert lib.sdpa_supports(F32, 129, 0, 0) == -1
    assert lib.sdpa_supports(SAME, 64, 0, 0) == -1


def call(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=4, Nq=128, Nk=128, d=64, scale=0.125,
         causal=0, cu=None, dt=F16, odt=SAME):
    return lib.sdpa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, cu, dt, odt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID),
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(Nq=0), INVALID), (dict(Nk=0), INVALID),
    (dict(d=0), INVALID), (dict(B=-1), INVALID), (dict(Nq=1 << 31), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(causal=2), INVALID), (dict(dt=SAME), INVALID), (dict(dt=7), INVALID),
    (dict(odt=9), INVALID),
    (dict(cu=0x1000, Nq=128, Nk=64), INVALID),
    (dict(q=Q + 8), INVALID), (dict(o=O + 2), INVALID), (dict(lse=L + 2), INVALID),
    (dict(cu=0x1002), INVALID),
    (dict(o=Q + 64), INVALID),  # output overlaps q
    (dict(d=48), UNSUPPORTED), (dict(d=16), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(dt=BF16, d=80), UNSUPPORTED), (dict(dt=F32, d=129), UNSUPPORTED),
    (dict(scale=-0.5), UNSUPPORTED), (dict(scale=3.0e38), UNSUPPORTED), (dict(dt=F16, odt=BF16), UNSUPPORTED),
    (dict(dt=F32, odt=F16), UNSUPPORTED),
])
def test_invalid_calls_rejected_on_host(lib, kw, status):
    assert call(lib, **kw) == status


def test_f32_path_needs_only_4_byte_alignment(lib):
    # misaligned for the f16 path, fine for f32: must get past validation and
    # then stop at the device check.  Only meaningful with no GPU present
    # (the addresses are fake and must never reach a kernel).
    if _gpu_present():
        pytest.skip("a GPU is present")
    assert call(lib, q=Q + 4, dt=F32, d=8) == DEVICE


def test_no_device_is_reported(lib):
    if _gpu_present():
        pytest.skip("a GPU is present")
    assert call(lib) == DEVICE


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def _strided_call(lib, qs=(4 * 128 * 64, 128 * 64, 64), ks=None, os_=None, q=0x1000000,
                  k=0x2000000, v=0x3000000, o=0x4000000, lse=0x6000000, B=2, H=4, N=128, d=64,
                  dt=0):
    import ctypes
    arr = lambda s: None if s is None else ctypes.cast((ctypes.c_int64 * 3)(*s), ctypes.c_void_p)
    ks = qs if ks is None else ks
    os_ = qs if os_ is None else os_
    return lib.sdpa_fwd_strided(q, k, v, o, lse, B, H, N, N, d, arr(qs), arr(ks), arr(os_),
                                0.125, 0, dt, 255, None)


def test_strided_calls_rejected_on_host(lib):
    INVALID, UNSUPPORTED, DEVICE = 1, 2, 4
    # the packed-QKV layout of a [2, 128, 3*256] projection, out [2, 128, 256]
    qkv = (128 * 768, 64, 768)
    out = (128 * 256, 64, 256)
    assert _strided_call(lib, qkv, qkv, out) in (0, DEVICE)
    assert _strided_call(lib, (1, 64, 768)) == INVALID           # not a multiple of 8
    assert _strided_call(lib, qkv, qkv, (128 * 256, 2, 256)) == INVALID   # out rows overlap
    assert _strided_call(lib, qkv, qkv, (0, 64, 256)) == INVALID  # batches share the output
    assert _strided_call(lib, qkv, qkv, out, o=0x1000000 + 4096) == INVALID  # out inside q
    assert _strided_call(lib, (-8, 64, 768)) == INVALID
    assert lib.sdpa_fwd_strided(0x1000000, 0x2000000, 0x3000000, 0x4000000, None, 1, 1, 8, 8,
                                64, None, None, None, 0.1, 0, 0, 255, None) == INVALID
    assert _strided_call(lib, qkv, qkv, out, dt=2) == UNSUPPORTED  # f32 inputs
    # a head's rows past 32-bit offsets
    assert _strided_call(lib, (0, 0, 1 << 24), (0, 0, 1 << 24), out, N=200) == UNSUPPORTED

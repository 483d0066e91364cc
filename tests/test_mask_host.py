"""Host-side checks of the elementwise-mask entry points (sdpa_fwd_masked,
sdpa_bwd_masked and their dropout forms):
every malformed call is rejected before any device work."""
import ctypes

import pytest

from exact_attention_sdpa_amd import _lib

OK, INVALID, UNSUPPORTED, LAUNCH, DEVICE = range(5)
F16, BF16, F32, SAME = 0, 1, 2, 255
MBOOL, MADD, MF32 = 0, 1, 2

# fake, distinct, aligned addresses (never dereferenced on these paths)
Q, K, V, O, L, M = 0x1000000, 0x2000000, 0x3000000, 0x4000000, 0x6000000, 0x10000000


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def arr(s):
    return None if s is None else ctypes.cast((ctypes.c_int64 * 3)(*s), ctypes.c_void_p)


def call(lib, ms=(4 * 128 * 128, 128 * 128, 128), kind=MBOOL, mask=M, B=2, H=4, N=128, d=64,
         dt=F16, strides=None, o=O, lse=L, causal=0):
    qs = ks = os_ = strides
    return lib.sdpa_fwd_masked(Q, K, V, o, lse, B, H, N, N, d, arr(qs), arr(ks), arr(os_),
                               0.125, causal, mask, kind, arr(ms), dt, SAME, None)


def test_valid_masked_calls_reach_the_device_check(lib):
    for kind in (MBOOL, MADD, MF32):
        assert call(lib, kind=kind) in (OK, DEVICE)
        assert call(lib, kind=kind, causal=1) in (OK, DEVICE)
    # broadcasts: one mask for every head and batch, a key-padding row
    assert call(lib, ms=(0, 0, 128)) in (OK, DEVICE)
    assert call(lib, ms=(128, 0, 0)) in (OK, DEVICE)
    # with explicit q/k/v/out strides (packed QKV layout)
    assert call(lib, strides=(128 * 768, 64, 768), o=0x8000000,
                lse=0x9000000) in (OK, DEVICE)


def test_masked_calls_rejected_on_host(lib):
    assert call(lib, mask=None) == INVALID
    assert lib.sdpa_fwd_masked(Q, K, V, O, L, 2, 4, 128, 128, 64, None, None, None, 0.125, 0,
                               M, MBOOL, None, F16, SAME, None) == INVALID   # no mask strides
    assert call(lib, kind=7) == INVALID
    assert call(lib, ms=(-4, 0, 128)) == INVALID
    assert call(lib, ms=(0, 0, 130)) == INVALID          # row stride not a multiple of 4
    assert call(lib, kind=MF32, mask=M + 4) == INVALID   # f32 mask not 16-byte aligned
    assert call(lib, kind=MADD, mask=M + 4) == INVALID   # 16-bit mask not 8-byte aligned
    assert call(lib, kind=MBOOL, mask=M + 4) in (OK, DEVICE)   # bytes: 4-byte aligned is fine
    assert call(lib, kind=MBOOL, mask=M + 2) == INVALID
    assert call(lib, dt=F32) == UNSUPPORTED               # f32 inputs
    # the mask must not overlap the output or the logsumexp
    assert call(lib, mask=O) == INVALID
    assert call(lib, mask=L) == INVALID
    # rows too far apart for a workgroup's 32-bit offsets
    assert call(lib, kind=MF32, ms=(0, 0, 1 << 21)) == UNSUPPORTED
    # only some of q/k/v/out strides given
    assert lib.sdpa_fwd_masked(Q, K, V, O, L, 2, 4, 128, 128, 64, arr((128 * 768, 64, 768)),
                               None, None, 0.125, 0, M, MBOOL, arr((0, 0, 128)), F16, SAME,
                               None) == INVALID
    # errors of the dense forward still apply
    assert call(lib, d=48) == UNSUPPORTED
    assert call(lib, N=0) == INVALID


def bcall(lib, ms=(4 * 128 * 128, 128 * 128, 128), kind=MBOOL, mask=M, dt=F16, N=128,
          work=0x9000000, dq=0x7000000):
    return lib.sdpa_bwd_masked(Q, K, V, O, 0x5000000, L, dq, 0x7800000, 0x8000000, work, 2, 4,
                               N, N, 64, 0.125, 0, mask, kind, arr(ms), dt, SAME, SAME, None)


def test_masked_backward_rejected_on_host(lib):
    for kind in (MBOOL, MADD, MF32):
        assert bcall(lib, kind=kind) in (OK, DEVICE)
    assert bcall(lib, mask=None) == INVALID
    assert lib.sdpa_bwd_masked(Q, K, V, O, 0x5000000, L, 0x7000000, 0x7800000, 0x8000000,
                               0x9000000, 2, 4, 128, 128, 64, 0.125, 0, M, MBOOL, None, F16,
                               SAME, SAME, None) == INVALID
    assert bcall(lib, kind=9) == INVALID
    assert bcall(lib, ms=(0, 0, 130)) == INVALID
    assert bcall(lib, kind=MF32, mask=M + 4) == INVALID
    assert bcall(lib, dt=F32) == UNSUPPORTED
    assert bcall(lib, mask=0x9000000) == INVALID      # overlaps the workspace
    assert bcall(lib, mask=0x7000000) == INVALID      # overlaps dq
    # a unit's mask beyond 32-bit offsets
    assert bcall(lib, kind=MF32, ms=(0, 0, 1 << 19), N=1024) == UNSUPPORTED


def dcall(lib, p=0.1, ms=(4 * 128 * 128, 128 * 128, 128), kind=MBOOL, mask=M, dt=F16, d=64,
          causal=0, o=O, lse=L):
    return lib.sdpa_fwd_masked_dropout(Q, K, V, o, lse, 2, 4, 128, 128, d, None, None, None,
                                       0.125, causal, mask, kind, arr(ms), p, 7, 3, dt, SAME,
                                       None)


def dbcall(lib, p=0.1, ms=(4 * 128 * 128, 128 * 128, 128), kind=MBOOL, mask=M, dt=F16):
    return lib.sdpa_bwd_masked_dropout(Q, K, V, O, 0x5000000, L, 0x7000000, 0x7800000,
                                       0x8000000, 0x9000000, 2, 4, 128, 128, 64, 0.125, 0, mask,
                                       kind, arr(ms), p, 7, 3, dt, SAME, SAME, None)


def test_masked_dropout_calls_on_host(lib):
    """sdpa_fwd_masked_dropout / sdpa_bwd_masked_dropout: the mask checks
    and the dropout checks both apply."""
    for kind in (MBOOL, MADD, MF32):
        for p in (0.0, 0.1, 0.999):
            assert dcall(lib, p=p, kind=kind) in (OK, DEVICE)
            assert dbcall(lib, p=p, kind=kind) in (OK, DEVICE)
        assert dcall(lib, kind=kind, causal=1) in (OK, DEVICE)
    for f in (dcall, dbcall):
        assert f(lib, mask=None) == INVALID
        assert f(lib, ms=None) == INVALID
        assert f(lib, kind=5) == INVALID
        assert f(lib, ms=(0, 0, 130)) == INVALID
        assert f(lib, kind=MF32, mask=M + 4) == INVALID
        assert f(lib, dt=F32) == UNSUPPORTED
        for p in (1.0, -0.1, 1.5, float("nan")):
            assert f(lib, p=p) == INVALID
        assert f(lib, p=float(1 - 2 ** -18)) == UNSUPPORTED   # nothing would be kept
    assert dcall(lib, mask=O) == INVALID
    assert dcall(lib, mask=L) == INVALID
    assert dcall(lib, d=48) == UNSUPPORTED
    assert dbcall(lib, mask=0x9000000) == INVALID      # overlaps the workspace

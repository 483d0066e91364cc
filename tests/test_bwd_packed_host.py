"""Host-side checks of the packed-batch backward entry point
(sdpa_bwd_packed): malformed calls are rejected before any device work."""
import pytest

from exact_attention_sdpa_amd import _lib

OK, INVALID, UNSUPPORTED, LAUNCH, DEVICE = range(5)
F16, BF16, F32, SAME = 0, 1, 2, 255

# fake, distinct, aligned addresses (never dereferenced on these paths)
Q, K, V, O, G, L = 0x1000000, 0x2000000, 0x3000000, 0x4000000, 0x5000000, 0x6000000
DQ, DK, DV, W, CU = 0x7000000, 0x8000000, 0x9000000, 0xA000000, 0xB000000


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def call(lib, B=4, H=2, T=1000, maxlen=400, d=64, cu=CU, p=0.0, dt=F16, dq=DQ, w=W, far=False):
    if far:   # tensors of several GiB: addresses 64 GiB apart
        a = [(i + 1) << 36 for i in range(10)]
        return lib.sdpa_bwd_packed(*a[:6], a[6], a[7], a[8], a[9], B, H, T, maxlen, d, 0.125, 0,
                                   cu, p, 7, 0, dt, SAME, SAME, None)
    return lib.sdpa_bwd_packed(Q, K, V, O, G, L, dq, DK, DV, w, B, H, T, maxlen, d, 0.125, 0,
                               cu, p, 7, 0, dt, SAME, SAME, None)


def test_valid_packed_backward_reaches_the_device_check(lib):
    assert call(lib) in (OK, DEVICE)
    assert call(lib, p=0.3) in (OK, DEVICE)
    assert call(lib, d=128, dt=BF16) in (OK, DEVICE)


def test_packed_backward_rejected_on_host(lib):
    assert call(lib, cu=None) == INVALID
    assert call(lib, cu=CU + 2) == INVALID              # int32 offsets: 4-byte aligned
    assert call(lib, B=0) == INVALID
    assert call(lib, T=0) == INVALID
    assert call(lib, maxlen=0) == INVALID
    assert call(lib, p=1.0) == INVALID
    assert call(lib, p=-0.1) == INVALID
    assert call(lib, dt=F32) == UNSUPPORTED
    assert call(lib, d=48) == UNSUPPORTED
    assert call(lib, dq=Q) == INVALID                    # output overlaps an input
    assert call(lib, w=DK) == INVALID                    # workspace overlaps an output
    # a sequence's rows beyond 32-bit offsets (row stride H*d)
    assert call(lib, H=4096, d=128, maxlen=4096, T=4096, far=True) == UNSUPPORTED
    assert call(lib, H=16, d=128, maxlen=4096, T=4096, far=True) in (OK, DEVICE)

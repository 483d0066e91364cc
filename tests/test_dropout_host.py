"""sdpa_fwd_dropout on the host: malformed calls are rejected before any
device work."""
import pytest

from exact_attention_sdpa_amd import _lib

OK, INVALID, UNSUPPORTED, LAUNCH, DEVICE = range(5)
F16, BF16, F32, SAME = 0, 1, 2, 255

# fake, well separated, 256-byte aligned addresses (never dereferenced)
BASE = {"q": 0x1000000, "k": 0x2000000, "v": 0x3000000, "o": 0x4000000, "lse": 0x6000000}


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def call(lib, B=2, H=4, Nq=128, Nk=128, d=64, scale=0.125, causal=0, p=0.1, seed=1, off=0,
         dt=F16, odt=SAME, **ptrs):
    a = dict(BASE)
    a.update(ptrs)
    return lib.sdpa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], B, H, Nq, Nk, d, scale,
                                causal, None, p, seed, off, dt, odt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=1.0), INVALID), (dict(p=-0.1), INVALID), (dict(p=float("nan")), INVALID),
    (dict(p=1.5), INVALID), (dict(q=None), INVALID), (dict(B=0), INVALID),
    (dict(dt=F32), UNSUPPORTED), (dict(d=48), UNSUPPORTED),
    # 1 - p below 2^-17: the 16-bit keep threshold rounds to 0, nothing
    # would be kept
    (dict(p=float(1 - 2 ** -18)), UNSUPPORTED), (dict(p=float(1 - 2 ** -20)), UNSUPPORTED),
])
def test_invalid_dropout_calls_rejected_on_host(lib, kw, status):
    assert call(lib, **kw) == status


def test_valid_calls_reach_the_device_check(lib):
    try:
        import torch
        if torch.cuda.device_count() > 0:
            pytest.skip("a GPU is present")
    except Exception:
        pass
    for kw in (dict(), dict(p=0.0), dict(p=0.999, seed=2 ** 64 - 1, off=2 ** 32 - 1),
               dict(dt=BF16, odt=F32, causal=1)):
        assert call(lib, **kw) == DEVICE

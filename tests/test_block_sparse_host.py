"""sdpa_fwd_block_sparse on the host: malformed calls are rejected before any
device work."""
import pytest

from exact_attention_sdpa_amd import _lib

OK, INVALID, UNSUPPORTED, LAUNCH, DEVICE = range(5)
F16, BF16, F32, SAME = 0, 1, 2, 255

# fake, well separated, 256-byte aligned addresses (never dereferenced: every
# call here returns before any HIP call)
BASE = {"q": 0x1000000, "k": 0x2000000, "v": 0x3000000, "o": 0x4000000,
        "lse": 0x6000000, "m": 0x7000000}


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def call(lib, B=2, H=4, Nq=300, Nk=200, d=64, scale=0.125, causal=0, mh=4, dt=F16, odt=SAME,
         **ptrs):
    p = dict(BASE)
    p.update(ptrs)
    return lib.sdpa_fwd_block_sparse(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, Nq, Nk,
                                     d, scale, causal, p["m"], mh, dt, odt, None)


def test_block_size_matches_header():
    import re
    from tests.test_abi_host import HEADER
    m = re.search(r"#define\s+SDPA_BLOCK_SPARSE_BLOCK\s+(\d+)", open(HEADER).read())
    assert int(m.group(1)) == _lib.SDPA_BLOCK_SPARSE_BLOCK == 128


@pytest.mark.parametrize("kw,status", [
    (dict(m=None), INVALID), (dict(mh=0), INVALID), (dict(mh=2), INVALID),
    (dict(mh=5), INVALID), (dict(q=None), INVALID), (dict(B=0), INVALID),
    (dict(causal=2), INVALID), (dict(q=BASE["q"] + 8), INVALID),
    # mask [4][3][2] = 24 bytes must not overlap out or lse
    (dict(m=BASE["o"] + 64), INVALID), (dict(m=BASE["lse"] - 8), INVALID),
    (dict(dt=F32), UNSUPPORTED), (dict(d=48), UNSUPPORTED), (dict(dt=BF16, odt=F16),
                                                               UNSUPPORTED),
])
def test_invalid_block_sparse_calls_rejected_on_host(lib, kw, status):
    assert call(lib, **kw) == status


def test_unaligned_mask_is_fine_and_shared_mask_accepted(lib):
    try:
        import torch
        if torch.cuda.device_count() > 0:
            pytest.skip("a GPU is present")
    except Exception:
        pass
    # every argument valid: the call gets as far as the device check
    assert call(lib, m=BASE["m"] + 1, mh=1) == DEVICE
    assert call(lib, mh=4, causal=1, dt=BF16, odt=F32) == DEVICE


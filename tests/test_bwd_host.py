"""sdpa_bwd on the host: malformed calls are rejected before any device work,
and the workspace size is B*H*Nq floats."""
import pytest

from exact_attention_sdpa_amd import _lib

OK, INVALID, UNSUPPORTED, LAUNCH, DEVICE = range(5)
F16, BF16, F32, SAME = 0, 1, 2, 255

# fake, well separated, 256-byte aligned addresses (never dereferenced: every
# call here returns before any HIP call)
BASE = {"q": 0x1000000, "k": 0x2000000, "v": 0x3000000, "o": 0x4000000, "g": 0x5000000,
        "lse": 0x6000000, "dq": 0x7000000, "dk": 0x8000000, "dv": 0x9000000,
        "w": 0xA000000}


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def call(lib, B=2, H=4, Nq=128, Nk=128, d=64, scale=0.125, causal=0, dt=F16, odt=SAME,
         gdt=SAME, **ptrs):
    p = dict(BASE)
    p.update(ptrs)
    return lib.sdpa_bwd(p["q"], p["k"], p["v"], p["o"], p["g"], p["lse"], p["dq"], p["dk"],
                        p["dv"], p["w"], B, H, Nq, Nk, d, scale, causal, dt, odt, gdt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(g=None), INVALID),
    (dict(lse=None), INVALID), (dict(dq=None), INVALID), (dict(w=None), INVALID),
    (dict(B=0), INVALID), (dict(Nk=0), INVALID), (dict(d=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(causal=3), INVALID), (dict(dt=9), INVALID),
    (dict(odt=7), INVALID), (dict(gdt=7), INVALID),
    (dict(q=BASE["q"] + 8), INVALID), (dict(dk=BASE["dk"] + 4), INVALID),
    (dict(lse=BASE["lse"] + 2), INVALID),
    (dict(dq=BASE["q"] + 256), INVALID),     # dq overlaps q
    (dict(dv=BASE["dk"] + 512), INVALID),    # dv overlaps dk
    (dict(w=BASE["lse"]), INVALID),          # workspace overlaps lse
    (dict(dt=F32), UNSUPPORTED), (dict(d=48), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(scale=-1.0), UNSUPPORTED), (dict(dt=BF16, gdt=F16), UNSUPPORTED),
    (dict(dt=F16, odt=BF16), UNSUPPORTED),
])
def test_invalid_bwd_calls_rejected_on_host(lib, kw, status):
    assert call(lib, **kw) == status


def test_workspace_bytes(lib):
    assert lib.sdpa_bwd_workspace_bytes(2, 3, 5) == 2 * 3 * 5 * 4
    assert lib.sdpa_bwd_workspace_bytes(0, 3, 5) == 0
    assert lib.sdpa_bwd_workspace_bytes(-1, 3, 5) == -1
    assert lib.sdpa_bwd_workspace_bytes(1 << 40, 1 << 40, 1) == -1


def test_no_device_is_reported(lib):
    try:
        import torch
        if torch.cuda.device_count() > 0:
            pytest.skip("a GPU is present")
    except Exception:
        pass
    assert call(lib) == DEVICE


@pytest.mark.parametrize("pd,status", [(1.0, INVALID), (-0.5, INVALID), (float("nan"), INVALID),
                                       (1 - 2 ** -18, UNSUPPORTED)])
def test_invalid_dropout_rate_rejected_on_host(lib, pd, status):
    a = BASE
    st = lib.sdpa_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["g"], a["lse"], a["dq"], a["dk"],
                              a["dv"], a["w"], 2, 4, 128, 128, 64, 0.125, 0, pd, 1, 0, F16, SAME,
                              SAME, None)
    assert st == status


def test_block_sparse_backward_rejected_on_host():
    from exact_attention_sdpa_amd import _lib
    lib = _lib.lib()
    OK_, INVALID_, UNSUP_, DEVICE_ = 0, 1, 2, 4
    Q, K, V, O, G, L, DQ, DK, DV, W, M = (0x1000000 * (i + 1) for i in range(11))

    def call(mask=M, heads=1, dt=0, w=W):
        return lib.sdpa_bwd_block_sparse(Q, K, V, O, G, L, DQ, DK, DV, w, 2, 4, 256, 256, 64,
                                         0.125, 0, mask, heads, dt, 255, 255, None)
    assert call() in (OK_, DEVICE_)
    assert call(heads=4) in (OK_, DEVICE_)
    assert call(mask=None) == INVALID_
    assert call(heads=3) == INVALID_
    assert call(dt=2) == UNSUP_
    assert call(mask=DQ) == INVALID_        # overlaps an output


def test_noalloc_backward_refuses_sizes_beyond_its_array(lib):
    """sdpa_bwd_noalloc checks the size against its fixed array before any
    device call: B*H*Nq above SDPA_BWD_NOALLOC_MAX_ROWS is unsupported,
    non-positive sizes are invalid."""
    a = BASE
    rows = _lib.SDPA_BWD_NOALLOC_MAX_ROWS

    def call(B, H, Nq):
        return lib.sdpa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["g"], a["lse"], a["dq"],
                                    a["dk"], a["dv"], B, H, Nq, 128, 64, 0.125, 0, F16, SAME,
                                    SAME, None)

    assert call(1, 1, rows + 1) == UNSUPPORTED
    assert call(2, 16, rows // 16) == UNSUPPORTED
    assert call(2 ** 40, 2 ** 40, 2 ** 40) == INVALID     # the byte count overflows
    assert call(0, 1, 128) == INVALID
    assert call(1, 1, 0) == INVALID

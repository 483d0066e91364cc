"""The seeded input generator: determinism, rounding, workload statistics."""
import hashlib

import numpy as np
import pytest
import torch

from exact_attention_sdpa_amd import inputs


def _digest(w):
    h = hashlib.sha256()
    for a in (w.q, w.k, w.v):
        h.update(np.ascontiguousarray(a).tobytes())
    if w.cu_seqlens is not None:
        h.update(w.cu_seqlens.tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    a = inputs.make_dense(2, 3, 17, 17, 32, "bf16", "normal", seed=5, cfg=9)
    b = inputs.make_dense(2, 3, 17, 17, 32, "bf16", "normal", seed=5, cfg=9)
    c = inputs.make_dense(2, 3, 17, 17, 32, "bf16", "normal", seed=6, cfg=9)
    assert _digest(a) == _digest(b) != _digest(c)
    # q, k and v are drawn from different streams
    assert not np.array_equal(a.q, a.k) and not np.array_equal(a.k, a.v)


def test_bf16_rounding_matches_torch():
    """Bit-level round-to-nearest-even agrees with torch's float32->bfloat16
    conversion, including ties and values near overflow."""
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125, -2.5,
                  3.3895314e38, 1e-30, -1e-38, 65504.0, 65520.0], dtype=np.float32),
        # exact ties: low 16 bits == 0x8000 with even and odd kept LSB
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000],
                 dtype=np.uint32).view(np.float32),
    ])
    ours = inputs.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    ours = inputs.bf16_bits_to_f64(finite)
    ref = torch.from_numpy(finite.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_f16_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65519.0, 0.1], dtype=np.float32)
    y = inputs.to_storage(x, "f16")
    assert y.dtype == np.float16
    assert y[0] == np.float16(1.0) and y[1] == np.float16(1.0 + 2 ** -9)
    assert y[2] == np.float16(65504.0)
    assert np.array_equal(inputs.storage_to_f64(y, "f16"), y.astype(np.float64))


def test_uniform_never_reaches_one():
    w = inputs.make_dense(1, 4, 4096, 4096, 32, "f16", "uniform", seed=0, cfg=2)
    for a in (w.q, w.k, w.v):
        assert a.min() >= 0 and a.max() < 1.0


def test_config_shapes_small():
    w1 = inputs.make_config(1)
    assert (w1.B, w1.H, w1.Nq, w1.Nk, w1.d, w1.dtype) == (2, 1, 3, 3, 8, "f32")
    assert w1.q.shape == (2, 1, 3, 8) and w1.q.dtype == np.float32
    assert w1.scale == np.float32(1 / np.sqrt(8)) and not w1.is_causal
    assert w1.flops() == 4 * 2 * 3 * 3 * 8


def test_config4_lengths():
    """The NestedTensor recipe: lengths around 256 with one forced to 512."""
    w = inputs.make_config(4)
    lens = np.diff(w.cu_seqlens.astype(np.int64))
    assert len(lens) == 32 and w.cu_seqlens[0] == 0
    assert lens.max() == 512 and (lens == 512).sum() >= 1
    others = lens[lens != 512]
    assert 240 <= others.min() and others.max() <= 272
    assert 8000 < w.cu_seqlens[-1] < 8900
    assert w.q.shape == (int(w.cu_seqlens[-1]), 8, 64) and w.q.dtype == np.float16
    assert w.Nq == w.Nk == 512 and w.B == 32


@pytest.mark.slow
def test_large_configs_shapes():
    w2 = inputs.make_config(2)
    assert w2.q.shape == (32, 32, 1024, 32) and w2.dtype == "f16"
    assert w2.flops() == pytest.approx(137.438953472e9)
    w3 = inputs.make_config(3)
    assert w3.q.shape == (32, 8, 1024, 64) and w3.is_causal and w3.scale == np.float32(0.125)
    assert w3.flops() == pytest.approx(34.359738368e9)
    w5 = inputs.make_config(5)
    assert w5.q.shape == (1, 16, 65536, 64) and w5.q.dtype == np.uint16
    assert len(w5.rows) == 256 and len(np.unique(w5.rows)) == 256
    assert w5.rows.min() >= 0 and w5.rows.max() < 65536


def test_visible_pairs_counts_the_oracle_visibility():
    """The block-sparse FLOP count equals the number of visible pairs of the
    oracle's visibility matrix (small shapes, ragged blocks, causal)."""
    from oracle import block_sparse as obsp
    for nq, nk, causal, heads in [(300, 200, False, 3), (300, 300, True, 1), (129, 257, True, 2),
                                  (1, 130, False, 1)]:
        m = inputs.make_block_mask(heads, nq, nk, 0.5, seed=nq, cfg=nk)
        want = sum(int(obsp.visibility(nq, nk, m[h], 128, causal).sum()) for h in range(heads))
        assert inputs.visible_pairs(m, nq, nk, causal, heads) == want
        # a one-head mask counts once per head
        assert inputs.visible_pairs(m[:1], nq, nk, causal, 4) == \
            4 * int(obsp.visibility(nq, nk, m[0], 128, causal).sum())


# --- the late-maximum families -------------------------------------------------

def _log2_scores(w, b=0, h=0):
    """Scaled scores of one unit in log2 units, causal pairs set to -inf."""
    s = float(w.scale) * 1.4426950408889634 * (w.q64[b, h] @ w.k64[b, h].T)
    if w.is_causal:
        s = np.where(np.tri(s.shape[0], s.shape[1], dtype=bool), s, -np.inf)
    return s


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rescale_families_move_the_row_maximum(dtype, d, causal):
    """Every family puts a row's maximum well after its first 32 keys: the
    jump over the first block's maximum is >= 20 log2 units (late,
    low_first), and rising scores climb >= 100 log2 units over 2048 keys."""
    for fam, n in (("late", 520), ("low_first", 520), ("rising", 2090)):
        w = inputs.make_rescale(fam, 1, 1, n, n, d, dtype, causal, seed=3, cfg=9)
        s = _log2_scores(w)
        first = np.max(s[:, :32], axis=1)
        later = np.max(s[:, 32:], axis=1)
        rows = np.arange(n) >= 64
        if fam == "rising":
            rows = np.arange(n) >= 2048 if causal else np.ones(n, bool)
            jump = np.max(s[:, 2016:2048], axis=1) - first
            assert np.min(jump[rows]) >= 100, (fam, float(np.min(jump[rows])))
        else:
            jump = later - first
            assert np.min(jump[rows]) >= 20, (fam, float(np.min(jump[rows])))
        assert np.all(np.isfinite(w.q64)) and np.all(np.abs(w.q64) < 1e4)
        assert np.all(np.abs(w.k64) < 1e4)


def test_rescale_packed_families_restart_per_sequence():
    w = inputs.make_rescale("low_first", None, 2, None, None, 64, "f16", True, seed=1, cfg=9,
                            lens=[40, 0, 70])
    cu = w.cu_seqlens
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        k0 = w.k64[a:b, 0, 0]
        if b - a:
            assert np.all(k0[:min(32, b - a)] < -1) and np.all(k0[32:] == 0)

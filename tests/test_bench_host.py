"""Host-side accounting of bench.py (no GPU): the algorithmic bytes the
roofline divides by, the one-GPU refusal, and the rule that stored counter
traffic is only reported for the kernel sources it was measured on.

Expected byte counts are written out from their definition: q, k and v are
read once, the output and the fp32 logsumexp written once, and an
elementwise mask read once at its storage width.
"""
import json
import types

import numpy as np

import bench


def _w(B, H, Nq, Nk, d, dtype="f16", cu=None, mask=None, kind=None):
    return types.SimpleNamespace(B=B, H=H, Nq=Nq, Nk=Nk, d=d, dtype=dtype, varlen=cu is not None,
                                 cu_seqlens=None if cu is None else np.asarray(cu, np.int32),
                                 attn_mask=mask, mask_kind=kind)


def test_headline_bytes():
    # B32 H32 N1024 d32 f16: 3 x 32*32*1024*32 halves read; 32*32*1024 rows of
    # 32 halves + one float written
    r, wr = bench.algorithmic_bytes(_w(32, 32, 1024, 1024, 32))
    assert r == 3 * 32 * 32 * 1024 * 32 * 2 == 201_326_592
    assert wr == 32 * 32 * 1024 * (32 * 2 + 4) == 71_303_168


def test_cross_attention_and_bf16_output():
    # Nq != Nk: q counts Nq rows, k and v Nk rows each; bf16 writes f32 out
    r, wr = bench.algorithmic_bytes(_w(2, 3, 100, 300, 64, dtype="bf16"))
    assert r == (2 * 100 + 2 * 2 * 300) * 3 * 64 * 2
    assert wr == 2 * 100 * 3 * (64 * 4 + 4)


def test_packed_rows_come_from_offsets():
    # two sequences of 5 and 7 tokens: 12 rows, whatever B and N say
    r, wr = bench.algorithmic_bytes(_w(2, 4, 512, 512, 32, cu=[0, 5, 12]))
    assert r == 3 * 12 * 4 * 32 * 2
    assert wr == 12 * 4 * (32 * 2 + 4)


def test_mask_bytes_by_kind():
    add = np.zeros((2, 1, 8, 16), np.uint16)
    boolean = np.zeros((2, 1, 1, 16), np.bool_)
    assert bench.mask_bytes(_w(2, 1, 8, 16, 32, mask=add, kind="add")) == 2 * 8 * 16 * 2
    assert bench.mask_bytes(_w(2, 1, 8, 16, 32, mask=boolean, kind="bool")) == 2 * 16
    assert bench.mask_bytes(_w(2, 1, 8, 16, 32, dtype="f32", mask=add, kind="add")) == 2 * 8 * 16 * 4
    assert bench.mask_bytes(_w(2, 1, 8, 16, 32)) == 0
    # the masked workload's [32, 8, 1024, 1024] f16 bias is 512 MiB
    full = types.SimpleNamespace(size=32 * 8 * 1024 * 1024)
    assert bench.mask_bytes(_w(32, 8, 1024, 1024, 64, mask=full, kind="add")) == 512 << 20
    r, _ = bench.algorithmic_bytes(_w(32, 8, 1024, 1024, 64, mask=full, kind="add"))
    assert r == 3 * 32 * 8 * 1024 * 64 * 2 + (512 << 20)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_code_digest_ignores_comments_and_layout():
    a = "int f(int x) {  // the sum\n  return x + 1; /* one */ }"
    b = "int f(int x) {\n return x + 1;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("return x + 2;") != bench._code_only("return x + 1;")


def test_stored_traffic_needs_matching_sources(tmp_path, monkeypatch):
    rec = {"kernel_sources": "abc", "workloads": {"noncausal": {"bytes_per_launch": 123}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda prefix="fwd_": "abc")
    assert bench.stored_traffic("noncausal") == 123
    assert bench.stored_traffic("causal") is None
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda prefix="fwd_": "changed")
    assert bench.stored_traffic("noncausal") is None

"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that at least one pin catches each of them.

Each mutant replaces the oracle's per-unit routine (or the varlen driver)
with a variant carrying one mistake: a dropped term, a wrong sign, a wrong
index or a transposed operand.
"""
import types

import numpy as np
import pytest

from oracle import sdpa as real
from tests import oracle_pins


def _unit(q, k, v, scale, is_causal, row_ids=None, *, mistake):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if row_ids is None or mistake == "rows_ignored":
        row_ids = np.arange(nq)
    sc = 1.0 if mistake == "scale_dropped" else float(scale)
    if mistake == "scale_squared":
        sc = float(scale) ** 2
    if mistake == "transposed":
        s = sc * (k @ q.T)
    else:
        s = sc * (q @ k.T)
    cols = np.arange(nk)[None, :]
    rows = row_ids[:, None]
    if is_causal:
        allowed = {"causal_strict": cols < rows, "causal_flipped": cols >= rows,
                   "causal_off": np.ones_like(cols >= rows)}.get(mistake, cols <= rows)
        s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s + m) if mistake == "shift_sign" else np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    vv = k if mistake == "k_for_v" else v
    out = e @ vv if mistake == "unnormalised" else (e @ vv) / l
    if mistake == "lse_no_max":
        lse = np.log(l[:, 0])
    elif mistake == "lse_log2":
        lse = m[:, 0] + np.log2(l[:, 0])
    else:
        lse = m[:, 0] + np.log(l[:, 0])
    if mistake == "sum_wrong_axis":
        l0 = np.sum(e, axis=0, keepdims=True)
        out = (e / l0) @ vv
    return out, lse


UNIT_MISTAKES = ["scale_dropped", "scale_squared", "transposed", "causal_strict",
                 "causal_flipped", "causal_off", "shift_sign", "k_for_v", "unnormalised",
                 "lse_no_max", "lse_log2", "sum_wrong_axis", "rows_ignored"]


def _varlen_cross(q, k, v, cu_seqlens, scale, is_causal=False):
    """Mistake: sequences attend across their boundaries (whole packed batch)."""
    T, H, d = q.shape
    O = np.zeros((T, H, d))
    L = np.zeros((T, H))
    for h in range(H):
        O[:, h], L[:, h] = real._attend_unit(q[:, h], k[:, h], v[:, h], scale, is_causal)
    return O, L


def _run_pins(impl):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("mistake", UNIT_MISTAKES)
def test_unit_mutant_is_caught(monkeypatch, mistake):
    monkeypatch.setattr(real, "_attend_unit",
                        lambda *a, **kw: _unit(*a, **kw, mistake=mistake))
    failed = _run_pins(real)
    assert failed, f"mutant {mistake!r} passed every pin"


def test_varlen_mutant_is_caught():
    impl = types.SimpleNamespace(sdpa_fwd=real.sdpa_fwd, sdpa_fwd_rows=real.sdpa_fwd_rows,
                                 sdpa_fwd_varlen=_varlen_cross)
    assert "pin_varlen_concat" in _run_pins(impl)


def test_unmutated_copy_passes_every_pin(monkeypatch):
    """Control: the harness itself does not fail a correct copy."""
    monkeypatch.setattr(real, "_attend_unit",
                        lambda *a, **kw: _unit(*a, **kw, mistake="none"))
    assert _run_pins(real) == []

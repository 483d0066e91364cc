#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the whole forward (sdpa_fwd) over one batch of
synthetic input already resident in device memory.  The default workload is
the one the headline metric is quoted on: B=32, H=32, N=1024, d=32, f16,
uniform [0,1) inputs, non-causal (the PyTorch SDPA tutorial's dispatcher
benchmark).  Prints one JSON line.  The default run also times, after the
headline's timed region, the two d = 64 causal workloads (B32 H8 N1024 f16
and B1 H16 N65536 bf16) under ``targets``, each with the same event method.

Throughput counts 4*B*H*Nq*Nk*d FLOPs per step (halved when causal; summed
per sequence for packed batches; 4*d per visible (query, key) pair for the
block-sparse workload, which calls sdpa_fwd_block_sparse; every pair for the
elementwise-mask workloads, which call sdpa_fwd_masked and compute every
pair).  `--dropout P`
times sdpa_fwd_dropout instead (sdpa_fwd_masked_dropout on the
elementwise-mask workloads; same FLOPs).  `roofline.achieved` divides the
same FLOPs by the kernel's own average duration from HIP events recorded around
each launch on the launch stream; the peak is MI355X's published dense
fp16/bf16 matrix rate, 2.5 PFLOP/s.  `cpu_baseline` times the fp64 CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused SDPA fwd TFLOP/s + % of MFMA fp16 peak (B32 H32 N1024 d32)"
METRIC_BWD = "fused SDPA bwd TFLOP/s (2.5x forward FLOPs) + % of MFMA fp16 peak"
PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak (published)
# the tutorial's flash-backend time for B32 H32 N1024 d32 fp16 (hardware
# unstated): 2262.901 us -> 4*32*32*1024*1024*32 / 2262.901e-6 = 60.74 TFLOP/s
PAGES_FLASH_TFLOPS = 137.438953472e9 / 2262.901e-6 / 1e12

WORKLOADS = {"noncausal": 2, "causal": 3, "varlen": 4, "long": 5, "block_sparse": 6,
             "masked": 7, "padded": 8}
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E (published)


def _code_only(src: str) -> str:
    """C++ source with comments removed and whitespace collapsed (the kernel
    sources hold no string literals that contain comment markers)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_sources_digest(prefix: str = "fwd_") -> str:
    """Hash of the code (comments and layout ignored) of one kernel family's
    HIP sources (file names starting with ``prefix``; the forward's by
    default), used to tell whether stored counter results still describe the
    current kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_sdpa_amd", "csrc")
    shared = ("philox.h",)   # included by both kernel families
    for name in sorted(os.listdir(csrc)):
        if (name.startswith(prefix) or name in shared) and name.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(csrc, name)) as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("workloads", {}).get(workload)
    if not ent or rec.get("kernel_sources") != kernel_sources_digest():
        return None
    return ent.get("bytes_per_launch")


def describe(w, name, dropout=0.0):
    cfg = {"workload": f"{name}: B{w.B} H{w.H} Nq{w.Nq} Nk{w.Nk} d{w.d} {w.dtype}"
                       f"{' causal' if w.is_causal else ''}{' packed' if w.varlen else ''}",
           "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.is_causal,
           "inputs": "uniform [0,1)" if name == "noncausal" else "normal(0,1)"}
    if w.varlen:
        cfg["total_rows"] = int(w.cu_seqlens[-1])
    if dropout > 0:
        cfg["workload"] += f" dropout p={dropout:g}"
        cfg["dropout_p"] = dropout
    if w.block_mask is not None:
        cfg["workload"] += " block-sparse"
        cfg["block_mask"] = (f"{w.block_mask.shape[0]} x {w.block_mask.shape[1]} x "
                             f"{w.block_mask.shape[2]} blocks of 128x128, p=1/4 + diagonal, "
                             f"{100 * float(w.block_mask.mean()):.2f}% kept")
    if w.attn_mask is not None:
        import numpy as np

        from exact_attention_sdpa_amd import inputs
        shape = "x".join(str(x) for x in w.attn_mask.shape)
        cfg["workload"] += f" {w.mask_kind} mask [{shape}]"
        cfg["attn_mask"] = (f"{w.mask_kind} [{shape}]"
                            + (f" {w.dtype}, N(0,2), {100 * float(np.mean(np.isneginf(inputs.storage_to_f64(w.attn_mask, w.dtype)))):.1f}% -inf"
                               if w.mask_kind == "add" else
                               f", {100 * float(np.mean(w.attn_mask)):.1f}% of keys kept"))
    return cfg


def mask_bytes(w) -> int:
    """Bytes of the elementwise mask as stored (read once per launch)."""
    if w.attn_mask is None:
        return 0
    return int(w.attn_mask.size) * (1 if w.mask_kind == "bool" else
                                    (4 if w.dtype == "f32" else 2))


def algorithmic_bytes(w):
    """(read, written) bytes per launch: q, k, v and the mask read once; out
    and lse written once (bf16 inputs write an f32 out)."""
    el = 2 if w.dtype != "f32" else 4
    rows_q = int(w.cu_seqlens[-1]) if w.varlen else w.B * w.Nq
    rows_k = int(w.cu_seqlens[-1]) if w.varlen else w.B * w.Nk
    out_el = 4 if w.dtype == "bf16" else el
    return ((rows_q + 2 * rows_k) * w.H * w.d * el + mask_bytes(w),
            rows_q * w.H * (w.d * out_el + 4))


def cpu_baseline(w, budget_s: float, dropout: float = 0.0):
    """Time the fp64 oracle on whole (batch, head) units of the workload
    until about `budget_s` seconds of CPU work, and scale to TFLOP/s (the
    dropout oracle when ``dropout`` > 0)."""
    import numpy as np

    import oracle
    from exact_attention_sdpa_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    if w.block_mask is not None:
        return _cpu_baseline_block_sparse(w, budget_s, threads)
    if w.attn_mask is not None:
        return _cpu_baseline_masked(w, budget_s, threads, dropout)
    if dropout > 0:
        return _cpu_baseline_dropout(w, budget_s, threads, dropout)
    flops = 0.0
    n = 0
    t0 = time.perf_counter()
    if w.varlen:
        cu = w.cu_seqlens.astype(np.int64)
        units = [(s, h) for s in range(w.B) for h in range(w.H)]
    else:
        units = [(b, h) for b in range(w.B) for h in range(w.H)]
    for (a, h) in units:
        if w.varlen:
            s0, s1 = int(cu[a]), int(cu[a + 1])
            dec = lambda x: inputs.storage_to_f64(x[s0:s1, h:h + 1], w.dtype).transpose(1, 0, 2)[None]
            nq = nk = s1 - s0
        else:
            dec = lambda x: inputs.storage_to_f64(x[a:a + 1, h:h + 1], w.dtype)
            nq, nk = w.Nq, w.Nk
        if w.Nq > 8192:   # long sequences: a block of 256 query rows per unit
            rows = np.arange(nk - 256, nk)
            oracle.sdpa_fwd_rows(dec(w.q), dec(w.k), dec(w.v), w.scale, w.is_causal, rows)
            f = 4.0 * w.d * (float(np.sum(rows + 1)) if w.is_causal else 256.0 * nk)
        else:
            oracle.sdpa_fwd(dec(w.q), dec(w.k), dec(w.v), w.scale, w.is_causal)
            f = 4.0 * nq * nk * w.d / (2 if w.is_causal else 1)
        flops += f
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    sample = f"{n} of {len(units)} (batch, head) units"
    if w.Nq > 8192:
        sample += ", last 256 query rows each"
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle", "sample": sample, "seconds": round(dt, 2),
           "host_cpus": len(os.sched_getaffinity(0))}
    # the whole workload at the sampled rate (scaled by FLOPs: the oracle's
    # time grows with the pairs it computes)
    rec["full_workload_seconds_extrapolated"] = round(dt * w.flops() / flops, 1)
    return rec


def _cpu_baseline_block_sparse(w, budget_s, threads):
    """The fp64 block-sparse oracle on the last 256 query rows of each
    (batch, head) unit in turn, FLOPs counted over the visible pairs."""
    import numpy as np

    from exact_attention_sdpa_amd import inputs
    from oracle import block_sparse as obsp
    rows = np.arange(w.Nq - 256, w.Nq)
    flops, n = 0.0, 0
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    t0 = time.perf_counter()
    for (b, h) in units:
        m = w.block_mask[h if w.block_mask.shape[0] == w.H else 0]
        vis = obsp.visibility(w.Nq, w.Nk, m, 128, w.is_causal, rows)
        q = inputs.storage_to_f64(w.q[b, h, rows], w.dtype)
        k = inputs.storage_to_f64(w.k[b, h], w.dtype)
        v = inputs.storage_to_f64(w.v[b, h], w.dtype)
        obsp.attend_masked(q, k, v, w.scale, vis)
        flops += 4.0 * w.d * float(vis.sum())
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{n} of {len(units)} (batch, head) units, last 256 "
                                        f"query rows each",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0))}


def _cpu_baseline_masked(w, budget_s, threads, dropout=0.0):
    """The fp64 masked oracle (the mask-with-dropout one when ``dropout`` >
    0) on whole (batch, head) units in turn, FLOPs counted as the metric
    does (every pair)."""
    import numpy as np

    from exact_attention_sdpa_amd import inputs
    from oracle import dropout as odrop
    from oracle import masked as om
    m = w.attn_mask
    m = m.reshape((1,) * (4 - m.ndim) + m.shape)
    flops, n = 0.0, 0
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    t0 = time.perf_counter()
    for b, h in units:
        dec = lambda x: inputs.storage_to_f64(x[b:b + 1, h:h + 1], w.dtype)
        mu = m[b % m.shape[0], h % m.shape[1]]
        mu = mu if w.mask_kind == "bool" else inputs.storage_to_f64(mu, w.dtype)
        mu = np.broadcast_to(mu, (w.Nq, w.Nk))
        if dropout > 0:
            odrop.sdpa_fwd_masked_dropout(dec(w.q), dec(w.k), dec(w.v), mu[None, None],
                                          w.mask_kind, w.scale, w.is_causal, dropout, 2023)
        else:
            om.sdpa_fwd_masked(dec(w.q), dec(w.k), dec(w.v), mu[None, None], w.mask_kind,
                               w.scale, w.is_causal)
        flops += 4.0 * w.Nq * w.Nk * w.d / (2 if w.is_causal else 1)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{n} of {len(units)} (batch, head) units",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0))}


def _cpu_baseline_dropout(w, budget_s, threads, p):
    """The fp64 dropout oracle on whole (batch, head) units (dense
    workloads of at most 8192 rows)."""
    from exact_attention_sdpa_amd import inputs
    from oracle import dropout as odrop
    if w.varlen or w.Nq * w.Nk > (1 << 26):
        return None
    flops, n = 0.0, 0
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    t0 = time.perf_counter()
    for (b, h) in units:
        dec = lambda x: inputs.storage_to_f64(x[b, h], w.dtype)
        odrop.attend_dropout(dec(w.q), dec(w.k), dec(w.v), w.scale, w.is_causal, p, 1, 0,
                             b * w.H + h)
        flops += 4.0 * w.Nq * w.Nk * w.d / (2 if w.is_causal else 1)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{n} of {len(units)} (batch, head) units",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_bwd(w, budget_s, cfg, dropout=0.0):
    """The fp64 gradient oracle on whole (batch, head) units of the workload,
    until about ``budget_s`` seconds have passed (same FLOP convention as
    the GPU line).  None for sequences too long to hold a unit's N x N
    matrices in host memory."""
    import numpy as np
    import oracle
    from exact_attention_sdpa_amd import inputs
    if w.Nq * w.Nk > (1 << 26):
        return None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    do = inputs.make_grad_out(w, cfg=cfg)
    flops, n = 0.0, 0
    t0 = time.perf_counter()
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    for (b, h) in units:
        if w.varlen:   # (sequence, head) units of the packed batch
            s0, s1 = int(w.cu_seqlens[b]), int(w.cu_seqlens[b + 1])
            dec = lambda x: inputs.storage_to_f64(x[s0:s1, h], w.dtype)
            if dropout > 0:
                oracle.attention_grads_dropout(dec(w.q), dec(w.k), dec(w.v), dec(do), w.scale,
                                               w.is_causal, dropout, 2023, 0, b * w.H + h)
            else:
                oracle.attention_grads(dec(w.q), dec(w.k), dec(w.v), dec(do), w.scale,
                                       w.is_causal)
            flops += 2.5 * 4.0 * (s1 - s0) ** 2 * w.d / (2 if w.is_causal else 1)
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
            continue
        dec = lambda x: inputs.storage_to_f64(x[b:b + 1, h:h + 1], w.dtype)
        if w.attn_mask is not None:   # the masked gradient oracle on the unit's mask
            m4 = w.attn_mask.reshape((1,) * (4 - w.attn_mask.ndim) + w.attn_mask.shape)
            mu = m4[b % m4.shape[0], h % m4.shape[1]]
            mu = mu if w.mask_kind == "bool" else inputs.storage_to_f64(mu, w.dtype)
            mu = np.broadcast_to(mu, (w.Nq, w.Nk))[None, None]
            if dropout > 0:
                oracle.sdpa_bwd_masked_dropout(dec(w.q), dec(w.k), dec(w.v), dec(do), mu,
                                               w.mask_kind, w.scale, w.is_causal, dropout, 2023)
            else:
                oracle.sdpa_bwd_masked(dec(w.q), dec(w.k), dec(w.v), dec(do), mu, w.mask_kind,
                                       w.scale, w.is_causal)
        elif dropout > 0:
            oracle.sdpa_bwd_dropout(dec(w.q), dec(w.k), dec(w.v), dec(do), w.scale, w.is_causal,
                                    dropout, 2023, 0)
        else:
            oracle.sdpa_bwd(dec(w.q), dec(w.k), dec(w.v), dec(do), w.scale, w.is_causal)
        flops += 2.5 * 4.0 * w.Nq * w.Nk * w.d / (2 if w.is_causal else 1)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} of {len(units)} ({'sequence' if w.varlen else 'batch'}, head) units",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0))}


def copy_calibration(torch) -> int:
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / 5
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n,
                      "ms_per_copy": round(ms, 4), "GBps": round(2 * n / ms / 1e6, 1)}))
    return 0


def gemm_calibration(torch) -> int:
    """Attainable matrix-core rate for reference: the vendor BLAS (torch.mm on
    ROCm: hipBLASLt) on square 8192 GEMMs, fp16 and bf16, fp32 accumulate."""
    n = 8192
    for dt in (torch.float16, torch.bfloat16):
        a = torch.randn(n, n, device="cuda").to(dt)
        b = torch.randn(n, n, device="cuda").to(dt)
        for _ in range(3):
            torch.mm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            torch.mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"calibration": "gemm", "dtype": str(dt).replace("torch.", ""),
                          "m": n, "n": n, "k": n, "ms": round(ms, 4),
                          "TFLOPs": round(tf, 1),
                          "pct_of_peak": round(100.0 * tf / PEAK_TFLOPS, 1)}))
    return 0


def _csv_rows(d, name):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", f"*{name}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{name} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_kib(d, kernel_match):
    vals = [float(r["Counter_Value"]) for r in _csv_rows(d, "counter_collection.csv")
            if kernel_match in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no dispatch matching {kernel_match!r} in {d}")
    return sum(vals) / len(vals), len(vals)


# SQ counters of the forward kernel, from two rocprofv3 --pmc passes (the
# per-pass limit is 8 SQ counters) on the same workload:
SQ_PASS_A = ("SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
             "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_LDS")
SQ_PASS_B = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_WAIT_INST_LDS "
             "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_ANY SQ_CYCLES GRBM_GUI_ACTIVE")
SIMDS = 1024          # 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9      # the clock the published peak assumes


def _counters_by_name(d, kernel_match):
    """Average per dispatch of each counter over the matching dispatches."""
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in _csv_rows(d, "counter_collection.csv"):
        if kernel_match in r["Kernel_Name"]:
            per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch matching {kernel_match!r} in {d}")
    return {n: sum(v.values()) / len(v) for n, v in per.items()}


def issue_shares(c, avg_ns):
    """Shares of the SIMD-cycles (1024 SIMDs x duration x 2.4 GHz) in which
    the matrix cores are busy (SQ_VALU_MFMA_BUSY_CYCLES), the vector unit
    issues (4 x SQ_ACTIVE_INST_VALU: the counter ticks once per 4-cycle
    issue of a wave64 instruction), and both at once
    (SQ_VALU_MFMA_COEXEC_CYCLES); the larger of the first two names the
    binding unit."""
    cyc = SIMDS * avg_ns * 1e-9 * CLOCK_HZ
    mf = c["SQ_VALU_MFMA_BUSY_CYCLES"] / cyc
    va = 4.0 * c["SQ_ACTIVE_INST_VALU"] / cyc
    co = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / cyc
    return {"mfma_busy_share": round(mf, 3), "valu_issue_share": round(va, 3),
            "coexec_share": round(co, 3), "idle_share": round(max(0.0, 1.0 - mf - va + co), 3),
            "valu_per_mfma": round(c["SQ_INSTS_VALU"] / max(c["SQ_INSTS_MFMA"], 1.0), 2),
            "lds_bank_conflicts": c.get("SQ_LDS_BANK_CONFLICT", 0.0),
            "binding": "vector issue" if va > mf else "matrix core"}


def stored_counters(workload: str):
    """Issue shares from the committed SQ-counter record, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "sq_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources") != kernel_sources_digest():
        return None
    return rec.get("workloads", {}).get(workload)


def summarize_counters(a) -> int:
    """profiles/sq_counters.json (and its text form) from the kernel-trace
    run and the two SQ-counter passes of one workload."""
    stats = _csv_rows(a.trace_dir, "kernel_stats.csv")
    ker = [r for r in stats if "fwd_mfma" in r["Name"]]
    k = max(ker, key=lambda r: float(r["TotalDurationNs"]))
    avg_ns = float(k["AverageNs"])
    c = _counters_by_name(a.ctr_a_dir, "fwd_mfma")
    c.update(_counters_by_name(a.ctr_b_dir, "fwd_mfma"))
    sh = issue_shares(c, avg_ns)
    path = os.path.join(ROOT, "profiles", "sq_counters.json")
    rec = {"kernel_sources": kernel_sources_digest(), "workloads": {}}
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f)
        if old.get("kernel_sources") == rec["kernel_sources"]:
            rec = old
    rec["workloads"][a.workload] = dict(sh, avg_kernel_us=round(avg_ns / 1e3, 3),
                                        counters={n: c[n] for n in sorted(c)})
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    lines = [f"# fwd_mfma: issue counters (SQ_*) of the forward kernel",
             "",
             "commands (two passes per workload, one counter set each):",
             f"  rocprofv3 --pmc {SQ_PASS_A} -f csv -d <dir> -o run -- python3 bench.py "
             "--workload W --steps 3 --warmup 1 --cpu-budget 0 --cold-reps 0 --no-targets",
             f"  rocprofv3 --pmc {SQ_PASS_B} (same program)",
             "values: per dispatch of the attention kernel, averaged over the dispatches; whole GPU.",
             "shares: of 1024 SIMDs x the kernel-trace average duration x 2.4 GHz; vector issue",
             "counts 4 cycles per SQ_ACTIVE_INST_VALU tick (a wave64 instruction on a 16-lane SIMD);",
             "one 32x32x16 MFMA keeps the matrix core busy 32 cycles.  'bound by' names the unit",
             "with the larger share; 'neither' is time lost to waits (memory, LDS, barriers).", ""]
    for wl, e in sorted(rec["workloads"].items()):
        lines += [f"## {wl} (kernel average {e['avg_kernel_us']:.1f} us from the kernel-trace profile)"]
        lines += [f"  {n:28s} {v:.4g}" for n, v in e["counters"].items()]
        c = e["counters"]
        lines += [f"  32 x SQ_INSTS_MFMA / SQ_VALU_MFMA_BUSY_CYCLES: "
                  f"{32 * c['SQ_INSTS_MFMA'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}",
                  f"  co-executing share of matrix-busy cycles: "
                  f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.2f}",
                  f"  VALU instructions per MFMA: {e['valu_per_mfma']}",
                  f"  share of SIMD-cycles: matrix core busy {e['mfma_busy_share']}, vector issue "
                  f"{e['valu_issue_share']}, both at once {e['coexec_share']}, neither "
                  f"{e['idle_share']} -> bound by {e['binding']}", ""]
    lines.append(f"kernel sources digest: {kernel_sources_digest()}")
    with open(os.path.join(ROOT, "profiles", "fwd_mfma_sq_counters.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def summarize_bwd(a) -> int:
    """Turn the rocprofv3 kernel trace of a backward run (bench.py --pass bwd)
    into profiles/bwd_<workload>[_dropout].txt: each backward kernel's
    average duration and share, and the pass's TFLOP/s from their sum."""
    stats = _csv_rows(a.trace_dir, "kernel_stats.csv")
    ker = [r for r in stats if "bwd_" in r["Name"] or "fwd_mfma" in r["Name"]]
    if not ker:
        raise SystemExit("no attention kernel in the kernel trace")
    from exact_attention_sdpa_amd import inputs
    w = inputs.make_config(WORKLOADS[a.workload])
    short = lambda n: n.split("(")[0].replace("void ", "").replace("sdpa::", "")
    bwd = [r for r in ker if "bwd_" in r["Name"]]
    total_us = sum(float(r["AverageNs"]) for r in bwd) / 1e3
    flops = 2.5 * w.flops()
    tag = f"bwd_{a.workload}" + ("_dropout" if a.dropout > 0 else "")
    dflag = f" --dropout {a.dropout:g}" if a.dropout > 0 else ""
    txt = [f"# {tag}: rocprofv3 summary of the backward pass, workload "
           f"{describe(w, a.workload, a.dropout)['workload']}", "",
           f"  command: rocprofv3 --kernel-trace --stats -f csv -d <dir> -o run -- python3 bench.py "
           f"--pass bwd --workload {a.workload}{dflag} --steps {a.steps} --warmup {a.warmup} "
           f"--cpu-budget 0 --cold-reps 0 --no-targets",
           "  (the forward runs once first to produce out and lse; it is listed for completeness)",
           "", f"{'kernel':62s}{'calls':>7s}{'average us':>13s}   share of backward"]
    for r in sorted(ker, key=lambda r: -float(r["TotalDurationNs"])):
        us = float(r["AverageNs"]) / 1e3
        share = f"{100 * us / total_us:9.1f}%" if "bwd_" in r["Name"] else "        -"
        txt.append(f"  {short(r['Name'])[:60]:60s}{r['Calls']:>7s}{us:13.2f}  {share}")
    txt += ["", f"backward FLOPs per call (2.5x the forward's {w.flops():.4g}): {flops:.3g}",
            f"sum of the backward kernels' averages: {total_us:.2f} us -> "
            f"{flops / total_us / 1e6:.1f} TFLOP/s ({100 * flops / total_us / 1e6 / PEAK_TFLOPS:.1f}% "
            f"of {PEAK_TFLOPS:.0f})", "",
            f"kernel sources digest (bwd_*): {kernel_sources_digest('bwd_')}"]
    with open(os.path.join(ROOT, "profiles", f"{tag}.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")
    print("\n".join(txt))
    return 0


def summarize(a) -> int:
    """Turn rocprofv3 outputs of the commands printed below into the text
    summary profiles/<kernel>_<workload>.txt and the HBM-traffic record
    profiles/hbm_traffic.json that the benchmark line reports.

    FETCH_SIZE / WRITE_SIZE are scaled by what the same counters read for a
    plain copy of 1 GiB (bench.py --calibrate-copy), so that a counter
    that sees only part of the memory channels still yields bytes."""
    stats = _csv_rows(a.trace_dir, "kernel_stats.csv")
    ker = [r for r in stats if "fwd_mfma" in r["Name"] or "fwd_f32" in r["Name"]]
    if not ker:
        raise SystemExit("no attention kernel in the kernel trace")
    k = max(ker, key=lambda r: float(r["TotalDurationNs"]))
    avg_ns = float(k["AverageNs"])
    fetch, nf = _counter_kib(a.fetch_dir, "fwd_mfma")
    write, nw = _counter_kib(a.write_dir, "fwd_mfma")
    cfetch, _ = _counter_kib(a.copy_fetch_dir, "copyBuffer")
    cwrite, _ = _counter_kib(a.copy_write_dir, "copyBuffer")
    gib_kib = float(1 << 20)
    ffac, wfac = gib_kib / cfetch, gib_kib / cwrite
    read_b = fetch * ffac * 1024
    write_b = write * wfac * 1024
    from exact_attention_sdpa_amd import inputs
    w = inputs.make_config(WORKLOADS[a.workload])
    alg_read, alg_write = algorithmic_bytes(w)
    name = k["Name"].split("(")[0].replace("void ", "").replace("sdpa::", "")
    tag = f"fwd_mfma_{a.workload}" + ("_dropout" if a.dropout > 0 else "")
    dflag = f" --dropout {a.dropout:g}" if a.dropout > 0 else ""
    txt = [
        f"# {tag}: rocprofv3 summary, workload {describe(w, a.workload, a.dropout)['workload']}",
        "",
        "Kernel trace (average over the profiled launches):",
        f"  command: rocprofv3 --kernel-trace --stats -f csv -d <dir> -o run -- "
        f"python3 bench.py --workload {a.workload}{dflag} --steps {a.steps} --warmup {a.warmup} "
        f"--cpu-budget 0 --cold-reps 0 --no-targets",
        f"  kernel:  {k['Name']}",
        f"  calls {k['Calls']}  average {avg_ns / 1e3:.2f} us  min {float(k['MinNs']) / 1e3:.2f} us"
        f"  max {float(k['MaxNs']) / 1e3:.2f} us",
        f"  metric FLOPs per launch {w.flops():.6g} -> {w.flops() / avg_ns / 1e3:.1f} TFLOP/s at the "
        f"average duration ({100 * w.flops() / avg_ns / 1e3 / PEAK_TFLOPS:.1f}% of {PEAK_TFLOPS:.0f})",
        "",
        "HBM traffic (separate counter passes, one counter block each):",
        f"  commands: rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o run -- python3 bench.py "
        f"--workload {a.workload}{dflag} --steps 5 --warmup 1 --cpu-budget 0 --cold-reps 0 "
        "--no-targets",
        "            rocprofv3 --pmc WRITE_SIZE (same program)",
        "            rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE -- python3 bench.py --calibrate-copy",
        f"  copy of 1 GiB reads FETCH_SIZE {cfetch:.0f} KiB, WRITE_SIZE {cwrite:.0f} KiB"
        f" -> scale factors {ffac:.4f} (fetch), {wfac:.4f} (write)",
        f"  kernel: FETCH_SIZE {fetch:.0f} KiB/dispatch ({nf} dispatches), WRITE_SIZE {write:.0f} "
        f"KiB/dispatch ({nw})",
        f"  -> {read_b / 1e6:.2f} MB read + {write_b / 1e6:.2f} MB written per launch",
        f"  algorithmic (q,k,v{', mask' if w.attn_mask is not None else ''} read once; out and lse written once): {alg_read / 1e6:.2f} MB read + "
        f"{alg_write / 1e6:.2f} MB written",
        f"  measured / algorithmic: read {read_b / alg_read:.3f}, write {write_b / alg_write:.3f}",
        f"  achieved HBM rate at the average duration: {(read_b + write_b) / avg_ns:.1f} GB/s",
        "",
        f"kernel sources digest: {kernel_sources_digest()}",
    ]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{tag}.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    rec = {"kernel_sources": kernel_sources_digest(), "workloads": {}}
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f)
        if old.get("kernel_sources") == rec["kernel_sources"]:
            rec = old
    rec["workloads"][a.workload + ("_dropout" if a.dropout > 0 else "")] = {
        "bytes_per_launch": round(read_b + write_b), "read_bytes": round(read_b),
        "write_bytes": round(write_b), "algorithmic_bytes": alg_read + alg_write,
        "avg_kernel_us": round(avg_ns / 1e3, 3), "fetch_scale": round(ffac, 5),
        "write_scale": round(wfac, 5), "kernel": name}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print("\n".join(txt))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="noncausal", choices=sorted(WORKLOADS))
    ap.add_argument("--pass", dest="which", default="fwd", choices=("fwd", "bwd"),
                    help="time the forward (default, the headline metric) or the backward "
                         "pass (sdpa_bwd: dQ, dK, dV; dense workloads)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout rate on the attention weights (sdpa_fwd_dropout on dense and "
                         "packed workloads, sdpa_fwd_masked_dropout on masked ones)")
    ap.add_argument("--cold-reps", type=int, default=None,
                    help="launches timed with cold caches (a 512 MiB write before each); "
                         "default 50, 10 for the 64k-token workloads, 0 = skip")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU work for the oracle baseline (0 = skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (5 times), the "
                         "reference for scaling HBM byte counters")
    ap.add_argument("--calibrate-gemm", action="store_true",
                    help="run only square 8192 fp16/bf16 GEMMs through the vendor BLAS, "
                         "an attainable matrix-core rate for reference")
    ap.add_argument("--no-targets", dest="targets", action="store_false",
                    help="skip timing the causal and long workloads after the headline")
    ap.add_argument("--summarize-counters", action="store_true",
                    help="write profiles/sq_counters.json from --trace-dir, --ctr-a-dir, "
                         "--ctr-b-dir (rocprofv3 outputs of the SQ_PASS_A / SQ_PASS_B sets)")
    ap.add_argument("--ctr-a-dir")
    ap.add_argument("--ctr-b-dir")
    ap.add_argument("--summarize", action="store_true",
                    help="summarize rocprofv3 CSV outputs into profiles/ (no GPU needed)")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    a = ap.parse_args(argv)
    if a.cold_reps is None:
        a.cold_reps = 10 if a.workload in ("long", "block_sparse") else 50
    if a.summarize_counters:
        return summarize_counters(a)
    if a.summarize:
        return summarize_bwd(a) if a.which == "bwd" else summarize(a)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the path shards by (batch, head) "
              "with no exchange, so --gpus N > 1 is not measured here.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import exact_attention_sdpa_amd as sdpa
    from exact_attention_sdpa_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if a.calibrate_copy:
        return copy_calibration(torch)
    if a.calibrate_gemm:
        return gemm_calibration(torch)
    w = inputs.make_config(WORKLOADS[a.workload])

    def up(x):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    q, k, v = up(w.q), up(w.k), up(w.v)
    out_f32 = w.dtype == "bf16"  # bf16 inputs: f32 output (one bf16 rounding exceeds 1e-3)
    out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device="cuda")
    lse_shape = (q.shape[0], q.shape[1]) if w.varlen else tuple(q.shape[:3])
    lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda")
    cu = torch.from_numpy(w.cu_seqlens).cuda() if w.varlen else None
    dt = {"f16": sdpa.SDPA_F16, "bf16": sdpa.SDPA_BF16, "f32": sdpa.SDPA_F32}[w.dtype]
    odt = sdpa.SDPA_F32 if out_f32 else sdpa.SDPA_SAME
    H = w.H
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    L = sdpa._lib.lib()
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), w.B, H,
            w.Nq, w.Nk, w.d, float(w.scale), int(w.is_causal),
            cu.data_ptr() if cu is not None else None, dt, odt, handle]

    def step():
        st = L.sdpa_fwd(*args)
        if st != 0:
            raise sdpa.SdpaError(st)

    if a.dropout > 0:
        if w.block_mask is not None:
            print("bench.py: dropout with a block mask is not supported", file=sys.stderr)
            return 2
        dargs = args[:13] + [float(a.dropout), 2023, 0, dt, odt, handle]

        def step():  # noqa: F811 -- the dropout entry point
            st = L.sdpa_fwd_dropout(*dargs)
            if st != 0:
                raise sdpa.SdpaError(st)

    if w.block_mask is not None:
        bm = torch.from_numpy(np.ascontiguousarray(w.block_mask)).cuda()
        sargs = args[:12] + [bm.data_ptr(), int(bm.shape[0]), dt, odt, handle]

        def step():  # noqa: F811 -- the block-sparse entry point
            st = L.sdpa_fwd_block_sparse(*sargs)
            if st != 0:
                raise sdpa.SdpaError(st)

    if w.attn_mask is not None:
        import ctypes
        m = w.attn_mask
        m = m.reshape((1,) * (4 - m.ndim) + m.shape)
        mt = (torch.from_numpy(np.ascontiguousarray(m)).cuda() if w.mask_kind == "bool"
              else up(m))
        mstr = tuple(st if n > 1 else 0 for st, n in zip(mt.stride()[:3], mt.shape[:3]))
        mstr_c = (ctypes.c_int64 * 3)(*mstr)
        mkind = sdpa.SDPA_MASK_BOOL if w.mask_kind == "bool" else sdpa.SDPA_MASK_ADD
        margs = args[:10] + [None, None, None, float(w.scale), int(w.is_causal), mt.data_ptr(),
                             mkind, ctypes.cast(mstr_c, ctypes.c_void_p), dt, odt, handle]

        def step():  # noqa: F811 -- the elementwise-mask entry point
            st = L.sdpa_fwd_masked(*margs)
            if st != 0:
                raise sdpa.SdpaError(st)

        if a.dropout > 0:
            mdargs = margs[:18] + [float(a.dropout), 2023, 0] + margs[18:]

            def step():  # noqa: F811 -- the mask-with-dropout entry point
                st = L.sdpa_fwd_masked_dropout(*mdargs)
                if st != 0:
                    raise sdpa.SdpaError(st)

    if a.which == "bwd":
        step()   # the forward's out and lse feed the backward
        g = up(inputs.make_grad_out(w, cfg=WORKLOADS[a.workload]))
        gdt = torch.float32 if out_f32 else q.dtype
        dq, dk, dv = (torch.empty(x.shape, dtype=gdt, device="cuda") for x in (q, k, v))
        work = torch.empty(lse.shape, dtype=torch.float32, device="cuda")
        bargs = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), g.data_ptr(),
                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), work.data_ptr(),
                 w.B, H, w.Nq, w.Nk, w.d, float(w.scale), int(w.is_causal), dt, odt,
                 sdpa.SDPA_F32 if out_f32 else sdpa.SDPA_SAME, handle]

        if a.dropout > 0:   # the forward above ran with the same dropout contract
            bargs = bargs[:17] + [float(a.dropout), 2023, 0] + bargs[17:]

        def step():  # noqa: F811 -- the timed step is the backward call
            st = (L.sdpa_bwd_dropout if a.dropout > 0 else L.sdpa_bwd)(*bargs)
            if st != 0:
                raise sdpa.SdpaError(st)

        if w.block_mask is not None:   # the block-sparse backward, same mask
            bsargs = bargs[:17] + [bm.data_ptr(), int(bm.shape[0]), dt, odt,
                                   sdpa.SDPA_F32 if out_f32 else sdpa.SDPA_SAME, handle]

            def step():  # noqa: F811 -- the block-sparse backward
                st = L.sdpa_bwd_block_sparse(*bsargs)
                if st != 0:
                    raise sdpa.SdpaError(st)

        if w.attn_mask is not None:   # the elementwise-mask backward, same mask layout
            margs_b = bargs[:17] + [mt.data_ptr(), mkind, ctypes.cast(mstr_c, ctypes.c_void_p),
                                    dt, odt, sdpa.SDPA_F32 if out_f32 else sdpa.SDPA_SAME,
                                    handle]

            def step():  # noqa: F811 -- the masked backward
                st = L.sdpa_bwd_masked(*margs_b)
                if st != 0:
                    raise sdpa.SdpaError(st)

            if a.dropout > 0:
                mdargs_b = margs_b[:20] + [float(a.dropout), 2023, 0] + margs_b[20:]

                def step():  # noqa: F811 -- the mask-with-dropout backward
                    st = L.sdpa_bwd_masked_dropout(*mdargs_b)
                    if st != 0:
                        raise sdpa.SdpaError(st)

        if w.varlen:
            T = int(w.cu_seqlens[-1])
            pargs = bargs[:10] + [w.B, H, T, w.Nq, w.d, float(w.scale), int(w.is_causal),
                                  cu.data_ptr(), float(a.dropout), 2023, 0, dt, odt,
                                  sdpa.SDPA_F32 if out_f32 else sdpa.SDPA_SAME, handle]

            def step():  # noqa: F811 -- the packed-batch backward
                st = L.sdpa_bwd_packed(*pargs)
                if st != 0:
                    raise sdpa.SdpaError(st)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches between one pair of events on
    # the launch stream; the event span / K is the kernel's average duration
    # (its launch gaps included, as the steps run back to back).
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(a.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kmean = t_start.elapsed_time(t_end) / a.steps

    # Per-launch spread, from a separate untimed pass with events around
    # each launch.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(a.steps, 50))]
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    kern_ms = [e0.elapsed_time(e1) for e0, e1 in ev]

    # Cold caches: before each of these launches a 512 MiB write evicts L2
    # and the Infinity Cache (256 MB); the events bracket the attention
    # launch only.  Untimed by the step clock.
    kern_cold = []
    if a.cold_reps > 0:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(a.cold_reps)]
        for i, (e0, e1) in enumerate(evc):
            scrub.fill_(i & 0xff)
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        kern_cold = [e0.elapsed_time(e1) for e0, e1 in evc]
        del scrub

    # backward: the usual convention of 2.5x the forward's FLOPs (five
    # products of the forward's size: S, dP, dV, dK, dQ)
    flops = w.flops() * (2.5 if a.which == "bwd" else 1.0)
    ms_per_step = wall * 1e3 / a.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kmean * 1e-3) / 1e12
    # the elementwise-mask workload reads a mask as large as the score
    # matrix: its kernel is bound by HBM, so its roofline is bytes / time
    hbm_bound = a.workload == "masked" and a.which == "fwd"
    if hbm_bound:
        alg_bytes = sum(algorithmic_bytes(w))
        roof = {"bound": "hbm", "achieved": round(alg_bytes / (kmean * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(alg_bytes / (kmean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "algorithmic_bytes": alg_bytes}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4)}
    roof["traffic"] = (stored_traffic(a.workload + ("_dropout" if a.dropout > 0 else ""))
                       if a.which == "fwd" else None)
    # the nominal roofline is the matrix cores'; the issue counters (when
    # taken on these kernel sources) say which unit actually binds
    sq = stored_counters(a.workload) if a.which == "fwd" and a.dropout == 0 else None
    if sq:
        for key in ("mfma_busy_share", "valu_issue_share", "coexec_share", "idle_share",
                    "binding"):
            roof[key] = sq[key]
    rec = {
        "metric": METRIC if a.which == "fwd" else METRIC_BWD,
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": (round(value / PAGES_FLASH_TFLOPS, 2)
                        if a.workload == "noncausal" and a.which == "fwd" else None),
        "dtype": w.dtype, "data": "synthetic", "config": describe(w, a.workload, a.dropout),
        "pct_of_mfma_peak": round(100.0 * value / PEAK_TFLOPS, 2),
        "kernel_ms": {"mean": round(kmean, 4), "median_single": round(float(np.median(kern_ms)), 4),
                      "min_single": round(float(np.min(kern_ms)), 4),
                      "stdev_single": round(float(np.std(kern_ms)), 4)},
        **({"kernel_ms_cold": {"mean": round(float(np.mean(kern_cold)), 4),
                               "median": round(float(np.median(kern_cold)), 4),
                               "min": round(float(np.min(kern_cold)), 4),
                               "stdev": round(float(np.std(kern_cold)), 4),
                               "reps": len(kern_cold),
                               "note": "512 MiB write before each launch"}}
           if kern_cold else {}),
        "roofline": roof,
    }
    if a.which == "bwd":
        rec["kernels"] = "rowdot + dq + dkdv (kernel_ms spans all three)"
    if a.targets and a.which == "fwd" and a.workload == "noncausal" and a.dropout == 0:
        # the two d = 64 causal workloads the 50%-of-peak target names, timed
        # after the headline's timed region (never inside it)
        del q, k, v, out, lse
        rec["targets"] = {
            "causal": time_target(torch, sdpa, inputs, np, "causal", max(a.steps, 20), 5, 50),
            "long": time_target(torch, sdpa, inputs, np, "long", max(3, min(a.steps, 10)), 2, 10)}
    if a.cpu_budget > 0:
        rec["cpu_baseline"] = (cpu_baseline(w, a.cpu_budget, a.dropout) if a.which == "fwd"
                               else cpu_baseline_bwd(w, a.cpu_budget, WORKLOADS[a.workload],
                                                     a.dropout))
    if rec.get("cpu_baseline"):
        rec["cpu_baseline"]["cpu_model"] = _cpu_model()
    print(json.dumps(rec), flush=True)
    return 0


def time_target(torch, sdpa, inputs, np, name, steps, warmup, reps):
    """Warm kernel time of one more workload, measured like the headline:
    ``steps`` back-to-back sdpa_fwd launches between two HIP events on the
    launch stream, after ``warmup`` launches; then ``reps`` single launches
    for the median, minimum and spread.  bf16 inputs take an f32 output, as
    in the headline run's rule."""
    w = inputs.make_config(WORKLOADS[name])

    def up(x):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    q, k, v = up(w.q), up(w.k), up(w.v)
    out_f32 = w.dtype == "bf16"
    out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device="cuda")
    lse = torch.empty(tuple(q.shape[:3]), dtype=torch.float32, device="cuda")
    dt = {"f16": sdpa.SDPA_F16, "bf16": sdpa.SDPA_BF16}[w.dtype]
    stream = torch.cuda.current_stream()
    L = sdpa._lib.lib()
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), w.B, w.H,
            w.Nq, w.Nk, w.d, float(w.scale), int(w.is_causal), None, dt,
            sdpa.SDPA_F32 if out_f32 else sdpa.SDPA_SAME, stream.cuda_stream]

    def step():
        st = L.sdpa_fwd(*args)
        if st != 0:
            raise sdpa.SdpaError(st)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # single launches, each between its own pair of events: the spread
    single = []
    for _ in range(reps):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        step()
        a1.record(stream)
        torch.cuda.synchronize()
        single.append(a0.elapsed_time(a1))
    tf = w.flops() / (ms * 1e-3) / 1e12
    return {"workload": describe(w, name)["workload"], "kernel_ms": round(ms, 4),
            "tflops": round(tf, 2), "frac_of_mfma_peak": round(tf / PEAK_TFLOPS, 4),
            "steps": steps,
            "single_ms": {"median": round(float(np.median(single)), 4),
                          "min": round(float(np.min(single)), 4),
                          "stdev": round(float(np.std(single)), 4), "reps": reps}}


def _cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())

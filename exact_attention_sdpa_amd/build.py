"""Build libsdpa.so (gfx950 HIP kernels + C-ABI) in-tree with hipcc.

    python -m exact_attention_sdpa_amd.build [-j N] [--verbose]

Objects go to ``_build/`` next to the package; the library lands in the
package directory, where ``exact_attention_sdpa_amd._lib`` loads it.

A second library, ``libsdpa_debug.so`` (objects in ``_build/debug/``), is
the same sources built with -DSDPA_LDS_POISON=1: the forward kernels fill
their LDS with NaN before writing it, so that a read of LDS ahead of its
data shows up as NaN in the output (tests/test_lds_poison_gpu.py).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsdpa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# Packed-FP32 VALU instructions are disabled for every HIP translation unit.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
          "-Wno-unused-command-line-argument"]


LIB_DEBUG = os.path.join(PKG, "libsdpa_debug.so")
DEBUG_FLAGS = ["-DSDPA_LDS_POISON=1"]


def _compile(src: str, verbose: bool, outdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + list(extra) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC, "-Wall",
               "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 8, verbose: bool = False, debug: bool = True) -> str:
    """Build libsdpa.so and (``debug``) libsdpa_debug.so; returns the first."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    dbg_dir = os.path.join(BUILD, "debug")
    os.makedirs(dbg_dir, exist_ok=True)
    jobs_list = [(s, BUILD, ()) for s in srcs]
    if debug:
        jobs_list += [(s, dbg_dir, DEBUG_FLAGS) for s in srcs if s.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1], j[2]), jobs_list))
    n = len(srcs)
    _link(objs[:n], LIB)
    if debug:
        # the host-only sources are shared; the kernels are the debug ones
        host = [o for s, o in zip(srcs, objs[:n]) if s.endswith(".cpp")]
        _link(objs[n:] + host, LIB_DEBUG)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--no-debug", dest="debug", action="store_false",
                    help="skip the LDS-poisoning debug library")
    a = ap.parse_args(argv)
    print(build(a.j, a.verbose, a.debug))
    return 0


if __name__ == "__main__":
    sys.exit(main())

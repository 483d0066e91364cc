"""The C ABI's host-side argument checks (csrc/sdpa_validate.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer: a fuzz driver
(tests/sanitize/validate_fuzz.cpp) is built with g++ together with the
checks and run over seeded random arguments that mix ordinary sizes with
edge values (0, negative, around the int32 and int64 limits), non-finite
scales and rates, and null, misaligned and overlapping fake pointers.  The
checks never dereference device pointers, so no GPU is needed; any signed
overflow, out-of-range shift or out-of-bounds access aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_sdpa_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_validation_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "validate_fuzz")
    flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + flags +
           ["-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
            "-I", CSRC, os.path.join(ROOT, "tests", "sanitize", "validate_fuzz.cpp"),
            os.path.join(CSRC, "sdpa_validate.cpp"), "-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # verify_asan_link_order=0: the environment's own preloaded libraries
    # (if any) may come before the ASan runtime; they are left as they are
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "100000"], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " 0 unexpected outcomes" in out
    import re
    m = re.search(r"accepted (\d+) forward and (\d+) backward calls", out)
    assert m and int(m.group(1)) > 1000 and int(m.group(2)) > 1000, out[-500:]

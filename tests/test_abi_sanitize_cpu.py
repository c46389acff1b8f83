"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library sources (device code for gfx950 as usual, host code with
the two sanitizers) together with tests/sanitize/abi_checks.cpp, a driver
that calls every entry point with null, misaligned, overlapping and extreme
arguments, and runs it. Needs hipcc, no GPU: the driver runs nothing when a
device is present, and this test is skipped there.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp8_linear_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.skipif(_gpu_present(), reason="host-only check: the driver passes made-up pointers")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + san
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [DRIVER]
    objs = [str(tmp_path / (os.path.basename(p) + ".o")) for p in srcs]

    def compile_one(pair):
        src, obj = pair
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        r = subprocess.run(common + lang + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"{os.path.basename(src)}:\n{r.stderr[-3000:]}"

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    exe = str(tmp_path / "abi_checks")
    r = subprocess.run([hipcc, "--offload-arch=gfx950"] + san + objs + ["-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # leaks inside the HIP runtime are not this library's; every other report is fatal
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "OK: 0 failures" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]

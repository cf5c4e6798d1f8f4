"""Host-side sanitizers over the C ABI's validation code (CPU, no GPU).

The library's host code (argument checking, workspace sizing, the
thread-local error string) is built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (device code is unchanged)
and driven by tests/sanitizer/abi_driver.cpp, which calls every entry point
with arguments that validation must reject, from one thread and then from
four at once.  Nothing reaches a device.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_quantization_awq_amd", "csrc")
BUILD = os.path.join(ROOT, "weight_only_quantization_awq_amd", "_build")
KERNELS = ["k_stats", "k_search", "k_pack", "k_decode", "k_prefill", "k_clip"]
HIPCC = "/opt/rocm/bin/hipcc"
BASE = ["--offload-arch=gfx950", "-O1", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
        "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _kernel_object(name: str, tmp: str) -> str:
    """The build's object if it is newer than its source, else a fresh one."""
    src = os.path.join(CSRC, name + ".hip")
    obj = os.path.join(BUILD, name + ".o")
    if os.path.exists(obj) and os.path.getmtime(obj) >= os.path.getmtime(src):
        return obj
    out = os.path.join(tmp, name + ".o")
    subprocess.run([HIPCC, *BASE, "-O3", "-c", src, "-o", out], check=True, capture_output=True)
    return out


@pytest.mark.timeout(600)
def test_abi_validation_under_host_sanitizers(tmp_path):
    if not os.path.exists(HIPCC) or shutil.which("c++filt") is None:
        pytest.skip("ROCm toolchain not present")
    tmp = str(tmp_path)
    api = os.path.join(tmp, "awq_api_san.o")
    r = subprocess.run([HIPCC, *BASE, *SAN, "-c", os.path.join(CSRC, "awq_api.hip"), "-o", api],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    objs = [_kernel_object(k, tmp) for k in KERNELS]
    drv = os.path.join(tmp, "abi_driver.o")
    r = subprocess.run([HIPCC, *BASE, *SAN, "-c", os.path.join(ROOT, "tests", "sanitizer", "abi_driver.cpp"), "-o",
                        drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = os.path.join(tmp, "abi_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, drv, api, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ)
    # the HIP runtime's own allocations outlive main(); leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "sanitized ABI checks passed" in r.stdout

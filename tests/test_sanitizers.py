"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the prefix-cache block pool driven by random requests, and the C
ABI's argument checks and workspace layout with the kernel launchers
replaced by checking stubs (tests/sanitize/*.cpp).  Only host code is built
with the sanitizers (hipcc compiles api.hip for the host alone)."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "paged_kv_cache_23_amd", "csrc")
DRV = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(not shutil.which("g++"), reason="g++ not installed")
def test_block_pool_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pool_driver")
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", INC, os.path.join(CSRC, "prefix_cache.cpp"),
          os.path.join(DRV, "pool_driver.cpp"), "-o", exe])
    res = _run([exe], env=ENV, timeout=300)
    assert "pool driver: ok" in res.stdout and "Sanitizer" not in res.stderr


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC)), reason="ROCm clang / hipcc not installed")
def test_c_abi_checks_under_sanitizers(tmp_path):
    host = [f"-Xarch_host {f}".split() for f in SAN]
    api_o, drv_o, pc_o, exe = (str(tmp_path / n) for n in ("api.o", "drv.o", "pc.o", "abi_driver"))
    _run([HIPCC, "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1", "-g", *[a for f in host for a in f],
          "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    _run([HIPCC, "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1", "-g", *[a for f in host for a in f],
          "-I", INC, "-I", CSRC, "-c", os.path.join(DRV, "abi_driver.cpp"), "-o", drv_o])
    _run([CLANG, "-std=c++17", "-O1", "-g", *SAN, "-I", INC, "-c", os.path.join(CSRC, "prefix_cache.cpp"),
          "-o", pc_o])
    _run([CLANG, *SAN, api_o, drv_o, pc_o, "-o", exe])
    res = _run([exe], env=ENV, timeout=300)
    assert "abi driver: ok" in res.stdout and "Sanitizer" not in res.stderr

"""Compile the HIP sources into ``libpkv.so`` (in-tree) with hipcc for gfx950.

Run ``python -m paged_kv_cache_23_amd.build`` or call ``build()``.  The
library is written next to this file; the Python binding loads it from
there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libpkv.so")
SOURCES = ["api.hip", "append.hip", "copy.hip", "decode.hip", "prefill.hip", "shared.hip", "prefix_cache.cpp"]
# the read-stream ceiling probe that bench.py --tile-probe times (not part of the attention library)
PROBE_PATH = os.path.join(HERE, "libpkv_probe.so")
PROBE_SOURCES = ["probe.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep hipcc from forming packed-fp32 instructions (v_pk_fma_f32 & co.)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    # a local that shadows another is an error: one such name once sent a
    # ring read to the wrong LDS offset
    "-Werror=shadow",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")
    return exe


def _compile(sources, out: str, verbose: bool, extra_flags) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source (the library and the read-stream probe); return the library path."""
    _compile(PROBE_SOURCES, PROBE_PATH, verbose, extra_flags)
    return _compile(SOURCES, LIB_PATH, verbose, extra_flags)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libkda.so (gfx950) in place: the kernel layer (csrc/kda_decode.hip)
with hipcc, the host layer (csrc/kda_host.cpp: C ABI, validation, launch
plan) with the host C++ compiler, linked into one shared library.

    python -m linear_attention_recurrent_decode_amd.build [--kernarg-preload N]

--kernarg-preload sets how many leading kernel arguments arrive in SGPRs at
wave launch (default 8; 0 turns preloading off, which is slower but is what
a kernel-tracing profiler's dispatch path sees: see the notes on tracing).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRC = os.path.join(CSRC, "kda_decode.hip")
HOST_SRC = os.path.join(CSRC, "kda_host.cpp")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
# the benchmark's tile-stream reference (include/kda_stream.h), a library of its own
STREAM_SRC = os.path.join(CSRC, "kda_stream.hip")
STREAM_LIB = os.path.join(PKG, "libkda_stream.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # every fused multiply-add in the kernels is an explicit fmaf: no implicit
    # contraction, so inlined copies of the same code round the same way
    "-ffp-contract=off",
    # the decode kernel's eight leading scalar arguments arrive in SGPRs at
    # wave launch (gfx950 kernel-argument preloading)
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
    # no packed-fp32 instructions: scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# the host layer: plain C++17
HOST_CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def host_cxx() -> str:
    path = shutil.which("g++") or shutil.which("c++")
    if not path:
        raise RuntimeError("no host C++ compiler")
    return path


def _run(cmd, what):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"{what} failed:\n" + "\n".join(msgs))
    return msgs


KERNARG_PRELOAD = 8


def build(verbose: bool = False, kernarg_preload: int = KERNARG_PRELOAD) -> str:
    """Compile libkda.so next to this file (always recompiles)."""
    if not 0 <= kernarg_preload <= 16:
        raise ValueError("kernarg_preload must be in 0..16")
    flags = [f"-amdgpu-kernarg-preload-count={kernarg_preload}" if f.startswith("-amdgpu-kernarg-preload-count=")
             else f for f in HIPCC_FLAGS]
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmp:
        host_o = os.path.join(tmp, "kda_host.o")
        dev_o = os.path.join(tmp, "kda_decode.o")
        msgs = _run([host_cxx(), *HOST_CXX_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", HOST_SRC, "-o", host_o],
                    "host layer")
        msgs += _run([hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, "-c", SRC, "-o", dev_o], "kernel layer")
        tmp_lib = LIB + ".tmp"
        msgs += _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, dev_o, host_o], "link")
        tmp_stream = STREAM_LIB + ".tmp"
        msgs += _run([hipcc(), *flags, "-shared", "-fPIC", "-I", INCLUDE, "-o", tmp_stream, STREAM_SRC],
                     "stream reference")
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp_lib, LIB)
    os.replace(tmp_stream, STREAM_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description="build libkda.so (gfx950) in place")
    ap.add_argument("--kernarg-preload", type=int, default=KERNARG_PRELOAD,
                    help="leading kernel arguments preloaded into SGPRs (0: off)")
    print(build(verbose=True, kernarg_preload=ap.parse_args().kernarg_preload))

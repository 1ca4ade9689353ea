"""The sanitizer tier (CPU): the CPU oracle's pins and planted-mutant checks,
and the host-side C ABI tests, each in a child process that preloads the
AddressSanitizer and UndefinedBehaviorSanitizer runtimes, against builds
made with both sanitizers, every finding fatal:

  * the oracle (oracle/kda_oracle.c) built with -fsanitize=address,undefined
    (oracle.SANITIZE: KDA_ORACLE_SANITIZE=1), under test_oracle_pins.py and
    test_oracle_mutants.py (the mutants are built with the same flags);
  * the library's host layer (csrc/kda_host.cpp: argument validation, the
    launch plan, the C ABI entry points) built host-only with the same
    sanitizers next to a stand-in for the kernel layer
    (tests/sanitize/kernel_layer_stub.cpp: no device), under
    test_abi_cpu.py and test_binding_cpu.py (conftest.py loads that build
    when KDA_TEST_HOST_LIBRARY names it).

The GPU kernels are not part of this tier: the GPU tests guard every buffer
the kernels write with guard regions instead (kda_harness.Guarded)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_recurrent_decode_amd")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"no {name} in this toolchain")
    return path


def _env(**extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    # torch and numpy are not built with the sanitizers: their leaks and the
    # ODR of their own libraries are not what this tier checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:detect_odr_violation=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra)
    return env


def _pytest(args, env):
    # -s: a sanitizer report goes straight to the child's stderr (a finding
    # ends the child before pytest could print what it captured)
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu", *args]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_pins_and_mutants_under_sanitizers():
    out = _pytest(["tests/test_oracle_pins.py", "tests/test_oracle_mutants.py"], _env(KDA_ORACLE_SANITIZE="1"))
    assert " passed" in out


def test_host_layer_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libkda_host_san.so")
    subprocess.run(["g++", "-std=c++17", "-g", "-O1", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    os.path.join(PKG, "csrc", "kda_host.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "kernel_layer_stub.cpp"), "-o", lib], check=True)
    out = _pytest(["tests/test_abi_cpu.py", "tests/test_binding_cpu.py"], _env(KDA_TEST_HOST_LIBRARY=lib))
    assert " passed" in out

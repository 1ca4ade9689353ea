"""The C ABI from a plain C program (tests/c_abi/kda_c_smoke.c): compiled
with gcc against include/kda.h, libkda.so and the oracle library.  The CPU
test only compiles and links it; the GPU test runs it."""
import os
import subprocess

import pytest

import linear_attention_recurrent_decode_amd as kda
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "kda_c_smoke.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(tmp_path):
    oracle._load()                                     # builds liboracle.so if needed
    if not os.path.exists(kda.library_path):
        pytest.skip("libkda.so is not built")
    exe = str(tmp_path / "kda_c_smoke")
    pkg, odir = os.path.dirname(kda.library_path), os.path.dirname(oracle.LIB)
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", exe,
           f"-L{pkg}", "-l:libkda.so", f"-L{odir}", "-l:liboracle.so", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{pkg}:{odir}:{ROCM}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert "warning" not in res.stderr, res.stderr
    return exe


def test_c_program_compiles_against_the_header(tmp_path):
    _compile(tmp_path)


@pytest.mark.gpu
def test_c_program_decodes_like_the_oracle(tmp_path):
    exe = _compile(tmp_path)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("c abi ok")

"""bench.py's host logic (no GPU): algorithmic bytes, the cold slot sets,
the kernel-code fingerprint of the recorded counters, and the one-GPU exit."""
import os
import subprocess
import sys

import numpy as np

import bench
import kda_inputs as ki

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_headline():
    p = ki.workload("n32_t1_h8")
    nb = bench.algorithmic_bytes(p)
    state = 2 * 32 * 8 * 128 * 128 * 4                      # read + write of 256 fp32 tiles
    per_token = 2 * 8 * 128 * 2 + 8 * 128 * 2 + 8 * 128 * 4 + 8 * 4 + 8 * 128 * 2   # q,k; v; g; beta; out
    assert nb["state"] == state == 33_554_432
    assert nb["total"] == state + 32 * per_token + 32 * 4 == 33_948_800
    assert nb["units"] == 256
    assert bench.algorithmic_bytes(p, 2)["state"] == state // 2


def test_algorithmic_bytes_fused_gate_and_packed():
    p = ki.workload("n32_t1_h8_rawgate")
    per_token = 2 * 8 * 128 * 2 + 8 * 128 * 2 + 8 * 128 * 2 + 8 * 2 + 8 * 128 * 2   # raw gate and beta in bf16
    assert bench.algorithmic_bytes(p)["total"] == 33_554_432 + 32 * per_token + 32 * 4 + 8 * 4 + 8 * 128 * 4
    q = ki.workload("packed_n256_h12")
    nb = bench.algorithmic_bytes(q)
    live = q.live_requests()
    assert len(live) == 230 and nb["units"] == 230 * 12
    assert nb["state"] == 2 * 230 * 12 * 128 * 128 * 4


def test_slot_sets_are_disjoint_and_keep_padding():
    p = ki.workload("packed_n256_h12")
    sets = bench.slot_sets(p, ki)
    live = p.live_requests()
    pad = np.setdiff1d(np.arange(p.N), live)
    assert np.array_equal(sets[0], p.slot_idx)
    seen = set()
    for s in sets:
        assert np.all(s[pad] == -1)
        vals = s[live]
        assert len(set(vals.tolist())) == len(live)            # distinct within a call
        assert np.all((vals >= 0) & (vals < p.num_slots))
        assert not (seen & set(vals.tolist()))                 # disjoint across calls
        seen |= set(vals.tolist())
    assert len(sets) == p.num_slots // len(live)


def test_kernel_code_fingerprint_ignores_comments(tmp_path):
    src = open(bench.KERNEL_SRC).read()
    commented = tmp_path / "a.hip"
    commented.write_text("// a new comment\n" + src.replace("\n", "\n  ", 3) + "\n/* trailing */\n")
    assert bench.kernel_code_sha256(str(commented)) == bench.kernel_code_sha256()
    changed = tmp_path / "b.hip"
    changed.write_text(src.replace("constexpr int STAGE_TOKENS = 4;", "constexpr int STAGE_TOKENS = 5;"))
    assert bench.kernel_code_sha256(str(changed)) != bench.kernel_code_sha256()


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr

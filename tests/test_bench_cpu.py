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
    kern, host = bench.CODE_SOURCES
    src = open(kern).read()
    commented = tmp_path / "a.hip"
    commented.write_text("// a new comment\n" + src.replace("\n", "\n  ", 3) + "\n/* trailing */\n")
    assert bench.kernel_code_sha256((str(commented), host)) == bench.kernel_code_sha256()
    changed = tmp_path / "b.hip"
    changed.write_text(src.replace("constexpr int STAGE_TOKENS = 4;", "constexpr int STAGE_TOKENS = 5;"))
    assert bench.kernel_code_sha256((str(changed), host)) != bench.kernel_code_sha256()
    # a change of the launch plan voids the counters too
    plan = tmp_path / "h.cpp"
    plan.write_text(open(host).read().replace("c.units <= 1024 ? 4 : 8", "c.units <= 512 ? 4 : 8"))
    assert bench.kernel_code_sha256((kern, str(plan))) != bench.kernel_code_sha256()


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_block_order_interleaves_two_arms():
    assert bench.block_order(3, False) == ["A"] * 3
    order = bench.block_order(4, True)
    assert order == ["A", "B", "B", "A", "A", "B", "B", "A"]
    assert order.count("A") == order.count("B") == 4


def test_spread_of_blocks():
    sp = bench.spread([5.0, 1.0, 3.0, 2.0, 4.0])
    assert sp["median"] == 3.0 and sp["p10"] == 1.4 and abs(sp["p90"] - 4.6) < 1e-12


def test_request_chunks_cover_the_call():
    for n, parts in ((32, 8), (256, 8), (3, 8), (1, 1), (10, 3)):
        ch = bench.request_chunks(n, parts)
        assert ch[0][0] == 0 and ch[-1][1] == n
        assert all(a < b for a, b in ch)
        assert all(ch[i][1] == ch[i + 1][0] for i in range(len(ch) - 1))
        assert len(ch) == min(n, parts)


def test_threaded_oracle_equals_one_thread():
    """The all-core CPU baseline splits a call's requests over threads; the
    split changes nothing in the result (each range owns its slots and rows)."""
    import oracle
    p = ki.make_problem("split", 5, N=10, H=2, HV=2, K=8, V=8, num_slots=14, T=None, n_pad=3)
    live = p.live_requests()
    pool0 = p.state_slots(p.slot_idx[live]).astype(np.float64)
    remap = np.full(p.N, -1, dtype=np.int32)
    remap[live] = np.arange(len(live), dtype=np.int32)
    one = pool0.copy()
    ref = oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, one, remap, p.cu_seqlens, p.scale)
    split = pool0.copy()
    out = np.full_like(ref, np.nan)
    cu = p.cu_seqlens.astype(np.int32)
    for a, b in bench.request_chunks(p.N, 4):
        oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, split, np.ascontiguousarray(remap[a:b]),
                             np.ascontiguousarray(cu[a:b + 1]), p.scale, out=out)
    assert np.array_equal(split, one)
    assert np.array_equal(np.isnan(out), np.isnan(ref)) and np.array_equal(out[~np.isnan(ref)], ref[~np.isnan(ref)])


def test_default_block_count():
    """About 2000 timed calls by default, an odd count from 5 to 101."""
    assert bench.default_blocks(2000) == 5
    assert bench.default_blocks(400) == 5
    assert bench.default_blocks(20) == 101
    assert bench.default_blocks(100) == 21
    assert bench.default_blocks(1) == 101
    assert all(bench.default_blocks(k) % 2 == 1 for k in range(1, 3000, 7))

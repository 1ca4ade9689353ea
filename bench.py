#!/usr/bin/env python3
"""Recurrent KDA decode benchmark on one MI355X.

A step is one decode call: every live request of the workload advanced by its
tokens (fused decay, delta correction, rank-1 update, readout, optional gated
RMSNorm, in-place state write-back).  The default workload is the dominant
serving shape: 32 requests, one token each, 8 value heads, K = V = 128, fp32
state in a 512-slot pool (vLLM PR 57585, "Retained baseline trace
attribution": N = 32 is nearly every launch at 8 local heads).

Cold caches.  The pool (256 MiB at this shape) would sit in MI355X's 256 MiB
memory-side cache and 8 x 4 MiB L2 if every call used the same 32 slots, so
consecutive calls walk disjoint slot sets of the pool and rotate over several
copies of the pool: a call's state was last touched at least 1 GiB of state
traffic earlier.  Every call is still exactly the workload: N requests on N
distinct slots of a pool of num_slots slots.

Protocol (after vLLM PR 57585, "Microbenchmark and earlier serving limits":
cold caches, untimed warmup, interleaved blocks; and FlashInfer PR 4562,
description: a duration-calibrated graph warmup):
  1. --warmup eager calls, then graph replays of one full slot rotation until
     at least --warmup-ms of wall time have passed (untimed);
  2. --blocks timed blocks (by default enough for about 2000 timed calls:
     5 blocks of 2000, 101 of 20) of exactly --steps calls each.  A block's calls
     are enqueued on one stream right behind an untimed HIP graph replay of
     the calls before them in the rotation (at least a full rotation and
     2 ms of GPU time, and long enough that the host has enqueued the whole
     block while the GPU still runs the replay), so the GPU runs the block's calls back to back
     with cold caches; the block's time is the interval between HIP events
     recorded on that stream around its calls.  ``value`` is the median
     block's us per call, with the p10 and p90 of the blocks beside it.
     (Timing one graph replay of the block instead adds the fixed cost of
     starting a replay, about 12 us on this ROCm, to the block: reported
     beside, as graph_replay_us_per_call.)
Then, as extra keys: a plain device copy of the call's state bytes (read and
write, the same rotation and protocol), the tile-stream reference (the same
calls' live tiles moved in place by a kernel that computes nothing,
libkda_stream.so), the host cost of one enqueue through
the C ABI, the cache-resident time (--warm), and the CPU oracle on all host
cores and on one.  With --flags-b the blocks alternate A B B A ... between the
library's choice (A) and a call with extra flag bits (B), and the line
carries both medians (--flags-b 0x2: validated calls, KDA_FLAG_VALIDATE, against
trusted ones).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA decode µs/call + state HBM GB/s (% of peak), N32/T1/H8/K=V=128"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
COLD_BYTES = 1 << 30            # state traffic between two uses of the same slots
HOST_ENQUEUE_US_BOUND = 8.0     # above the host's time per enqueue (about 4 us from Python)
GAP_MIN_US = 2000.0             # the untimed replay before a block keeps the GPU busy at least this long
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "linear_attention_recurrent_decode_amd", "csrc")
# the kernels, and the host layer whose launch plan picks one for a workload
CODE_SOURCES = (os.path.join(CSRC, "kda_decode.hip"), os.path.join(CSRC, "kda_host.cpp"))
# kda_decode_plan(..., layout=True) values
LAYOUT_NAMES = {0: "32-column waves", 1: "16-column waves", 2: "16-column waves, split key rows"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def default_blocks(steps: int) -> int:
    """Timed blocks when --blocks is not given: enough for about 2000 timed
    calls (a median over more blocks when each block is short), odd, 5 to 101."""
    n = max(5, min(101, -(-2000 // max(1, steps))))
    return n if n % 2 else n + 1


def algorithmic_bytes(p, state_elem: int = 4) -> dict:
    """Bytes the call must move at least: each live (request, value head)
    reads and writes its K x V fp32 state once; each live token reads q, k
    (per q/k head), v, g, beta (per value head) and writes out (plus the gate
    with the norm); slot indices, cu_seqlens and the norm weight once.  With
    the fused gate activation each token reads the bf16 raw gate and raw beta
    instead of g and beta, and A_log and dt_bias are read once."""
    live = p.live_requests()
    lens = np.diff(p.cu_seqlens.astype(np.int64))
    live_tokens = int(lens[live].sum())
    state = 2 * len(live) * p.HV * p.K * p.V * state_elem
    gate_elem = 2 if p.raw else 4
    per_token = 2 * p.H * p.K * 2 + p.HV * p.V * 2 + p.HV * p.K * gate_elem + p.HV * gate_elem + p.HV * p.V * 2
    if p.gate is not None:
        per_token += p.HV * p.V * 2
    io = live_tokens * per_token + p.N * 4
    if p.T is None:
        io += (p.N + 1) * 4
    if p.gate is not None:
        io += p.V * 2
    if p.raw:
        io += p.HV * 4 + p.HV * p.K * 4
    return {"state": state, "io": io, "total": state + io, "units": len(live) * p.HV}


def slot_sets(p, ki):
    """Disjoint sets of live slots covering the pool; set 0 is the workload's own."""
    live = p.live_requests()
    own = p.slot_idx[live].astype(np.int64)
    taken = set(own.tolist())
    rest = [int(s) for s in ki.permutation(p.seed, 99, p.num_slots) if int(s) not in taken]
    order = np.concatenate([own, np.array(rest, dtype=np.int64)])
    n_sets = max(1, p.num_slots // max(1, len(live)))
    sets = []
    for j in range(n_sets):
        s = p.slot_idx.astype(np.int32).copy()
        s[live] = order[j * len(live):(j + 1) * len(live)]
        sets.append(s)
    return sets


def block_order(n_blocks: int, two_arms: bool) -> list:
    """Arm of each timed block: all 'A', or A B B A A B B A ... (each arm
    n_blocks times), so that a drift over the run weighs on both arms alike."""
    if not two_arms:
        return ["A"] * n_blocks
    order = []
    for i in range(n_blocks):
        order += ["A", "B"] if i % 2 == 0 else ["B", "A"]
    return order


def spread(values) -> dict:
    """Median, p10 and p90 of a list of per-block figures."""
    v = np.asarray(values, dtype=np.float64)
    return {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)), "p90": float(np.percentile(v, 90))}


def kernel_code_sha256(paths=CODE_SOURCES) -> str:
    """SHA-256 of the code of the kernels and of the launch plan: comments
    and whitespace removed, so that editing a comment does not void the
    recorded counters (the sources hold no string literal with a comment
    marker)."""
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"\s+", "", text)
        h.update(text.encode())
    return h.hexdigest()


def traffic_for(workload: str):
    """HBM bytes per call from the committed counter runs, or None if the
    kernel code changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[workload]
        if rec.get("code_sha256") != kernel_code_sha256():
            return None
        return rec["bytes_per_call"]
    except (OSError, KeyError, ValueError):
        return None


def shape_problem(ki, spec: str):
    """A problem of the shape ``spec`` ("N=24,T=4,H=8"; T=0 packed) drawn from
    the serving workloads' distributions."""
    kv = dict(item.split("=") for item in spec.split(",") if item)
    N, T, H = int(kv.get("N", 32)), int(kv.get("T", 1)), int(kv.get("H", 8))
    HV = int(kv.get("HV", H))
    slots = int(kv.get("slots", max(512, 2 * N)))
    name = "shape_" + "_".join(f"{k}{v}" for k, v in kv.items())
    return ki.make_problem(name, ki.SEED_BASE + 100 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=slots,
                           T=T or None, raw_gates=kv.get("raw") == "1", norm=kv.get("norm") == "1")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def request_chunks(n: int, parts: int) -> list:
    """Contiguous ranges of a call's requests, one per worker (empty ones dropped)."""
    parts = max(1, min(parts, n))
    bounds = np.linspace(0, n, parts + 1).round().astype(int)
    return [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]


def cpu_baseline(p, pool_live: np.ndarray, budget_s: float, threads: int) -> dict:
    """The CPU oracle on full calls of the same workload and inputs, on a
    compact pool that holds the live requests' slots.  With threads > 1 the
    call's requests are split into contiguous ranges that threads run at
    once (the oracle's C code releases the interpreter lock; each range owns
    its requests' state slots and output rows)."""
    import oracle
    live = p.live_requests()
    remap = np.full(p.N, -1, dtype=np.int32)
    remap[live] = np.arange(len(live), dtype=np.int32)
    cu = p.cu_seqlens.astype(np.int32)
    kw = {}
    if p.gate is not None:
        kw = dict(gate=p.gate, norm_weight=p.norm_weight, eps=p.eps)
    if p.raw:
        kw.update(raw_gate=p.raw_gate, raw_beta=p.raw_beta, A_log=p.A_log, dt_bias=p.dt_bias)
    pool = pool_live.astype(np.float64)
    out = np.zeros((p.tokens, p.HV, p.V), dtype=np.float64)
    jobs = [(np.ascontiguousarray(remap[a:b]), np.ascontiguousarray(cu[a:b + 1]))
            for a, b in request_chunks(p.N, threads)]

    def run(job):
        slots, cu_r = job
        oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, pool, slots, cu_r, p.scale, out=out, **kw)

    ex = concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) if len(jobs) > 1 else None

    def one_call():
        if ex is None:
            run(jobs[0])
        else:
            list(ex.map(run, jobs))

    try:
        one_call()   # warm-up
        n, t0 = 0, time.perf_counter()
        while True:
            one_call()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    finally:
        if ex is not None:
            ex.shutdown()
    us = el / n * 1e6
    how = (f"the call's requests split into {len(jobs)} contiguous ranges run by {len(jobs)} threads at once"
           if len(jobs) > 1 else "one host thread")
    return {"value": round(us, 3), "unit": "us/call", "cores": len(jobs), "kind": "oracle",
            "sample": f"{n} full calls of the {p.name} workload ({p.N} requests x {p.HV} value heads, "
                      f"{p.tokens} tokens), same inputs as the GPU run, double-precision sequential oracle, "
                      f"{how}, {el:.1f} s",
            "cpu_model": cpu_model(), "host_cores_available": len(os.sched_getaffinity(0))}


class Timer:
    """Timing of blocks of calls on one stream (protocol in the module
    docstring): each timed block is enqueued behind an untimed graph replay
    of the rotation, so that the GPU is still busy with the replay while the
    host enqueues the block, and runs the block's calls back to back."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream

    def capture(self, body):
        torch = self.torch
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            with torch.cuda.graph(graph, stream=self.stream):
                body()
        torch.cuda.synchronize()
        return graph

    def time_block(self, gap_graph, enqueue, calls: int) -> float:
        """us per call of ``calls`` calls that ``enqueue()`` issues on the
        stream right after an untimed replay of ``gap_graph``."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            gap_graph.replay()
            e0.record(self.stream)
            enqueue()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / calls

    def time_replay(self, gap_graph, graph, calls: int) -> float:
        """us per call of one replay of ``graph`` (after an untimed replay of
        it and of ``gap_graph``), events around the replay."""
        torch = self.torch
        graph.replay()
        return self.time_block(gap_graph, graph.replay, calls)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="calls per timed block")
    ap.add_argument("--warmup", type=int, default=200, help="untimed eager calls before the calibrated warmup")
    ap.add_argument("--warmup-ms", type=float, default=100.0, help="minimum wall time of graph-replayed warmup")
    ap.add_argument("--blocks", type=int, default=None,
                    help="timed blocks (at least 3; default: enough blocks for about 2000 timed calls, 5 to 101)")
    ap.add_argument("--workload", default="n32_t1_h8")
    ap.add_argument("--shape", default=None,
                    help="a workload of another shape with the same value distributions instead of --workload: "
                         "comma-separated N=, T= (0: packed, 1..4 tokens per request), H=, HV=, slots=, "
                         "raw=1 (fused gate), norm=1")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="seconds of oracle work per cpu_baseline run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the copy reference and the enqueue cost")
    ap.add_argument("--warm", action="store_true", help="also time cache-resident calls (same slots every call)")
    ap.add_argument("--state", choices=("fp32", "bf16"), default="fp32", help="state pool element type")
    ap.add_argument("--flags-b", type=lambda s: int(s, 0), default=None,
                    help="extra call flag bits of a second arm, timed in A B B A order against the default")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run 5 plain device copies of this many MiB (untimed), "
                         "a known-size reference for hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: recurrent KDA decode has no cross-GPU step here; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.blocks is None and args.steps >= 1:
        args.blocks = default_blocks(args.steps)
    if args.blocks < 3 or args.steps < 1:
        print("bench.py needs --blocks >= 3 and --steps >= 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_inputs as ki
    import linear_attention_recurrent_decode_amd as kda

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = kda.library()

    p = ki.workload(args.workload) if args.shape is None else shape_problem(ki, args.shape)
    bf16_state = args.state == "bf16"
    state_dtype = torch.bfloat16 if bf16_state else torch.float32
    state_elem = 2 if bf16_state else 4
    nbytes = algorithmic_bytes(p, state_elem)
    sets = slot_sets(p, ki)
    per_call_read = nbytes["state"] // 2
    R = max(1, math.ceil(COLD_BYTES / max(1, len(sets) * per_call_read)))
    pool_bytes = p.num_slots * p.slot_elems * state_elem
    if R * pool_bytes > (96 << 30):
        R = max(1, (96 << 30) // pool_bytes)
    log(f"[bench] workload {p.name}: N={p.N} T={p.T} H={p.H} HV={p.HV} tokens={p.tokens} "
        f"slot_sets={len(sets)} pool_copies={R} pool={pool_bytes / 2**20:.0f} MiB")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = bf(p.q), bf(p.k), bf(p.v)
    g = beta = None
    raw = {}
    if p.raw:
        raw = dict(raw_gate=bf(p.raw_gate), raw_beta=bf(p.raw_beta), A_log=torch.from_numpy(p.A_log).to(dev),
                   dt_bias=torch.from_numpy(p.dt_bias).to(dev))
    else:
        g = torch.from_numpy(p.g).to(dev)
        beta = torch.from_numpy(p.beta).to(dev)
    gate = bf(p.gate) if p.gate is not None else None
    w = bf(p.norm_weight) if p.norm_weight is not None else None
    cu = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(dev)
    out = torch.zeros((p.tokens, p.HV, p.V), dtype=torch.bfloat16, device=dev)

    pools = [torch.empty((p.num_slots, p.HV, p.K, p.V), dtype=state_dtype, device=dev) for _ in range(R)]
    chunk = max(1, (64 << 20) // (p.slot_elems * 4))
    for s0 in range(0, p.num_slots, chunk):
        sl = np.arange(s0, min(p.num_slots, s0 + chunk))
        vals = p.state_slots(sl)
        if bf16_state:
            vals = ki.bf16_bits_to_f32(ki.f32_to_bf16_bits(vals))
        pools[0][s0:s0 + len(sl)] = torch.from_numpy(vals).to(dev).to(state_dtype)
    for r in range(1, R):
        pools[r].copy_(pools[0])
    pool_live = pools[0][torch.from_numpy(p.slot_idx[p.live_requests()].astype(np.int64)).to(dev)].float().cpu().numpy()
    set_t = [torch.from_numpy(s).to(dev) for s in sets]

    # a verdict word for calls with KDA_FLAG_VALIDATE (--flags-b 0x2: the
    # metadata check's cost); calls without the flag ignore it
    verdict = torch.zeros(1, dtype=torch.int32, device=dev)
    combos = []
    for r in range(R):
        for s in set_t:
            combos.append(kda.decode_args(q, k, v, g, beta, pools[r], s, out, p.scale, gate, w, p.eps,
                                          device_status=verdict, **raw))
    T = p.T if p.T is not None else 0
    packed = p.T is None
    base_flags = kda.KDA_FLAG_STATE_BF16 if bf16_state else 0
    cu_ptr = cu.data_ptr()

    def launch(i, stream_handle, extra_flags=0, which=None):
        a = (which or combos)[i % len(which or combos)]
        if packed:
            st = lib.kda_decode_packed(ctypes.byref(a), cu_ptr, p.tokens, base_flags | extra_flags, stream_handle)
        else:
            st = lib.kda_decode_step(ctypes.byref(a), T, base_flags | extra_flags, stream_handle)
        if st != 0:
            raise kda.KdaError(st, "decode")

    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    timer = Timer(torch, stream)

    # 1. warmup: eager calls, then replays of one full rotation for >= warmup_ms
    pos = 0
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            launch(pos + i, sh)
    pos += args.warmup
    torch.cuda.synchronize()
    start = pos
    g_warm = timer.capture(lambda: [launch(start + i, sh) for i in range(len(combos))])
    warm_calls, t0 = 0, time.perf_counter()
    while True:
        g_warm.replay()
        torch.cuda.synchronize()
        warm_calls += len(combos)
        warm_ms = (time.perf_counter() - t0) * 1000.0
        if warm_ms >= args.warmup_ms and warm_calls >= 20:
            break
    del g_warm
    log(f"[bench] calibrated warmup: {warm_calls} calls in {warm_ms:.1f} ms")

    # 2. timed blocks: `steps` calls each, enqueued behind an untimed replay of
    # the `gap` calls before them in the rotation (at least one full rotation,
    # so the block's slots are cold, and long enough that the host has
    # enqueued the whole block before the GPU finishes the replay)
    est_us = max(0.25, warm_ms * 1000.0 / warm_calls)
    gap = max(len(combos), math.ceil(args.steps * HOST_ENQUEUE_US_BOUND / est_us),
              math.ceil(GAP_MIN_US / est_us))
    arms = {"A": 0}
    if args.flags_b is not None:
        arms["B"] = int(args.flags_b)
    per_arm = {a: [] for a in arms}

    def block(extra_flags, which=None):
        nonlocal pos
        first = pos
        gap_graph = timer.capture(lambda: [launch(first + i, sh, which=which) for i in range(gap)])
        t0_call = first + gap
        pos = t0_call + args.steps
        us = timer.time_block(gap_graph, lambda: [launch(t0_call + i, sh, extra_flags, which)
                                                  for i in range(args.steps)], args.steps)
        del gap_graph
        return us

    for arm in block_order(args.blocks, len(arms) > 1):
        per_arm[arm].append(block(arms[arm]))
    blocks_a = per_arm["A"]
    sp = spread(blocks_a)
    us_per_call = sp["median"]
    log(f"[bench] {len(blocks_a)} blocks of {args.steps} calls (gap {gap}): median {us_per_call:.3f} us/call "
        f"(p10 {sp['p10']:.3f}, p90 {sp['p90']:.3f}); blocks {[round(x, 3) for x in blocks_a]}")

    extras = {}
    if args.warm:
        hot = [combos[0]]
        extras["cache_resident_us_per_call"] = round(block(0, which=hot), 4)
        log(f"[bench] cache-resident: {extras['cache_resident_us_per_call']:.3f} us/call")

    if not args.no_extras:
        # the same blocks as one graph replay each (events around the replay)
        replay = []
        for _ in range(3):
            first = pos
            gap_graph = timer.capture(lambda: [launch(first + i, sh) for i in range(gap)])
            t0_call = first + gap
            graph = timer.capture(lambda: [launch(t0_call + i, sh) for i in range(args.steps)])
            pos = t0_call + args.steps
            replay.append(timer.time_replay(gap_graph, graph, args.steps))
            del gap_graph, graph
        extras["graph_replay_us_per_call"] = {
            "median": round(float(np.median(replay)), 4), "blocks": [round(x, 4) for x in replay],
            "what": "the same blocks of calls captured as one HIP graph each, events around one replay "
                    "(after an untimed one): adds the fixed cost of starting a replay to the block"}
        log(f"[bench] graph replay: {extras['graph_replay_us_per_call']['median']:.3f} us/call")

        # a plain device copy of the call's state bytes (half read, half written), cold by rotation
        half = max(4, per_call_read // 4) * 4
        n_chunks = max(2, math.ceil(COLD_BYTES / half))
        src = torch.ones(n_chunks * half // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ch = half // 4

        def copies(first, n):
            for i in range(first, first + n):
                j = i % n_chunks
                dst[j * ch:(j + 1) * ch].copy_(src[j * ch:(j + 1) * ch])

        copy_gap = max(n_chunks, math.ceil(args.steps * 4 * HOST_ENQUEUE_US_BOUND / est_us))
        copy_blocks = []
        cpos = 0
        for _ in range(3):
            c0 = cpos
            gap_graph = timer.capture(lambda: copies(c0, copy_gap))
            cpos += copy_gap + args.steps
            with torch.cuda.stream(stream):
                copy_blocks.append(timer.time_block(gap_graph, lambda: copies(c0 + copy_gap, args.steps), args.steps))
            del gap_graph
        copy_us = float(np.median(copy_blocks))
        extras["copy_reference"] = {
            "us_per_call": round(copy_us, 4), "GBps": round(2 * half / (copy_us * 1e-6) / 1e9, 1),
            "bytes_per_call": 2 * half,
            "what": "torch device copy of the call's state bytes (read + write), one copy per call, the same "
                    "cold rotation and timing protocol: the achievable streaming rate at this size with the "
                    "same per-launch cost"}
        del src, dst
        log(f"[bench] copy reference: {copy_us:.3f} us/call, {extras['copy_reference']['GBps']} GB/s")

        # the tile-stream reference: each call's live tiles moved in place by
        # a kernel that computes nothing (libkda_stream.so), the same calls of
        # the same rotation, timed with the same protocol
        try:
            slib = kda.stream_library()
        except RuntimeError as e:   # an extra: the decode's line does not depend on it
            slib = None
            log(f"[bench] no stream reference: {e}")

        def stream_launch(i):
            a = combos[i % len(combos)]
            st = slib.kda_stream_tiles(a.state, state_elem, a.num_slots, a.slot_stride, a.slot_idx, a.N, a.HV, sh)
            if st != 0:
                raise kda.KdaError(st, "stream reference")

        stream_blocks = []
        for _ in range(5 if slib is not None else 0):
            first = pos
            gap_graph = timer.capture(lambda: [stream_launch(first + i) for i in range(gap)])
            t0_call = first + gap
            pos = t0_call + args.steps
            stream_blocks.append(timer.time_block(gap_graph, lambda: [stream_launch(t0_call + i)
                                                                      for i in range(args.steps)], args.steps))
            del gap_graph
        if stream_blocks:
            stream_us = float(np.median(stream_blocks))
            extras["stream_reference"] = {
                "us_per_call": round(stream_us, 4),
                "state_GBps": round(nbytes["state"] / (stream_us * 1e-6) / 1e9, 1),
                "decode_over_stream": round(us_per_call / stream_us, 4),
                "blocks": [round(x, 4) for x in stream_blocks],
                "what": "the call's live state tiles read and written back in place by a kernel that computes "
                        "nothing (one 512-lane workgroup per tile, all loads before the stores), the same calls "
                        "of the same cold rotation and timing protocol: the time of the call's state traffic "
                        "alone at its launch shape, in one access pattern (the decode's own lane layouts can "
                        "move the tiles faster)"}
            log(f"[bench] stream reference: {stream_us:.3f} us/call, {extras['stream_reference']['state_GBps']} GB/s")

        # host cost of one enqueue through the C ABI (validation + launch), from Python via ctypes
        batch, batches = 1000, 10
        per_batch = []
        with torch.cuda.stream(stream):
            for b in range(batches):
                torch.cuda.synchronize()
                t0 = time.perf_counter_ns()
                for i in range(batch):
                    launch(i, sh)
                per_batch.append((time.perf_counter_ns() - t0) / batch)
        torch.cuda.synchronize()
        extras["host_enqueue_ns"] = {
            "median": round(float(np.median(per_batch)), 1), "calls": batch * batches,
            "what": "host time per kda_decode_step / kda_decode_packed call (argument validation and kernel "
                    "launch), called from Python through ctypes, batches of 1000 enqueues with the GPU drained "
                    "between batches"}
        log(f"[bench] host enqueue: {extras['host_enqueue_ns']['median']:.0f} ns per call")

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 18            # floats
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    achieved = nbytes["total"] / (us_per_call * 1e-6) / 1e9
    state_gbps = nbytes["state"] / (us_per_call * 1e-6) / 1e9
    traffic = traffic_for(p.name) if not bf16_state else traffic_for(p.name + "_bf16state")
    result = {
        "metric": METRIC,
        "value": round(us_per_call, 4),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": p.name, "N": p.N, "T": p.T if p.T is not None else "1..4 packed",
                   "H": p.H, "HV": p.HV, "K": p.K, "V": p.V, "num_slots": p.num_slots,
                   "norm": p.gate is not None, "state_dtype": args.state,
                   "gate_input": "raw, activated in the kernel" if p.raw else "activated",
                   "cold_slot_sets": len(sets), "cold_pool_copies": R,
                   "vtile": kda.kda_decode_plan(p.N * p.HV, T or 1, p.gate is not None, bf16_state, packed,
                                                raw_gate=p.raw),
                   "lane_layout": LAYOUT_NAMES[kda.kda_decode_plan(p.N * p.HV, T or 1, p.gate is not None,
                                                                   bf16_state, packed, layout=True,
                                                                   raw_gate=p.raw)]},
        "blocks": len(blocks_a),
        "block_us_per_call": [round(x, 4) for x in blocks_a],
        "median": round(sp["median"], 4), "p10": round(sp["p10"], 4), "p90": round(sp["p90"], 4),
        "warmup_calibrated": {"calls": warm_calls, "ms": round(warm_ms, 1)},
        "state_GBps": round(state_gbps, 1),
        "state_frac_of_peak": round(state_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_call": nbytes["total"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
    }
    if "B" in per_arm:
        sb = spread(per_arm["B"])
        result["ab"] = {"flags_b": arms["B"], "order": "ABBA", "a_blocks": [round(x, 4) for x in blocks_a],
                        "b_blocks": [round(x, 4) for x in per_arm["B"]], "a_median": round(sp["median"], 4),
                        "b_median": round(sb["median"], 4),
                        "b_vs_a_pct": round(100.0 * (sb["median"] / sp["median"] - 1.0), 2)}
    result.update(extras)
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        log(f"[bench] timing the CPU oracle on {threads} threads ...")
        result["cpu_baseline"] = cpu_baseline(p, pool_live, args.cpu_budget, threads)
        if threads > 1:
            log("[bench] timing the CPU oracle on one thread ...")
            result["cpu_baseline_one_thread"] = cpu_baseline(p, pool_live, args.cpu_budget / 2, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

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

Timing.  The K timed calls are captured once into a HIP graph (no host
launch overhead) and replayed between two HIP events recorded on the replay
stream; the per-call time is the event interval over K.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "linear_attention_recurrent_decode_amd", "csrc", "kda_decode.hip")
# kda_decode_plan(..., layout=True) values
LAYOUT_NAMES = {0: "32-column waves", 1: "16-column waves", 2: "16-column waves, split key rows"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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


def kernel_code_sha256(path: str = KERNEL_SRC) -> str:
    """SHA-256 of the kernel source's code: comments and whitespace removed,
    so that editing a comment does not void the recorded counters (the
    source has no string literal that holds a comment marker)."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()


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


def cpu_baseline(p, pool_live: np.ndarray, budget_s: float) -> dict:
    """The CPU oracle, single-threaded, on full calls of the same workload."""
    import oracle
    live = p.live_requests()
    remap = np.full(p.N, -1, dtype=np.int32)
    remap[live] = np.arange(len(live), dtype=np.int32)
    kw = {}
    if p.gate is not None:
        kw = dict(gate=p.gate, norm_weight=p.norm_weight, eps=p.eps)
    if p.raw:
        kw.update(raw_gate=p.raw_gate, raw_beta=p.raw_beta, A_log=p.A_log, dt_bias=p.dt_bias)
    pool = pool_live.astype(np.float64)
    oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, pool, remap, p.cu_seqlens, p.scale, **kw)  # warm-up
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, pool, remap, p.cu_seqlens, p.scale, **kw)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    us = el / n * 1e6
    return {"value": round(us, 3), "unit": "us/call", "cores": 1, "kind": "oracle",
            "sample": f"{n} full calls of the {p.name} workload ({p.N} requests x {p.HV} value heads, "
                      f"{p.tokens} tokens), same inputs as the GPU run, double-precision sequential oracle "
                      f"on one host thread, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="n32_t1_h8")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="also time cache-resident calls (same slots every call)")
    ap.add_argument("--state", choices=("fp32", "bf16"), default="fp32", help="state pool element type")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run 5 plain device copies of this many MiB (untimed), "
                         "a known-size reference for hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: recurrent KDA decode has no cross-GPU step here; "
              "run it with --gpus 1", file=sys.stderr)
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

    p = ki.workload(args.workload)
    bf16_state = args.state == "bf16"
    state_dtype = torch.bfloat16 if bf16_state else torch.float32
    nbytes = algorithmic_bytes(p, 2 if bf16_state else 4)
    sets = slot_sets(p, ki)
    per_call_read = nbytes["state"] // 2
    R = max(1, math.ceil(COLD_BYTES / max(1, len(sets) * per_call_read)))
    pool_bytes = p.num_slots * p.slot_elems * (2 if bf16_state else 4)
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

    combos = []
    for r in range(R):
        for s in set_t:
            a = kda.decode_args(q, k, v, g, beta, pools[r], s, out, p.scale, gate, w, p.eps, **raw)
            combos.append(a)
    T = p.T if p.T is not None else 0
    packed = p.T is None
    call_flags = kda.KDA_FLAG_STATE_BF16 if bf16_state else 0
    cu_ptr = cu.data_ptr()

    def launch(i, stream_handle):
        a = combos[i % len(combos)]
        if packed:
            st = lib.kda_decode_packed(ctypes.byref(a), cu_ptr, p.tokens, call_flags, stream_handle)
        else:
            st = lib.kda_decode_step(ctypes.byref(a), T, call_flags, stream_handle)
        if st != 0:
            raise kda.KdaError(st, "decode")

    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    def capture(n, offset=0):
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for i in range(n):
                    launch(offset + i, sh)
        torch.cuda.synchronize()
        return graph

    # warm-up: eager calls, then the warm-up graph
    with torch.cuda.stream(stream):
        for i in range(min(args.warmup, 20)):
            launch(i, sh)
    torch.cuda.synchronize()
    g_warm = capture(max(1, args.warmup))
    g_warm.replay()
    torch.cuda.synchronize()
    g_timed = capture(args.steps, offset=args.warmup)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        g_timed.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    us_per_call = ms * 1000.0 / args.steps
    log(f"[bench] timed {args.steps} calls: {ms:.3f} ms, {us_per_call:.3f} us/call")

    warm = None
    if args.warm:
        hot = [combos[0]] * len(combos)
        saved, combos[:] = list(combos), hot
        g_hot = capture(args.steps)
        combos[:] = saved
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g_hot.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        warm = e0.elapsed_time(e1) * 1000.0 / args.steps
        log(f"[bench] cache-resident: {warm:.3f} us/call")

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
    traffic = traffic_for(p.name)
    result = {
        "metric": METRIC,
        "value": round(us_per_call, 4),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 6),
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
        "state_GBps": round(state_gbps, 1),
        "state_frac_of_peak": round(state_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_call": nbytes["total"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
    }
    if warm is not None:
        result["cache_resident_us_per_call"] = round(warm, 4)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(p, pool_live, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
serving workloads at full size and on small cases that span several tiles
with ragged tails, plus the bit-exact properties of the path."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import linear_attention_recurrent_decode_amd as kda
import oracle
from kda_harness import (DEV, assert_guards, bf16_tensor, bf16_to_f64, compare, f32_tensor, guarded_full, parity,
                         run_gpu, run_oracle, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def guards_intact():
    """After every test: no buffer any call of the test wrote through (pool,
    outputs, per-token states) was written past either end."""
    import kda_harness
    kda_harness.CREATED.clear()
    yield
    kda_harness.check_all_guards()


def _log(name, rep):
    print(f"[parity] {name}: {rep}", flush=True)


# ------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("name", list(ki.WORKLOADS))
def test_workload_full_size(name):
    print(f"[parity] start {name}", flush=True)
    p = ki.workload(name)
    _log(name, parity(p))


@pytest.mark.parametrize("width", [32, 64, 128])
def test_dominant_shape_every_tile_width(width):
    p = ki.workload("n32_t1_h8")
    _log(f"n32_t1_h8 vtile={width}", parity(p, flags=kda.KDA_FLAG_VTILE(width)))


def test_packed_workload_as_step_when_uniform():
    p = ki.workload("n16_t4_h8")
    _log("n16_t4_h8 packed", parity(p, packed=True))


# ------------------------------------------------------- small / ragged cases
SMALL = [
    # (N, H, HV, T, num_slots, n_pad, norm)
    (1, 1, 1, 1, 1, 0, False),
    (3, 2, 6, 1, 9, 0, False),      # HV = 3H: three value heads per q/k head
    (5, 3, 3, 3, 11, 1, False),
    (7, 2, 4, None, 19, 2, False),  # packed, ragged lengths, padding rows
    (9, 4, 4, 2, 12, 0, True),
    (6, 1, 2, None, 8, 1, True),
]


@pytest.mark.parametrize("case", SMALL)
def test_small_cases(case):
    N, H, HV, T, slots, n_pad, norm = case
    p = ki.make_problem("small", 77 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=slots, T=T,
                        n_pad=n_pad, norm=norm)
    _log(f"small {case}", parity(p))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("t_max", [6, 9])
def test_packed_long_requests(t_max, dtype):
    """Requests longer than one staging chunk of tokens (up to 9 tokens):
    restaged with an fp32 pool, loaded token by token with a bf16 pool."""
    p = ki.make_problem("long", 40 + t_max, N=24, H=4, HV=8, K=128, V=128, num_slots=40, T=None,
                        t_max=t_max, n_pad=3)
    assert np.diff(p.cu_seqlens).max() > 4
    _log(f"packed t_max={t_max} {dtype}", parity(p, state_dtype=dtype))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_packed_long_requests_fused_gate(dtype):
    p = ki.make_problem("longraw", 49, N=24, H=4, HV=8, K=128, V=128, num_slots=40, T=None, t_max=9, n_pad=3,
                        raw_gates=True)
    assert np.diff(p.cu_seqlens).max() > 4
    _log(f"packed raw t_max=9 {dtype}", parity(p, state_dtype=dtype))


def test_packed_long_requests_match_step_bitwise():
    """A uniform packed call with 6 tokens per request (past one staging
    chunk) gives the step call's bits, fp32 and bf16 pool."""
    p = ki.make_problem("long6", 50, N=12, H=2, HV=4, K=128, V=128, num_slots=20, T=6)
    for dtype in (torch.float32, torch.bfloat16):
        a = upload(p, state_dtype=dtype)
        run_gpu(a, packed=False)
        b = upload(p, state_dtype=dtype)
        run_gpu(b, packed=True)
        torch.cuda.synchronize()
        assert torch.equal(a.state.view(torch.int16) if dtype == torch.bfloat16 else a.state,
                           b.state.view(torch.int16) if dtype == torch.bfloat16 else b.state), dtype
        assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16)), dtype


def test_step_six_tokens():
    p = ki.make_problem("t6", 46, N=10, H=2, HV=4, K=128, V=128, num_slots=16, T=6)
    _log("step T=6", parity(p))


@pytest.mark.parametrize("N", [64, 128])
def test_loop_body_shapes(N):
    """One token per request from 512 tiles up with an fp32 pool: the
    library's choice (eight 16-column waves per workgroup), the prefetching
    loop body of the 32-column kernel (a forced 64- or 128-column tile) and
    the packed call over the same tokens give the same bits; and parity
    with the oracle."""
    p = ki.make_problem("loop", 60 + N, N=N, H=8, HV=8, K=128, V=128, num_slots=2 * N + 8, T=1)
    assert kda.kda_decode_plan(N * 8, 1, False) == 128
    assert kda.kda_decode_plan(N * 8, 1, packed=True) == 64     # packed: four 16-column waves to 1024 tiles
    _log(f"one token, {N * 8} tiles", parity(p))
    width = 64 if N * 8 < 1024 else 128
    runs = []
    for packed, flags in ((False, 0), (False, kda.KDA_FLAG_VTILE(width)), (True, 0), (True, kda.KDA_FLAG_VTILE(128))):
        d = _fresh(p)
        run_gpu(d, packed=packed, flags=flags)
        torch.cuda.synchronize()
        runs.append((d.state.clone(), d.out.view(torch.int16).clone()))
    for st, o in runs[1:]:
        assert torch.equal(st, runs[0][0]) and torch.equal(o, runs[0][1])


def test_packed_and_step_bodies_bit_identical():
    """A uniform packed call and the step call over the same tokens give the
    same bits (different kernel bodies, same arithmetic)."""
    for name in ("n32_t4_h8", "n8_t4_h8"):
        p = ki.workload(name)
        a = _fresh(p)
        run_gpu(a, packed=False)
        b = _fresh(p)
        run_gpu(b, packed=True)
        torch.cuda.synchronize()
        assert torch.equal(a.state, b.state), name
        assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16)), name


# ------------------------------------------------------- bf16 state pool
@pytest.mark.parametrize("name", ["n1_t1_h8", "n32_t1_h8", "n1_t4_h8", "n8_t4_h8", "n32_t4_h8", "n32_t1_h16_norm",
                                  "packed_n256_h12", "packed_n256_h12_rawgate"])
def test_bf16_state_workloads(name):
    p = ki.workload(name)
    _log(f"{name} bf16 state", parity(p, state_dtype=torch.bfloat16))


@pytest.mark.parametrize("case", SMALL[1:4])
def test_bf16_state_small_cases(case):
    N, H, HV, T, slots, n_pad, norm = case
    p = ki.make_problem("small", 177 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=slots, T=T,
                        n_pad=n_pad, norm=norm)
    parity(p, state_dtype=torch.bfloat16)


def test_bf16_state_tile_widths_bit_identical():
    """The library's choice (16-column waves with a bf16 pool at this shape)
    and every forced width of the 32-column kernel give the same bits."""
    p = ki.workload("n32_t1_h8")
    results = []
    for width in (0, 32, 64, 128):
        d = upload(p, state_dtype=torch.bfloat16)
        run_gpu(d, flags=kda.KDA_FLAG_VTILE(width) if width else 0)
        torch.cuda.synchronize()
        results.append((d.out.view(torch.int16).clone(), d.state.view(torch.int16).clone()))
    for o, s_ in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(s_, results[0][1])


# ------------------------------------------------------- per-token states (speculative decoding)
INTER_CASES = [
    ("n8_t4_h8", torch.float32),
    ("n32_t4_h8", torch.bfloat16),
    ("packed_small", torch.float32),
    ("packed_small", torch.bfloat16),
    ("n32_t1_h16_norm", torch.float32),
]


@pytest.mark.parametrize("name,dtype", INTER_CASES)
def test_intermediate_states(name, dtype):
    if name == "packed_small":
        p = ki.make_problem("ps", 61, N=40, H=4, HV=4, K=128, V=128, num_slots=64, T=None, t_max=6, n_pad=5)
    else:
        p = ki.workload(name)
    d = upload(p, state_dtype=dtype)
    sentinel = 1232.0                         # exact in fp32 and bf16
    inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), sentinel, dtype)
    run_gpu(d, inter_state=inter)
    torch.cuda.synchronize()
    assert_guards(d)
    ref_inter = np.full((p.tokens, p.HV, p.K, p.V), np.nan)
    ref_out, ref_state = run_oracle(p, state_bf16=dtype == torch.bfloat16, inter_state=ref_inter)
    compare(d, ref_out, ref_state)
    got = inter.float().cpu().numpy().astype(np.float64)
    live_rows = np.isfinite(ref_inter[:, 0, 0, 0])
    assert np.all(got[~live_rows] == sentinel)                    # skipped requests: not written
    err = np.abs(got[live_rows] - ref_inter[live_rows])
    r = np.abs(ref_inter[live_rows])
    if dtype == torch.bfloat16:
        assert np.all(err <= 2.0 ** -8 * r + 1e-6)
    else:
        assert np.all(err <= 1e-4 * r + 1e-6)
        assert err.max() <= 2e-6 * r.max()
    # the last token's state is the final pool state, bit for bit
    for n in p.live_requests():
        last = int(p.cu_seqlens[n + 1]) - 1
        if last >= int(p.cu_seqlens[n]):
            assert torch.equal(inter[last], d.state[int(p.slot_idx[n])])
    _log(f"inter {name} {dtype}: max|d| {err.max():.3e}", "")


# ------------------------------------------------------- fused gate activation
RAW_SMALL = SMALL + [(16, 8, 8, 1, 40, 0, False)]   # 128 tiles, one token: the peeled body


@pytest.mark.parametrize("case", RAW_SMALL)
def test_fused_gate_small_cases(case):
    N, H, HV, T, slots, n_pad, norm = case
    p = ki.make_problem("raw", 91 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=slots, T=T, n_pad=n_pad,
                        norm=norm, raw_gates=True)
    _log(f"raw gate {case}", parity(p))


@pytest.mark.parametrize("name,dtype", [("n32_t1_h8_rawgate", torch.bfloat16), ("n8_t4_h8", torch.float32),
                                        ("n32_t1_h16_norm", torch.float32), ("n32_t1_h16_norm", torch.bfloat16)])
def test_fused_gate_workload_variants(name, dtype):
    if name.endswith("_rawgate"):
        p = ki.workload(name)
    else:
        spec = dict(ki.WORKLOADS[name])
        spec.pop("cid")
        p = ki.make_problem(name, 123, K=128, V=128, raw_gates=True, **spec)
    _log(f"{name} raw gate {dtype}", parity(p, state_dtype=dtype))


def _run_fresh(p, **kw):
    d = _fresh(p)
    run_gpu(d, **kw)
    torch.cuda.synchronize()
    return d.out.view(torch.int16).clone(), d.state.clone()


def test_fused_gate_bodies_bit_identical():
    """The per-lane activation (loop and peeled bodies) and the cooperative
    one (staged body, packed calls) round identically."""
    for name, kw in (("loop", dict(N=32, HV=8, H=8, T=1, num_slots=64)),      # 256 tiles, T = 1
                     ("peeled", dict(N=16, HV=8, H=8, T=1, num_slots=64)),    # 128 tiles
                     ("peeled T=3", dict(N=9, HV=4, H=2, T=3, num_slots=16))):
        p = ki.make_problem("raw", 5, K=128, V=128, raw_gates=True, **kw)
        o1, s1 = _run_fresh(p, packed=False)
        o2, s2 = _run_fresh(p, packed=True)
        assert torch.equal(o1, o2) and torch.equal(s1, s2), name
    p = ki.make_problem("raw", 6, N=32, H=8, HV=8, K=128, V=128, num_slots=64, T=1, raw_gates=True)
    ref = _run_fresh(p)
    for width in (32, 64, 128):
        o, st = _run_fresh(p, flags=kda.KDA_FLAG_VTILE(width))
        assert torch.equal(o, ref[0]) and torch.equal(st, ref[1]), width


@pytest.mark.parametrize("N,T,packed", [(32, 1, False), (16, 1, False), (9, 3, False), (9, 3, True)])
def test_fused_gate_exact_values_equal_activated_call(N, T, packed):
    """Raw values whose activation is exact in fp32 (raw gate +inf or -inf:
    g = -inf or 0; raw beta 0, +inf, -inf: beta = 1/2, 1, 0) decode bit for
    bit like the activated call, in every body."""
    p = ki.make_problem("exact", 17, N=N, H=4, HV=8, K=128, V=128, num_slots=2 * N, T=T, raw_gates=True)
    pick = ki.draws(17, 50, np.arange(p.tokens * p.HV * p.K, dtype=np.uint64)).reshape(p.tokens, p.HV, p.K)
    clear = (pick % np.uint64(4)) == 0
    p.raw_gate[...] = np.where(clear, ki.to_bf16_bits(np.inf), ki.to_bf16_bits(-np.inf))
    choice = (ki.draws(17, 51, np.arange(p.tokens * p.HV, dtype=np.uint64)) % np.uint64(3)).astype(np.int64)
    choice = choice.reshape(p.tokens, p.HV)
    p.raw_beta[...] = ki.to_bf16_bits(np.choose(choice, [0.0, np.inf, -np.inf]))
    raw_out, raw_state = _run_fresh(p, packed=packed)
    act = ki.make_problem("exact", 17, N=N, H=4, HV=8, K=128, V=128, num_slots=2 * N, T=T)
    act.g[...] = np.where(clear, -np.inf, 0.0).astype(np.float32)
    act.beta[...] = np.choose(choice, [0.5, 1.0, 0.0]).astype(np.float32)
    act_out, act_state = _run_fresh(act, packed=packed)
    assert torch.equal(raw_out, act_out) and torch.equal(raw_state, act_state)
    # and both agree with the oracle
    d = _fresh(p)
    run_gpu(d, packed=packed)
    torch.cuda.synchronize()
    compare(d, *run_oracle(p))


def test_fused_gate_intermediate_states():
    p = ki.make_problem("ps", 62, N=40, H=4, HV=4, K=128, V=128, num_slots=64, T=None, t_max=6, n_pad=5,
                        raw_gates=True)
    d = upload(p)
    inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), 1232.0, torch.float32)
    run_gpu(d, inter_state=inter)
    torch.cuda.synchronize()
    assert_guards(d)
    ref_inter = np.full((p.tokens, p.HV, p.K, p.V), np.nan)
    ref_out, ref_state = run_oracle(p, inter_state=ref_inter)
    compare(d, ref_out, ref_state)
    live_rows = np.isfinite(ref_inter[:, 0, 0, 0])
    got = inter.cpu().numpy().astype(np.float64)
    err = np.abs(got[live_rows] - ref_inter[live_rows])
    assert np.all(err <= 1e-4 * np.abs(ref_inter[live_rows]) + 1e-6)
    assert np.all(got[~live_rows] == 1232.0)


def test_fused_gate_strided_fused_projection():
    """raw_gate and raw_beta as row-strided column blocks of one bf16
    projection (with q, k, v), as a serving model's fused input projection
    would hand them over."""
    p = ki.make_problem("rawfused", 12, N=6, H=2, HV=4, K=128, V=128, num_slots=9, T=2, raw_gates=True)
    d = upload(p)
    T, HK, HVV, HVK = p.tokens, p.H * p.K, p.HV * p.V, p.HV * p.K
    o_gate = 2 * HK + HVV
    o_beta = o_gate + HVK + 8
    width = (o_beta + p.HV + 7) // 8 * 8 + 8            # a multiple of 8: 16-byte rows for q, k and raw_gate
    fused = torch.zeros((T, width), dtype=torch.bfloat16, device=DEV)
    fused[:, :HK] = d.q.reshape(T, HK)
    fused[:, HK:2 * HK] = d.k.reshape(T, HK)
    fused[:, 2 * HK:2 * HK + HVV] = d.v.reshape(T, HVV)
    fused[:, o_gate:o_gate + HVK] = d.raw_gate.reshape(T, HVK)
    fused[:, o_beta:o_beta + p.HV] = d.raw_beta
    d.q = fused[:, :HK].view(T, p.H, p.K)
    d.k = fused[:, HK:2 * HK].view(T, p.H, p.K)
    d.v = fused[:, 2 * HK:2 * HK + HVV].view(T, p.HV, p.V)
    d.raw_gate = fused[:, o_gate:o_gate + HVK].view(T, p.HV, p.K)
    d.raw_beta = fused[:, o_beta:o_beta + p.HV]
    assert d.raw_gate.stride(0) == width and d.raw_beta.stride(0) == width
    for packed in (False, True):
        d2 = upload(p)
        d2.q, d2.k, d2.v, d2.raw_gate, d2.raw_beta = d.q, d.k, d.v, d.raw_gate, d.raw_beta
        run_gpu(d2, packed=packed)
        torch.cuda.synchronize()
        compare(d2, *run_oracle(p))


def test_fused_gate_graph_validate_and_stream():
    """The fused gate inside a HIP graph (replayed with eager work between),
    with device-side validation, on a non-default stream: bit for bit the
    eager call on the default stream."""
    p = ki.make_problem("rawgraph", 13, N=24, H=4, HV=8, K=128, V=128, num_slots=40, T=None, n_pad=3,
                        raw_gates=True)
    eager = _fresh(p)
    run_gpu(eager)
    torch.cuda.synchronize()
    d = _fresh(p)
    init = d.state.clone()
    status = _status_word()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run_gpu(d, device_status=status, stream=s)
    torch.cuda.synchronize()
    live_rows = torch.from_numpy(np.isfinite(run_oracle(p)[0][:, 0, 0])).to(DEV)
    for _ in range(3):
        d.state.copy_(init)                  # eager work between replays
        d.out.view(torch.int16).fill_(0)
        status.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0       # KDA_DEVICE_OK
        assert torch.equal(d.state, eager.state)
        assert torch.equal(d.out.view(torch.int16)[live_rows], eager.out.view(torch.int16)[live_rows])


# ------------------------------------------------------- a large batch, sampled
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_large_batch_sampled(dtype):
    """2048 requests x 16 value heads (32768 tiles of 128 columns) in a
    2112-slot pool (2.1 GiB fp32): the oracle checks a seeded sample of 24
    requests (outputs and final states); the 64 slots no request owns stay
    bitwise untouched.  The pool is drawn on the device, the sampled slots
    are copied back for the oracle."""
    N, H, HV, slots = 2048, 16, 16, 2112
    p = ki.make_problem("large", 77, N=N, H=H, HV=HV, K=128, V=128, num_slots=slots, T=1)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4321)
    state = (torch.randn((slots, HV, 128, 128), generator=gen, device=DEV) * 0.05).to(dtype)
    before = state.clone()
    out = torch.empty((N, HV, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_decode_step(bf16_tensor(p.q), bf16_tensor(p.k), bf16_tensor(p.v), f32_tensor(p.g), f32_tensor(p.beta),
                        state, torch.from_numpy(p.slot_idx).to(DEV), out, T=1, scale=p.scale)
    torch.cuda.synchronize()
    sample = np.sort(ki.permutation(77, 5, N)[:24])
    sslots = p.slot_idx[sample].astype(np.int64)
    pool = before[torch.from_numpy(sslots).to(DEV)].float().cpu().numpy().astype(np.float64)
    ref_out = oracle.decode_step(p.q[sample], p.k[sample], p.v[sample], p.g[sample], p.beta[sample], pool,
                                 np.arange(len(sample), dtype=np.int32), 1, p.scale)
    got_out = bf16_to_f64(out[torch.from_numpy(sample).to(DEV)])
    err = np.abs(got_out - ref_out)
    assert np.all(err <= 2e-3 + 2.0 ** -8 * np.abs(ref_out)), err.max()
    got_state = state[torch.from_numpy(sslots).to(DEV)].float().cpu().numpy().astype(np.float64)
    serr = np.abs(got_state - pool)
    if dtype == torch.bfloat16:
        assert np.all(serr <= 2.0 ** -8 * np.abs(pool) + 1e-6), serr.max()
    else:
        assert np.all(serr <= 1e-4 * np.abs(pool) + 1e-6), serr.max()
    spare = np.setdiff1d(np.arange(slots), p.slot_idx)
    assert len(spare) == 64
    idx = torch.from_numpy(spare).to(DEV)
    assert torch.equal(state[idx], before[idx])
    _log(f"large batch {dtype}", f"out max|d| {err.max():.3e}, state max|d| {serr.max():.3e}")


# ------------------------------------------------------- seeded random configurations
def _random_case(i):
    """A seeded draw over the option space: request count, head counts and
    ratio, step or packed lengths, padding, norm, raw gates, pool dtype,
    per-token states, forced tile width."""
    d = ki.draws(0x5EED, 70 + i, np.arange(16, dtype=np.uint64))
    pick = lambda j, n: int(d[j] % np.uint64(n))
    H = 1 + pick(0, 4)
    HV = H * (1 + pick(1, 3))
    N = 1 + pick(2, 40)
    packed = pick(3, 2) == 1
    T = None if packed else 1 + pick(4, 5)
    n_pad = min(pick(5, 4), N - 1) if N > 1 else 0
    norm = pick(6, 3) == 0
    raw = pick(7, 2) == 1
    bf16 = pick(8, 2) == 1
    inter = pick(9, 3) == 0
    width = [0, 32, 64, 128][pick(10, 4)] if not norm else 0
    return dict(N=N, H=H, HV=HV, T=T, t_max=1 + pick(11, 6), n_pad=n_pad, norm=norm, raw=raw, bf16=bf16,
                inter=inter, width=width)


@pytest.mark.parametrize("i", range(16))
def test_random_configurations(i):
    c = _random_case(i)
    p = ki.make_problem("rand", 900 + i, N=c["N"], H=c["H"], HV=c["HV"], K=128, V=128, num_slots=c["N"] + 7,
                        T=c["T"], t_max=c["t_max"], n_pad=c["n_pad"], norm=c["norm"], raw_gates=c["raw"])
    dtype = torch.bfloat16 if c["bf16"] else torch.float32
    flags = kda.KDA_FLAG_VTILE(c["width"]) if c["width"] else 0
    print(f"[parity] random case {i}: {c}", flush=True)
    d = upload(p, state_dtype=dtype)
    before = d.state.clone()
    inter = None
    if c["inter"]:
        inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), 1232.0, dtype)
    run_gpu(d, flags=flags, inter_state=inter)
    torch.cuda.synchronize()
    assert_guards(d)
    ref_inter = np.full((p.tokens, p.HV, p.K, p.V), np.nan) if c["inter"] else None
    ref_out, ref_state = run_oracle(p, state_bf16=c["bf16"], inter_state=ref_inter)
    compare(d, ref_out, ref_state)
    untouched = torch.ones(p.num_slots, dtype=torch.bool, device=DEV)
    if len(d.live_slots):
        untouched[torch.from_numpy(d.live_slots).to(DEV)] = False
    assert torch.equal(d.state[untouched], before[untouched])
    if c["inter"]:
        got = inter.float().cpu().numpy().astype(np.float64)
        rows = np.isfinite(ref_inter[:, 0, 0, 0])
        tol = (2.0 ** -8 if c["bf16"] else 1e-4) * np.abs(ref_inter[rows]) + 1e-6
        assert np.all(np.abs(got[rows] - ref_inter[rows]) <= tol)
        assert np.all(got[~rows] == 1232.0)


def test_concurrent_streams_on_disjoint_slots():
    """Two halves of a batch on two streams at once give the bits of one
    call over the whole batch (every (request, head) is independent)."""
    p = ki.make_problem("streams", 31, N=40, H=4, HV=8, K=128, V=128, num_slots=64, T=2)
    whole = _fresh(p)
    run_gpu(whole)
    torch.cuda.synchronize()
    d = _fresh(p)
    half = p.N // 2
    rows = half * p.T
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for lo, s in ((0, s1), (half, s2)):
        r = slice(lo * p.T, lo * p.T + rows)
        kda.kda_decode_step(d.q[r], d.k[r], d.v[r], d.g[r], d.beta[r], d.state, d.slot_idx[lo:lo + half], d.out[r],
                            T=p.T, scale=p.scale, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(d.state, whole.state)
    assert torch.equal(d.out.view(torch.int16), whole.out.view(torch.int16))


# ------------------------------------------------------- transactional validation
def _status_word():
    return torch.full((1,), -7, dtype=torch.int32, device=DEV)


def test_validate_passes_valid_metadata_bit_identical():
    for name in ("n32_t1_h8", "n8_t4_h8", "n24_t4_h8", "n32_t4_h8", "packed_n256_h12", "n32_t1_h16_norm"):
        p = ki.workload(name)
        a = _fresh(p)
        run_gpu(a)
        b = _fresh(p)
        st = _status_word()
        run_gpu(b, device_status=st)
        torch.cuda.synchronize()
        assert st.item() == 0, name
        assert torch.equal(a.state, b.state) and torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))


def _corrupt(p, case):
    live = p.live_requests()
    if case == "duplicate":
        p.slot_idx[live[5]] = p.slot_idx[live[2]]
        return 2
    if case == "past_pool":
        p.slot_idx[live[1]] = p.num_slots
        return 1
    if case == "negative":
        p.slot_idx[live[1]] = -3
        return 1
    if case == "both":                          # lowest code wins
        p.slot_idx[live[5]] = p.slot_idx[live[2]]
        p.slot_idx[live[7]] = p.num_slots + 9
        return 1
    if case == "decreasing":
        p.cu_seqlens[4] = p.cu_seqlens[6]
        return 3
    raise ValueError(case)


@pytest.mark.parametrize("case", ["duplicate", "past_pool", "negative", "both", "decreasing"])
def test_validate_rejects_and_touches_nothing(case):
    p = ki.workload("packed_n256_h12")
    code = _corrupt(p, case)
    d = upload(p)
    before = d.state.clone()
    st = _status_word()
    run_gpu(d, device_status=st)
    torch.cuda.synchronize()
    assert st.item() == code
    assert torch.equal(d.state, before)
    assert torch.all(d.out.view(torch.int16) == np.int16(np.uint16(0xC640).view(np.int16)))


@pytest.mark.parametrize("case", ["duplicate", "past_pool"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name", ["n8_t4_h8", "n24_t4_h8", "n32_t4_h8"])
def test_validate_rejects_on_quarter_waves(case, dtype, name):
    """The 16-column waves honour the verdict too, nothing written: step
    calls of four tokens at 64 tiles (split-key waves with an fp32 pool,
    four waves per workgroup with bf16, both loading the tile first), 192
    tiles (split-key, fp32: the first token's inputs before the tile) and
    256 tiles (four waves, fp32: inputs first)."""
    p = ki.workload(name)
    code = _corrupt(p, case)
    d = upload(p, state_dtype=dtype)
    before = d.state.clone()
    st = _status_word()
    run_gpu(d, device_status=st)
    torch.cuda.synchronize()
    assert st.item() == code
    assert torch.equal(d.state, before)
    assert torch.all(d.out.view(torch.int16) == np.int16(np.uint16(0xC640).view(np.int16)))


SMALL_VALIDATED = [
    # (N, H, HV, T (None: packed), bf16 pool, fused gate): calls of at most
    # 64 requests, checked by the decode's own waves, on every kernel family
    (32, 8, 8, 1, False, False),     # 32-column waves
    (20, 4, 8, 1, False, True),      # 32-column waves, fused gate
    (64, 8, 8, 1, False, False),     # 512 tiles: eight 16-column waves
    (16, 2, 8, 2, False, False),     # split-key waves
    (64, 8, 8, 4, False, False),     # four 16-column waves, inputs first
    (32, 8, 8, 1, True, False),      # bf16 pool: four 16-column waves
    (9, 1, 2, 1, True, False),       # bf16 pool, one token, 18 tiles: split-key waves
    (9, 1, 3, 3, True, False),       # bf16 pool, three tokens, 27 tiles: split-key waves
    (40, 8, 8, None, False, False),  # packed: four 16-column waves
    (12, 2, 8, None, True, True),    # packed, bf16 pool, fused gate
    (65, 1, 2, None, False, False),  # one request more: the check kernel
]


@pytest.mark.parametrize("shape,case", [(shape, case) for shape in SMALL_VALIDATED
                                        for case in ("valid", "duplicate", "past_pool", "negative", "both", "decreasing")
                                        if case != "decreasing" or shape[3] is None])   # cu_seqlens: packed calls
def test_validate_small_calls(shape, case):
    """Validated calls of up to 64 requests are checked by the decode kernel's
    own waves: the same codes as the check kernel, nothing written on a
    rejection, the verdict word written either way, and valid metadata gives
    the unvalidated call's bits."""
    N, H, HV, T, bf16, raw = shape
    p = ki.make_problem("vsmall", 70 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=N + 9, T=T, n_pad=N // 6,
                        raw_gates=raw)
    dtype = torch.bfloat16 if bf16 else torch.float32
    code = 0 if case == "valid" else _corrupt(p, case)
    d = upload(p, state_dtype=dtype)
    before = d.state.clone()
    st = _status_word()
    run_gpu(d, device_status=st)
    torch.cuda.synchronize()
    assert st.item() == code
    if code:
        assert torch.equal(d.state, before)
        assert torch.all(d.out.view(torch.int16) == np.int16(np.uint16(0xC640).view(np.int16)))
    else:
        ref = upload(p, state_dtype=dtype)
        run_gpu(ref)
        torch.cuda.synchronize()
        assert torch.equal(d.state, ref.state) and torch.equal(d.out.view(torch.int16), ref.out.view(torch.int16))


@pytest.mark.parametrize("N,HV", [(2, 8), (33, 8), (64, 8)])
def test_validate_small_duplicate_at_every_distance(N, HV):
    """The in-wave duplicate check compares lanes through rotations: every
    pair of requests on one slot, whatever their distance in the call
    (1 to N - 1, across the wave's halves too), is rejected with code 2 and
    leaves the pool untouched; the intact call passes."""
    p = ki.make_problem("vdist", 130 + N, N=N, H=8, HV=HV, K=128, V=128, num_slots=N + 5, T=1)
    d = upload(p)
    before = d.state.clone()
    slots = d.slot_idx.clone()
    st = _status_word()
    missed = []
    for i in range(N):
        for j in range(i + 1, N):
            d.slot_idx.copy_(slots)
            d.slot_idx[j] = slots[i]
            st.fill_(-7)
            run_gpu(d, device_status=st)
            if st.item() != 2:
                missed.append((i, j))
    torch.cuda.synchronize()
    assert not missed, missed[:10]
    assert torch.equal(d.state, before)
    d.slot_idx.copy_(slots)
    run_gpu(d, device_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0


@pytest.mark.parametrize("N", [8, 64])
def test_validate_small_packed_cu_seqlens_past_the_tokens(N):
    """A packed call of at most 64 requests whose cu_seqlens ends past the
    call's token rows: code 3 from the decode's own check."""
    import ctypes
    p = ki.make_problem("vpast", 90 + N, N=N, H=2, HV=4, K=128, V=128, num_slots=N + 3, T=None)
    d = upload(p)
    before = d.state.clone()
    st = _status_word()
    a = kda.decode_args(d.q, d.k, d.v, d.g, d.beta, d.state, d.slot_idx, d.out, p.scale, device_status=st)
    rc = kda.library().kda_decode_packed(ctypes.byref(a), d.cu_seqlens.data_ptr(), p.tokens - 1,
                                         kda.KDA_FLAG_VALIDATE, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and st.item() == 3
    assert torch.equal(d.state, before)


def test_validate_rejects_cu_seqlens_past_the_tokens():
    """cu_seqlens[N] beyond total_tokens: the call is given fewer token rows
    than the tensors hold, so even an unvalidated run would stay in bounds."""
    import ctypes
    p = ki.workload("packed_n256_h12")
    d = upload(p)
    before = d.state.clone()
    st = _status_word()
    a = kda.decode_args(d.q, d.k, d.v, d.g, d.beta, d.state, d.slot_idx, d.out, p.scale, device_status=st)
    rc = kda.library().kda_decode_packed(ctypes.byref(a), d.cu_seqlens.data_ptr(), p.tokens - 1,
                                         kda.KDA_FLAG_VALIDATE, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and st.item() == 3
    assert torch.equal(d.state, before)


@pytest.mark.parametrize("case", ["valid", "duplicate", "past_pool", "cu_seqlens"])
def test_validate_many_requests(case):
    """10000 requests: the duplicate check's hash table takes 4096 values per
    pass, so this call makes three passes; a duplicate of the first live
    slot in the last live request is still found, valid metadata decodes."""
    N = 10000
    p = ki.make_problem("manyreq", 13, N=N, H=1, HV=1, K=128, V=128, num_slots=N + 16, T=None, t_max=2,
                        n_pad=N // 10)
    live = p.live_requests()
    code = 0
    if case == "duplicate":
        p.slot_idx[live[-1]] = p.slot_idx[live[0]]
        code = 2
    elif case == "past_pool":
        p.slot_idx[live[-1]] = p.num_slots
        code = 1
    elif case == "cu_seqlens":
        p.cu_seqlens[N - 3] = p.cu_seqlens[N - 1]
        code = 3
    d = upload(p)
    before = d.state.clone()
    st = _status_word()
    run_gpu(d, device_status=st)
    torch.cuda.synchronize()
    assert st.item() == code
    if code:
        assert torch.equal(d.state, before)
    else:
        _log("validated call, 10000 requests", compare(d, *run_oracle(p)))


def test_validate_inside_a_graph():
    """A captured validated call: replays with valid metadata decode, a replay
    after the slot indices were corrupted in place touches nothing."""
    p = ki.workload("n32_t1_h8")
    ref = _fresh(p)
    run_gpu(ref)
    d = _fresh(p)
    init = d.state.clone()
    st = _status_word()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run_gpu(d, device_status=st)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert st.item() == 0 and torch.equal(d.state, ref.state)
    good = d.slot_idx.clone()
    d.slot_idx[3] = d.slot_idx[9]
    d.state.copy_(init)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert st.item() == 2 and torch.equal(d.state, init)
    d.slot_idx.copy_(good)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert st.item() == 0 and torch.equal(d.state, ref.state)


# ------------------------------------------------------- edge cases
def test_host_tensors_in_a_gpu_call_are_refused(monkeypatch):
    """A host tensor among device tensors is refused by the binding before
    the library is reached (its address would be a host address on the
    GPU), and nothing on the device changes."""
    p = ki.make_problem("host", 12, N=2, H=2, HV=2, K=128, V=128, num_slots=4, T=1)
    d = upload(p)
    before = d.state.clone()

    def refuse():
        raise AssertionError("the library was reached")

    monkeypatch.setattr(kda, "library", refuse)
    with pytest.raises(ValueError, match="slot_idx is on cpu"):
        kda.kda_decode_step(d.q, d.k, d.v, d.g, d.beta, d.state, d.slot_idx.cpu(), d.out, T=1, scale=p.scale)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        kda.kda_decode_step(d.q.cpu(), d.k, d.v, d.g, d.beta, d.state, d.slot_idx, d.out, T=1, scale=p.scale)
    with pytest.raises(ValueError, match="cu_seqlens is on cpu"):
        kda.kda_decode_packed(d.q, d.k, d.v, d.g, d.beta, d.state, d.slot_idx, d.cu_seqlens.cpu(), d.out,
                              scale=p.scale)
    monkeypatch.undo()
    torch.cuda.synchronize()
    assert torch.equal(d.state, before)


def test_all_requests_padding():
    p = ki.make_problem("allpad", 5, N=4, H=2, HV=2, K=128, V=128, num_slots=6, T=None, n_pad=4)
    parity(p)


def test_out_of_range_slots_are_skipped():
    p = ki.make_problem("oor", 6, N=5, H=2, HV=2, K=128, V=128, num_slots=8, T=2)
    p.slot_idx[1] = 8
    p.slot_idx[3] = -7
    parity(p)


@pytest.mark.parametrize("packed", [False, True])
def test_more_requests_than_one_grid_holds(packed):
    """A call with more requests than a launch grid's request dimension
    (65535) runs as launches over request ranges: live requests on both
    sides of each range boundary, in every kernel family, against the
    oracle; padding rows untouched."""
    N = 65535 + 300
    p = ki.make_problem("ranges", 8, N=N, H=1, HV=1, K=128, V=128, num_slots=32, T=None if packed else 2,
                        t_max=2, n_pad=N - 16)
    live = [0, 1, 65533, 65534, 65535, 65536, 65537, N - 2, N - 1]
    p.slot_idx[:] = -1
    p.slot_idx[live] = np.arange(len(live), dtype=p.slot_idx.dtype) * 3
    K_ = kda.KDA_FLAG_KERNEL
    kinds = [0, K_(kda.KDA_KERNEL_QUARTER4)] if packed else [0, K_(kda.KDA_KERNEL_WIDE), K_(kda.KDA_KERNEL_SPLIT)]
    for flags in kinds:
        _log(f"request ranges packed={packed} flags={flags:#x}", parity(p, packed=packed, flags=flags))


def test_zero_length_requests_leave_state_alone():
    p = ki.make_problem("zlen", 7, N=5, H=1, HV=2, K=128, V=128, num_slots=8, T=None)
    lens = np.array([2, 0, 1, 0, 3])
    p.cu_seqlens = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tokens = int(p.cu_seqlens[-1])
    for f in ("q", "k", "v", "g", "beta"):
        setattr(p, f, getattr(p, f)[:tokens].copy())
    free = [s for s in range(p.num_slots) if s not in set(p.slot_idx[[0, 2, 4]].tolist())]
    p.slot_idx[[1, 3]] = free[:2]      # live, distinct slots, but no tokens: nothing may change
    d = upload(p)
    before = d.state.clone()
    run_gpu(d, packed=True)
    torch.cuda.synchronize()
    for s in free[:2]:
        assert torch.equal(d.state[s], before[s])
    ref_out, ref_state = run_oracle(p)
    compare(d, ref_out, ref_state)


def test_zero_requests():
    p = ki.make_problem("z", 8, N=1, H=1, HV=1, K=128, V=128, num_slots=1, T=1)
    d = upload(p)
    before = d.state.clone()
    kda.kda_decode_step(d.q[:0], d.k[:0], d.v[:0], d.g[:0], d.beta[:0], d.state, d.slot_idx[:0], d.out[:0],
                        T=1, scale=p.scale)
    torch.cuda.synchronize()
    assert torch.equal(before, d.state)


def test_reset_and_identity_on_gpu():
    p = ki.make_problem("special", 9, N=4, H=2, HV=2, K=128, V=128, num_slots=4, T=1)
    p.g[0] = -np.inf                         # request 0: full reset
    p.g[1, :, ::3] = -np.inf                 # request 1: a third of the rows reset
    p.g[2] = 0.0                             # request 2: identity (g = 0, beta = 0)
    p.beta[2] = 0.0
    d = upload(p)
    before = d.state.clone()
    run_gpu(d)
    torch.cuda.synchronize()
    s2 = int(p.slot_idx[2])
    assert torch.equal(d.state[s2], before[s2])          # bitwise unchanged
    ref_out, ref_state = run_oracle(p)
    compare(d, ref_out, ref_state)


@pytest.mark.parametrize("N,T,raw", [(4, 2, False), (25, 4, False), (4, 1, True)])
def test_large_slot_offsets(N, T, raw):
    """Slots whose element offset exceeds 2^31 (pool > 8 GiB at HV = 8): 32
    tiles at T = 2 and 200 tiles at T = 4 (the multi-token kernels), and 32
    one-token tiles with the fused gate (two 16-column waves that store the
    state straight from the lanes)."""
    HV, slots = 8, 16400
    p = ki.make_problem("big", 10, N=N, H=8, HV=HV, K=128, V=128, num_slots=slots, T=T, raw_gates=raw)
    print(f"[parity] large offsets N={N} T={T} raw={raw}: layout "
          f"{kda.kda_decode_plan(N * HV, T, raw_gate=raw, layout=True)}", flush=True)
    p.slot_idx[:] = ([16399, 16384, 3, 16390] + list(range(16360, 16381)))[:N]
    d = upload(p)
    run_gpu(d)
    torch.cuda.synchronize()
    ref_out, ref_state = run_oracle(p)
    _log("large offsets", compare(d, ref_out, ref_state))
    del d
    torch.cuda.empty_cache()


def test_strided_views_of_fused_projection():
    p = ki.make_problem("fused", 11, N=6, H=2, HV=4, K=128, V=128, num_slots=9, T=2)
    d = upload(p)
    T, HK, HVV = p.tokens, p.H * p.K, p.HV * p.V
    fused = torch.zeros((T, 2 * HK + HVV + 64), dtype=torch.bfloat16, device=DEV)
    fused[:, :HK] = d.q.reshape(T, HK)
    fused[:, HK:2 * HK] = d.k.reshape(T, HK)
    fused[:, 2 * HK:2 * HK + HVV] = d.v.reshape(T, HVV)
    beta_wide = torch.zeros((T, p.HV + 3), dtype=torch.float32, device=DEV)
    beta_wide[:, :p.HV] = d.beta
    d.q = fused[:, :HK].view(T, p.H, p.K)
    d.k = fused[:, HK:2 * HK].view(T, p.H, p.K)
    d.v = fused[:, 2 * HK:2 * HK + HVV].view(T, p.HV, p.V)
    d.beta = beta_wide[:, :p.HV]
    run_gpu(d)
    torch.cuda.synchronize()
    ref_out, ref_state = run_oracle(p)
    compare(d, ref_out, ref_state)


# ------------------------------------------------------- bit-exact properties
def _fresh(p, seed=1234):
    d = upload(p, background_seed=seed)
    return d


def test_tile_widths_bit_identical():
    for name in ("n32_t1_h8", "n8_t4_h8", "packed_n256_h12"):
        p = ki.workload(name)
        results = []
        for width in (32, 64, 128):
            d = _fresh(p)
            run_gpu(d, flags=kda.KDA_FLAG_VTILE(width))
            torch.cuda.synchronize()
            results.append((d.out.view(torch.int16).clone(), d.state.clone()))
        for o, s in results[1:]:
            assert torch.equal(o, results[0][0]) and torch.equal(s, results[0][1]), name


# ------------------------------------------------------- 16-column waves
SPLIT, QUARTER = kda.KDA_LAYOUT_SPLIT, kda.KDA_LAYOUT_QUARTER
QUARTER_CASES = [
    # (N, H, HV, T, raw gates, the 16-column-wave layout the library picks);
    # the library also picks the load order: the first token's inputs before
    # the tile for calls of two or more tokens on the split-key waves from
    # 192 tiles to 256 and on four 16-column waves with three or more
    # tokens, the tile first otherwise
    (1, 8, 8, 4, False, SPLIT),       # 8 tiles
    (5, 1, 3, 2, False, SPLIT),       # three value heads per q/k head
    (9, 4, 8, 3, True, SPLIT),        # fused gate activation
    (24, 4, 8, 4, False, SPLIT),      # 192 tiles, four tokens, inputs first
    (7, 2, 4, 6, True, SPLIT),        # tokens past the four whose inputs load with the tile
    (8, 8, 8, 1, False, SPLIT),       # one token, 64 tiles
    (16, 2, 8, 1, False, SPLIT),      # one token, 128 tiles
    (8, 2, 8, 1, True, QUARTER),      # one token, 64 tiles, fused gate: two waves per workgroup
    (32, 8, 8, 4, False, SPLIT),      # 256 tiles: the split-key layout's last inputs-first size
    (40, 8, 8, 3, False, SPLIT),      # 320 tiles, three tokens, tile first: its last size
    (40, 8, 8, 4, False, SPLIT),      # 320 tiles, four tokens, tile first
    (24, 2, 8, 2, True, SPLIT),       # 192 tiles, two tokens, fused gate, inputs first
    (36, 4, 8, 4, False, SPLIT),      # 288 tiles, four tokens, tile first
    (42, 4, 8, 4, False, QUARTER),    # 336 tiles: four waves per workgroup, inputs first
    (41, 8, 8, 2, True, QUARTER),     # 328 tiles, two tokens, fused gate, tile first
    (44, 2, 6, 5, False, SPLIT),      # 264 tiles, five tokens
    (56, 2, 6, 5, False, QUARTER),    # 336 tiles, five tokens
    (60, 8, 8, 2, False, QUARTER),    # 480 tiles, two tokens
    (70, 8, 8, 4, False, QUARTER),    # 560 tiles, four tokens, inputs first
    (36, 8, 8, 1, False, QUARTER),    # one token, 288 tiles: four waves per workgroup
    (48, 2, 8, 1, False, QUARTER),    # one token, 384 tiles: the last size on four waves
    (34, 4, 8, 1, True, QUARTER),     # one token, 272 tiles, fused gate: four waves
]


LARGE_MULTI_TOKEN_CASES = [
    # (N, T, fused gate, columns per workgroup, layout): fp32 step calls past
    # the split-key range, H = HV = 8
    (72, 2, False, 64, kda.KDA_LAYOUT_WIDE),      # 576 tiles, two tokens: 32-column waves, 64 columns
    (90, 3, True, 128, kda.KDA_LAYOUT_WIDE),      # 720 tiles, three tokens: 32-column waves, 128 columns
    (100, 2, False, 64, QUARTER),                 # 800 tiles: four 16-column waves again, tile first
    (100, 4, True, 64, QUARTER),                  # 800 tiles, four tokens: inputs first
    (200, 2, False, 128, QUARTER),                # 1600 tiles: eight 16-column waves, inputs first
]


@pytest.mark.parametrize("case", LARGE_MULTI_TOKEN_CASES)
def test_large_multi_token_calls(case):
    """The plan's kernels for many tiles and several tokens per request
    against the oracle, and bit for bit against the 32-column kernel at a
    forced width and four forced 16-column waves."""
    N, T, raw, width, layout = case
    p = ki.make_problem("large", 500 + N, N=N, H=8, HV=8, K=128, V=128, num_slots=N + 11, T=T, n_pad=N // 10,
                        raw_gates=raw)
    assert kda.kda_decode_plan(N * 8, T, False, raw_gate=raw) == width
    assert kda.kda_decode_plan(N * 8, T, False, raw_gate=raw, layout=True) == layout
    results = []
    for flags in (0, kda.KDA_FLAG_VTILE(128), kda.KDA_FLAG_KERNEL(kda.KDA_KERNEL_QUARTER4)):
        d = _fresh(p)
        run_gpu(d, flags=flags)
        torch.cuda.synchronize()
        assert_guards(d)
        if flags == 0:
            _log(f"large multi-token {case}", compare(d, *run_oracle(p)))
        results.append((d.out.view(torch.int16).clone(), d.state.clone()))
    for o, st in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(st, results[0][1]), case


@pytest.mark.parametrize("case", QUARTER_CASES)
def test_quarter_waves_match_wide_waves_bitwise(case):
    """The 16-column-wave kernels (the library's choice at these shapes:
    split-key waves of 16 key rows per lane, or two or four waves of 32 rows
    per lane) and the 32-column kernel (every forced tile width) give the same
    bits: outputs, final states and per-token states; and they match the
    oracle."""
    N, H, HV, T, raw, layout = case
    p = ki.make_problem("quarter", 300 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=2 * N + 3, T=T,
                        n_pad=N // 4, raw_gates=raw)
    assert kda.kda_decode_plan(N * HV, T, False, layout=True, raw_gate=raw) == layout
    two_waves = raw and T == 1 and N * HV <= 64  # 32 columns per workgroup
    assert kda.kda_decode_plan(N * HV, T, False, raw_gate=raw) == (64 if layout == QUARTER and not two_waves else 32)
    results = []
    for flags in (0, kda.KDA_FLAG_VTILE(32), kda.KDA_FLAG_VTILE(64), kda.KDA_FLAG_VTILE(128)):
        d = _fresh(p)
        inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), 1232.0, torch.float32)
        run_gpu(d, flags=flags, inter_state=inter)
        torch.cuda.synchronize()
        assert_guards(d)
        if flags == 0:
            ref_inter = np.full((p.tokens, p.HV, p.K, p.V), np.nan)
            ref_out, ref_state = run_oracle(p, inter_state=ref_inter)
            _log(f"quarter waves {case}", compare(d, ref_out, ref_state))
            live_rows = np.isfinite(ref_inter[:, 0, 0, 0])
            got = inter.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(got[live_rows] - ref_inter[live_rows]) <= 1e-4 * np.abs(ref_inter[live_rows]) + 1e-6)
            assert np.all(got[~live_rows] == 1232.0)
        results.append((d.out.view(torch.int16).clone(), d.state.clone(), inter))
    for o, st, it in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(st, results[0][1]) and torch.equal(it, results[0][2])


@pytest.mark.parametrize("case", [(1, 8, 8, 1, False, SPLIT), (3, 8, 8, 1, False, SPLIT),
                                  (4, 8, 8, 1, False, QUARTER), (1, 8, 8, 1, True, QUARTER), (1, 8, 8, 2, False, SPLIT),
                                  (4, 8, 8, 4, True, SPLIT), (7, 2, 4, 6, False, SPLIT),
                                  (9, 4, 8, 3, True, QUARTER), (20, 4, 8, 4, False, QUARTER),
                                  (32, 8, 8, 2, False, QUARTER), (64, 8, 8, 1, False, QUARTER),
                                  (40, 4, 4, None, False, QUARTER), (25, 2, 6, None, True, QUARTER)])
def test_quarter_waves_bf16_pool_match_wide_waves_bitwise(case):
    """bf16 pool: the 16-column waves (widened exactly into LDS, rounded once
    on the way out; split-key waves for several tokens up to 32 tiles and
    for one token with activated gates up to 24, else 64-column
    workgroups), step and packed (T None: 1 to 6 tokens per
    request), against the forced 32-column kernel, bit for bit with
    per-token states; and against the oracle."""
    N, H, HV, T, raw, layout = case
    p = ki.make_problem("quarterbf", 400 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=2 * N + 3, T=T,
                        t_max=6, n_pad=N // 4, raw_gates=raw)
    assert kda.kda_decode_plan(N * HV, T or 1, bf16_state=True, packed=T is None, layout=True,
                               raw_gate=raw) == layout
    results = []
    for flags in (0, kda.KDA_FLAG_VTILE(32), kda.KDA_FLAG_VTILE(128)):
        d = upload(p, background_seed=1234, state_dtype=torch.bfloat16)
        inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), 1232.0, torch.bfloat16)
        run_gpu(d, flags=flags, inter_state=inter)
        torch.cuda.synchronize()
        assert_guards(d)
        if flags == 0:
            _log(f"quarter waves bf16 {case}", compare(d, *run_oracle(p, state_bf16=True)))
        results.append((d.out.view(torch.int16).clone(), d.state.view(torch.int16).clone(),
                        inter.view(torch.int16).clone()))
    for o, st, it in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(st, results[0][1]) and torch.equal(it, results[0][2])


NORM_QUARTER_CASES = [
    # (N, H, HV, T, raw gates, pool dtype): the library picks eight 16-column waves per workgroup
    (9, 4, 4, 2, False, torch.float32),
    (5, 2, 6, 5, True, torch.float32),       # tokens past the four loaded ahead
    (32, 16, 16, 4, False, torch.float32),
    (3, 2, 4, 1, False, torch.bfloat16),
    (32, 16, 16, 1, True, torch.bfloat16),
    (6, 1, 2, None, False, torch.bfloat16),  # packed, 1 to 6 tokens per request
]


@pytest.mark.parametrize("case", NORM_QUARTER_CASES)
def test_quarter_waves_norm_match_wide_waves_bitwise(case):
    """The gated RMSNorm epilogue on the 16-column waves (one head per
    workgroup, the sum of squares in the 32-column kernel's order) against
    the forced 32-column kernel, bit for bit with per-token states; and
    against the oracle."""
    N, H, HV, T, raw, dtype = case
    p = ki.make_problem("quarternorm", 600 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=2 * N + 3, T=T,
                        t_max=6, n_pad=N // 4, norm=True, raw_gates=raw)
    results = []
    for flags in (0, kda.KDA_FLAG_VTILE(128)):
        d = upload(p, background_seed=1234, state_dtype=dtype)
        inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), 1232.0, dtype)
        run_gpu(d, flags=flags, inter_state=inter)
        torch.cuda.synchronize()
        assert_guards(d)
        if flags == 0:
            _log(f"quarter waves norm {case}", compare(d, *run_oracle(p, state_bf16=dtype == torch.bfloat16)))
        results.append((d.out.view(torch.int16).clone(), d.state.view(torch.int16).clone(),
                        inter.view(torch.int16).clone()))
    o, st, it = results[1]
    assert torch.equal(o, results[0][0]) and torch.equal(st, results[0][1]) and torch.equal(it, results[0][2])


@pytest.mark.parametrize("case", [(64, 8, 8, 1, True, 128), (130, 4, 4, None, False, 64),
                                  (130, 4, 4, None, True, 64), (260, 4, 4, None, False, 128),
                                  (40, 4, 4, None, True, 64)])
def test_eight_quarter_waves_match_wide_waves_bitwise(case):
    """16-column waves of fp32 one-token calls from 400 tiles and packed
    calls (four waves per workgroup up to 1024 tiles, eight beyond; eight
    forced at every size) against the forced 32-column kernel, bit for bit
    with per-token states, fused gate or not; the final state against the
    oracle."""
    N, H, HV, T, raw, width = case
    p = ki.make_problem("eightq", 800 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=N + 9, T=T, t_max=3,
                        n_pad=N // 8, raw_gates=raw)
    assert kda.kda_decode_plan(N * HV, T or 1, packed=T is None) == width
    results = []
    for flags in (0, kda.KDA_FLAG_VTILE(128), kda.KDA_FLAG_KERNEL(kda.KDA_KERNEL_QUARTER8)):
        d = _fresh(p)
        inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), 1232.0, torch.float32)
        run_gpu(d, flags=flags, inter_state=inter)
        torch.cuda.synchronize()
        assert_guards(d)
        if flags == 0:
            _log(f"eight quarter waves {case}", compare(d, *run_oracle(p)))
        results.append((d.out.view(torch.int16).clone(), d.state.clone(), inter))
    for o, st, it in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(st, results[0][1]) and torch.equal(it, results[0][2])


@pytest.mark.parametrize("case", [(1, 8, 8, 4), (8, 8, 8, 4), (5, 2, 6, 3), (7, 1, 3, 2), (33, 8, 8, 2),
                                  (11, 4, 12, 4), (3, 1, 5, 6)])
def test_head_per_xcd_placement_bitwise(case):
    """Split-key calls with a head's value tiles placed on one XCD
    (KDA_PLACEMENT_HEAD_XCD: groups of 8 heads x 4 tiles, a partial last
    group when the head count is not a multiple of 8) against the default
    placement, bit for bit with per-token states, both load orders, with
    and without the fused gate; the placed call against the oracle."""
    N, H, HV, T = case
    split = kda.KDA_FLAG_KERNEL(kda.KDA_KERNEL_SPLIT)
    xcd = kda.KDA_FLAG_PLACEMENT(kda.KDA_PLACEMENT_HEAD_XCD)
    for raw in (False, True):
        p = ki.make_problem("xcd", 900 + N, N=N, H=H, HV=HV, K=128, V=128, num_slots=N + 5, T=T, n_pad=N // 5,
                            raw_gates=raw)
        for order in (kda.KDA_ORDER_TILE_FIRST, kda.KDA_ORDER_INPUTS_FIRST):
            results = []
            for placement in (0, xcd):
                d = _fresh(p)
                inter = guarded_full(d, (p.tokens, p.HV, p.K, p.V), 1232.0, torch.float32)
                run_gpu(d, flags=split | kda.KDA_FLAG_ORDER(order) | placement, inter_state=inter)
                torch.cuda.synchronize()
                assert_guards(d)
                if placement and order == kda.KDA_ORDER_INPUTS_FIRST:
                    _log(f"head per XCD {case} raw={raw}", compare(d, *run_oracle(p)))
                results.append((d.out.view(torch.int16).clone(), d.state.clone(), inter))
            (o0, s0, i0), (o1, s1, i1) = results
            assert torch.equal(o0, o1) and torch.equal(s0, s1) and torch.equal(i0, i1), (case, raw, order)


def test_quarter_waves_full_t4_sweep_match_wide_waves():
    """The T = 4 serving sweep: the library's choice against the forced
    32-column kernel, bit for bit."""
    for n in (1, 8, 16, 24, 32):
        p = ki.workload(f"n{n}_t4_h8")
        a = _fresh(p)
        run_gpu(a)
        b = _fresh(p)
        run_gpu(b, flags=kda.KDA_FLAG_VTILE(128))
        torch.cuda.synchronize()
        assert torch.equal(a.state, b.state) and torch.equal(a.out.view(torch.int16), b.out.view(torch.int16)), n


def _one_request(p, i):
    """Request i of problem p as a call of its own (same inputs, same slot)."""
    import dataclasses
    lo, hi = int(p.cu_seqlens[i]), int(p.cu_seqlens[i + 1])
    cut = lambda a: None if a is None else a[lo:hi].copy()
    return dataclasses.replace(p, N=1, cu_seqlens=np.array([0, hi - lo], dtype=np.int32),
                               slot_idx=p.slot_idx[i:i + 1].copy(), q=cut(p.q), k=cut(p.k), v=cut(p.v),
                               g=cut(p.g), beta=cut(p.beta), gate=cut(p.gate), raw_gate=cut(p.raw_gate),
                               raw_beta=cut(p.raw_beta))


@pytest.mark.parametrize("T,raw", [(1, False), (1, True), (2, True), (4, False)])
def test_results_do_not_depend_on_the_batch(T, raw):
    """A request decoded inside a batch of 64 (512 tiles: eight or four
    16-column waves) and alone (8 tiles: split-key or two 16-column waves)
    gives the same output and state bits."""
    N = 64
    p = ki.make_problem("batch", 40 + T, N=N, H=8, HV=8, K=128, V=128, num_slots=N + 4, T=T, raw_gates=raw)
    whole = _fresh(p)
    run_gpu(whole)
    torch.cuda.synchronize()
    assert kda.kda_decode_plan(8, T, False, raw_gate=raw, layout=True) != \
        kda.kda_decode_plan(N * 8, T, False, raw_gate=raw, layout=True) or T == 1
    for i in (0, 17, N - 1):
        alone = _fresh(_one_request(p, i))
        run_gpu(alone)
        torch.cuda.synchronize()
        lo, hi, slot = int(p.cu_seqlens[i]), int(p.cu_seqlens[i + 1]), int(p.slot_idx[i])
        assert torch.equal(alone.out.view(torch.int16), whole.out[lo:hi].view(torch.int16)), i
        assert torch.equal(alone.state[slot], whole.state[slot]), i


def test_chained_single_tokens_bit_identical():
    p = ki.workload("n32_t4_h8")
    d_multi = _fresh(p)
    run_gpu(d_multi)
    d = _fresh(p)
    N = p.N
    for t in range(4):
        rows = torch.arange(N, device=DEV) * 4 + t
        out_t = torch.empty((N, p.HV, p.V), dtype=torch.bfloat16, device=DEV)
        kda.kda_decode_step(d.q[rows], d.k[rows], d.v[rows], d.g[rows], d.beta[rows], d.state, d.slot_idx,
                            out_t, T=1, scale=p.scale)
        d.out[rows] = out_t
    torch.cuda.synchronize()
    assert torch.equal(d.state, d_multi.state)
    assert torch.equal(d.out.view(torch.int16), d_multi.out.view(torch.int16))


def test_request_permutation_bit_identical():
    p = ki.workload("packed_n256_h12")
    d = _fresh(p)
    run_gpu(d)
    perm = np.random.default_rng(3).permutation(p.N)
    cu = p.cu_seqlens
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in perm])
    lens = np.diff(cu)[perm]
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d2 = _fresh(p)
    r = torch.from_numpy(rows).to(DEV)
    out2 = torch.empty_like(d2.out)
    kda.kda_decode_packed(d2.q[r], d2.k[r], d2.v[r], d2.g[r], d2.beta[r], d2.state,
                          torch.from_numpy(p.slot_idx[perm].astype(np.int32)).to(DEV),
                          torch.from_numpy(cu2).to(DEV), out2, scale=p.scale)
    torch.cuda.synchronize()
    assert torch.equal(d2.state, d.state)
    live_rows = torch.from_numpy(np.isin(rows, np.concatenate(
        [np.arange(cu[n], cu[n + 1]) for n in p.live_requests()]))).to(DEV)
    assert torch.equal(out2.view(torch.int16)[live_rows], d.out.view(torch.int16)[r][live_rows])


def test_deterministic_and_non_default_stream():
    p = ki.workload("n32_t1_h16_norm")
    d1 = _fresh(p)
    run_gpu(d1)
    d2 = _fresh(p)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        run_gpu(d2)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(d1.state, d2.state)
    assert torch.equal(d1.out.view(torch.int16), d2.out.view(torch.int16))


@pytest.mark.parametrize("name", ["n32_t1_h8", "n8_t4_h8", "n32_t4_h8"])
def test_graph_replay_matches_eager(name):
    p = ki.workload(name)
    eager = _fresh(p)
    run_gpu(eager)
    torch.cuda.synchronize()
    d = _fresh(p)
    init = d.state.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run_gpu(d)
    torch.cuda.synchronize()
    for _ in range(3):
        d.state.copy_(init)                  # eager work between replays
        d.out.view(torch.int16).fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.state, eager.state)
        assert torch.equal(d.out.view(torch.int16), eager.out.view(torch.int16))


_FIRST_CALL_IN_CAPTURE = r"""
import sys, torch
sys.path[:0] = [sys.argv[1], sys.argv[1] + "/tests"]
import kda_inputs as ki
from kda_harness import run_gpu, upload
p = ki.make_problem("capture", 5, N=130, H=4, HV=4, K=128, V=128, num_slots=140, T=None, t_max=3, n_pad=5)
d = upload(p)
init = d.state.clone()
g = torch.cuda.CUDAGraph()
s = torch.cuda.Stream()
s.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(s):
    with torch.cuda.graph(g, stream=s):
        run_gpu(d)                       # the process's first library call
torch.cuda.synchronize()
outs = []
for _ in range(2):
    d.state.copy_(init)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    outs.append((d.state.clone(), d.out.clone()))
e = upload(p)
run_gpu(e)
torch.cuda.synchronize()
for st, o in outs:
    assert torch.equal(st, e.state) and torch.equal(o.view(torch.int16), e.out.view(torch.int16))
print("first call in capture ok")
"""


def test_first_library_call_inside_graph_capture():
    """A process whose first call is captured into a HIP graph (eight
    16-column waves: the library raises their LDS limit at its first call
    on a device) replays it correctly."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_IN_CAPTURE, root], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "first call in capture ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


# ------------------------------------------------------- standalone norm
@pytest.mark.parametrize("rows,V", [(512, 128), (5, 128), (3, 2), (7, 130), (33, 1024), (2, 8192)])
def test_gated_rmsnorm(rows, V):
    import oracle
    x = ki.to_bf16_bits(ki.normal(31, 1, rows * V).reshape(rows, V) * 0.05)
    z = ki.to_bf16_bits(ki.normal(31, 2, rows * V).reshape(rows, V))
    w = ki.to_bf16_bits(1.0 + 0.02 * ki.normal(31, 3, V))
    ref = oracle.gated_rmsnorm(x, z, w, 1e-6)
    xt, zt, wt = bf16_tensor(x), bf16_tensor(z), bf16_tensor(w)
    y = torch.empty_like(xt)
    kda.kda_gated_rmsnorm(xt, zt, wt, y, 1e-6)
    torch.cuda.synchronize()
    from kda_harness import bf16_to_f64, bf16_ulp
    got = bf16_to_f64(y)
    err = np.abs(got - ref)
    assert np.all(err <= 2e-3 + 2.0 ** -8 * np.abs(ref))
    assert np.all(err <= bf16_ulp(ref) + 1e-6 * np.abs(ref).max())
    # in place
    kda.kda_gated_rmsnorm(xt, zt, wt, xt, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(xt.view(torch.int16), y.view(torch.int16))


# ------------------------------------------------------- the benchmark's tile-stream reference
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_stream_reference_leaves_the_pool_unchanged(dtype):
    """libkda_stream.so moves the live tiles in place and computes nothing:
    the pool (and the guard bytes around it) are bitwise unchanged, slots
    outside the pool and padding rows are skipped, N = 0 enqueues nothing."""
    HV, slots = 4, 9
    elem = 4 if dtype == torch.float32 else 2
    g = torch.Generator(device="cpu").manual_seed(5)
    raw = torch.randint(-2 ** 15, 2 ** 15, (slots + 2, HV, 128, 128), dtype=torch.int32, generator=g)
    full = (raw.float() if dtype == torch.float32 else raw.to(torch.int16).view(torch.bfloat16)).to(DEV)
    pool = full[1:slots + 1]
    before = full.clone()
    slot_idx = torch.tensor([3, -1, 0, 8, slots, 5, -7], dtype=torch.int32, device=DEV)
    lib = kda.stream_library()
    sh = torch.cuda.current_stream().cuda_stream
    assert lib.kda_stream_tiles(pool.data_ptr(), elem, slots, HV * 128 * 128, slot_idx.data_ptr(), 7, HV, sh) == 0
    assert lib.kda_stream_tiles(pool.data_ptr(), elem, slots, HV * 128 * 128, slot_idx.data_ptr(), 0, HV, sh) == 0
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16 if elem == 2 else torch.int32),
                       before.view(torch.int16 if elem == 2 else torch.int32))

"""Test harness shared by the GPU tests: put a seeded problem on the GPU, run
the HIP path through the C ABI, run the CPU oracle on the same inputs, and
compare.

Tolerances (the stated ones are the acceptance bar; the strict ones are
what fp32 arithmetic on this path actually delivers and catch slips that the
stated bar would let through, such as a 1% scale error on outputs near 0.05):

  out, stated   |y_gpu - y_ref| <= 2e-3 + 2^-8 |y_ref|
                (2e-3 max-abs plus the half-ulp a bf16 rounding of the exact
                value may add: one bf16 ulp is at most 2^-7 |y|)
  out, strict   |y_gpu - y_ref| <= ulp_bf16(y_ref) + 1e-6 max|y_ref|
  state, stated |S_gpu - S_ref| <= 1e-4 |S_ref| + 1e-6
                (relative 1e-4, with an absolute floor for entries that
                cancel to ~0; the state's scale is ~0.05)
  state, strict |S_gpu - S_ref| <= 2e-6 max|S_ref| per (slot, head) tile
With a bf16 state pool the stored state carries one bf16 rounding:
  state, stated |S_gpu - S_ref| <= 2^-8 |S_ref| + 1e-6   (half a bf16 ulp)
  state, strict |S_gpu - S_ref| <= ulp_bf16(S_ref) + 2e-6 max|S_ref| per tile
where y_ref and S_ref are the oracle's double-precision values (the oracle
starts from the bf16 state widened exactly).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import kda_inputs as ki
import linear_attention_recurrent_decode_amd as kda
import oracle

DEV = "cuda:0"
SENTINEL_BITS = 0xC640     # bf16 -12288.0: marks output rows nobody may write
GUARD_BYTES = 4096         # guard region on each side of every buffer the library writes
GUARD_WORD = 0x7FA5        # 16-bit guard pattern (a NaN as bf16, and as the high half of an fp32)


class Guarded:
    """A device tensor with GUARD_BYTES of a fixed bit pattern on each side,
    carved out of one allocation, so that a write past either end of the
    tensor lands in a guard region and is seen by ``intact()``, instead of
    corrupting whatever torch put next to it."""

    def __init__(self, shape, dtype: torch.dtype):
        self.shape, self.dtype = tuple(shape), dtype
        nbytes = int(np.prod(self.shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = nbytes
        self.raw = torch.empty(2 * GUARD_BYTES + nbytes, dtype=torch.uint8, device=DEV)
        self.raw.view(torch.int16).fill_(GUARD_WORD)
        self.tensor = self.raw[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(self.shape)

    def intact(self) -> bool:
        words = self.raw.view(torch.int16)
        g = GUARD_BYTES // 2
        return bool((words[:g] == GUARD_WORD).all()) and bool((words[g + self.nbytes // 2:] == GUARD_WORD).all())


# every DeviceProblem upload() made since the last reset: a test's teardown
# checks all their guards (check_all_guards), whether or not it compared
CREATED: list = []


def check_all_guards():
    """Assert the guards of every problem uploaded since the last call, then forget them."""
    try:
        for d in CREATED:
            assert_guards(d)
    finally:
        CREATED.clear()


def guarded_empty(d, shape, dtype) -> torch.Tensor:
    """A guarded tensor whose guards ``compare`` (and ``assert_guards``)
    check along with the problem's own (for inter_state buffers and the like)."""
    gt = Guarded(shape, dtype)
    d.guards.append(gt)
    return gt.tensor


def guarded_full(d, shape, value, dtype=torch.float32) -> torch.Tensor:
    """guarded_empty filled with ``value``."""
    t = guarded_empty(d, shape, dtype)
    t.fill_(value)
    return t


def assert_guards(d):
    """Every guard region around the problem's written buffers still holds its pattern."""
    torch.cuda.synchronize()
    for gt in d.guards:
        assert gt.intact(), f"a write past the end of a {gt.dtype} {gt.shape} buffer"


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return ki.bf16_bits_to_f32(bits).astype(np.float64)


def f32_tensor(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


@dataclasses.dataclass
class DeviceProblem:
    p: ki.Problem
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor | None
    beta: torch.Tensor | None
    state: torch.Tensor
    slot_idx: torch.Tensor
    cu_seqlens: torch.Tensor
    out: torch.Tensor
    gate: torch.Tensor | None
    norm_weight: torch.Tensor | None
    live_slots: np.ndarray        # the pool slots of live requests, in request order
    raw_gate: torch.Tensor | None = None
    raw_beta: torch.Tensor | None = None
    A_log: torch.Tensor | None = None
    dt_bias: torch.Tensor | None = None
    guards: list = dataclasses.field(default_factory=list)

    def gate_kwargs(self) -> dict:
        """The raw gate inputs as keyword arguments of the binding (empty for
        activated problems)."""
        if self.raw_gate is None:
            return {}
        return dict(raw_gate=self.raw_gate, raw_beta=self.raw_beta, A_log=self.A_log, dt_bias=self.dt_bias)


def upload(p: ki.Problem, background_seed: int = 1234, state_dtype=torch.float32) -> DeviceProblem:
    """Inputs to the GPU.  The pool is filled with a seeded N(0, 0.05)
    background generated on the device (these slots are only checked for
    being left alone) and the live slots get the generator's values (rounded
    to bf16 for a bf16 pool)."""
    live = p.live_requests()
    live_slots = p.slot_idx[live].astype(np.int64)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(background_seed)
    state_g = Guarded((p.num_slots, p.HV, p.K, p.V), state_dtype)
    state = state_g.tensor
    state.copy_(torch.randn((p.num_slots, p.HV, p.K, p.V), generator=gen, device=DEV, dtype=torch.float32) * 0.05)
    if len(live_slots):
        vals = p.state_slots(live_slots)
        if state_dtype == torch.bfloat16:
            live_t = bf16_tensor(ki.f32_to_bf16_bits(vals))
        else:
            live_t = f32_tensor(vals)
        state[torch.from_numpy(live_slots).to(DEV)] = live_t
    out_g = Guarded((p.tokens, p.HV, p.V), torch.bfloat16)
    out = out_g.tensor
    out.view(torch.int16).fill_(int(np.uint16(SENTINEL_BITS).view(np.int16)))
    raw = {}
    if p.raw:
        raw = dict(raw_gate=bf16_tensor(p.raw_gate), raw_beta=bf16_tensor(p.raw_beta), A_log=f32_tensor(p.A_log),
                   dt_bias=f32_tensor(p.dt_bias))
    d = DeviceProblem(
        p=p, q=bf16_tensor(p.q), k=bf16_tensor(p.k), v=bf16_tensor(p.v),
        g=None if p.g is None else f32_tensor(p.g), beta=None if p.beta is None else f32_tensor(p.beta), state=state,
        slot_idx=torch.from_numpy(p.slot_idx.astype(np.int32)).to(DEV),
        cu_seqlens=torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(DEV), out=out,
        gate=None if p.gate is None else bf16_tensor(p.gate),
        norm_weight=None if p.norm_weight is None else bf16_tensor(p.norm_weight),
        live_slots=live_slots, guards=[state_g, out_g], **raw)
    CREATED.append(d)
    return d


def run_gpu(d: DeviceProblem, packed: bool | None = None, flags: int = 0, stream=None, device_status=None,
            inter_state=None):
    p = d.p
    if packed is None:
        packed = p.T is None
    kw = dict(scale=p.scale, gate=d.gate, norm_weight=d.norm_weight, eps=p.eps, flags=flags, stream=stream,
              device_status=device_status, inter_state=inter_state, **d.gate_kwargs())
    if packed:
        kda.kda_decode_packed(d.q, d.k, d.v, d.g, d.beta, d.state, d.slot_idx, d.cu_seqlens, d.out, **kw)
    else:
        kda.kda_decode_step(d.q, d.k, d.v, d.g, d.beta, d.state, d.slot_idx, d.out, T=p.T, **kw)


def run_oracle(p: ki.Problem, state_bf16: bool = False, inter_state=None):
    """Oracle over the live requests only, on a compact double pool holding
    just their slots.  Returns (out [tokens, HV, V] with NaN on skipped rows,
    final state [n_live, HV, K, V] in request order).  ``inter_state``: an
    optional float64 [tokens, HV, K, V] array that receives each token's state."""
    live = p.live_requests()
    slots = p.slot_idx[live].astype(np.int64)
    pool = p.state_slots(slots)
    if state_bf16:
        pool = ki.bf16_bits_to_f32(ki.f32_to_bf16_bits(pool))
    pool = pool.astype(np.float64)
    remap = np.full(p.N, -1, dtype=np.int32)
    remap[live] = np.arange(len(live), dtype=np.int32)
    kw = {}
    if p.gate is not None:
        kw = dict(gate=p.gate, norm_weight=p.norm_weight, eps=p.eps)
    if p.raw:
        kw.update(raw_gate=p.raw_gate, raw_beta=p.raw_beta, A_log=p.A_log, dt_bias=p.dt_bias)
    out = oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, pool, remap, p.cu_seqlens, p.scale,
                               inter_state=inter_state, **kw)
    return out, pool


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@dataclasses.dataclass
class Report:
    out_max_abs: float
    out_max_ulp: float
    state_max_rel_tile: float
    state_max_abs: float

    def __str__(self):
        return (f"out max|d|={self.out_max_abs:.3e} ({self.out_max_ulp:.2f} bf16 ulp), "
                f"state max|d|={self.state_max_abs:.3e} (tile-rel {self.state_max_rel_tile:.3e})")


def compare(d: DeviceProblem, ref_out: np.ndarray, ref_state: np.ndarray, strict: bool = True) -> Report:
    """Stated and strict tolerances on outputs and final state; skipped rows
    must still hold the sentinel; every guard region is intact."""
    p = d.p
    assert_guards(d)
    out = bf16_to_f64(d.out)
    live = np.isfinite(ref_out)
    dead_rows = ~live
    out_bits = d.out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(out_bits[dead_rows] == SENTINEL_BITS), "a skipped request's output row was written"
    y, r = out[live], ref_out[live]
    err = np.abs(y - r)
    assert np.all(err <= 2e-3 + 2.0 ** -8 * np.abs(r)), f"output outside the stated tolerance: max {err.max()}"
    floor = 1e-6 * (np.abs(r).max() if r.size else 0.0)
    if strict:
        bad = err > bf16_ulp(r) + floor
        assert not bad.any(), f"output beyond 1 bf16 ulp: {err[bad][:5]} at ref {r[bad][:5]}"

    bf16_state = d.state.dtype == torch.bfloat16
    if len(d.live_slots):
        S_t = d.state[torch.from_numpy(d.live_slots).to(DEV)]
        S = bf16_to_f64(S_t) if bf16_state else S_t.cpu().numpy().astype(np.float64)
    else:
        S = np.zeros((0, p.HV, p.K, p.V))
    serr = np.abs(S - ref_state)
    tile_max = np.abs(ref_state).max(axis=(2, 3), keepdims=True) if S.size else np.ones(1)
    rel_tile = (serr / tile_max).max() if S.size else 0.0
    if bf16_state:
        assert np.all(serr <= 2.0 ** -8 * np.abs(ref_state) + 1e-6), \
            f"bf16 state outside the stated tolerance: max {serr.max()}"
        if strict and S.size:
            assert np.all(serr <= bf16_ulp(ref_state) + 2e-6 * tile_max), "bf16 state beyond one ulp"
    else:
        assert np.all(serr <= 1e-4 * np.abs(ref_state) + 1e-6), f"state outside the stated tolerance: max {serr.max()}"
        if strict:
            assert rel_tile <= 2e-6, f"state error {rel_tile} of the tile scale"
    ulps = (err / bf16_ulp(r)).max() if r.size else 0.0
    return Report(float(err.max()) if err.size else 0.0, float(ulps), float(rel_tile),
                  float(serr.max()) if serr.size else 0.0)


def parity(p: ki.Problem, packed: bool | None = None, flags: int = 0, state_dtype=torch.float32) -> Report:
    d = upload(p, state_dtype=state_dtype)
    before = d.state.clone()
    run_gpu(d, packed=packed, flags=flags)
    torch.cuda.synchronize()
    ref_out, ref_state = run_oracle(p, state_bf16=state_dtype == torch.bfloat16)
    rep = compare(d, ref_out, ref_state)
    # every slot no live request owns is bit-for-bit untouched
    untouched = torch.ones(p.num_slots, dtype=torch.bool, device=DEV)
    if len(d.live_slots):
        untouched[torch.from_numpy(d.live_slots).to(DEV)] = False
    assert torch.equal(d.state[untouched], before[untouched]), "a slot outside the call changed"
    return rep

"""Seeded synthetic inputs for recurrent KDA decode.

This module holds random-number generation and the input recipe only.  No
step of the decode itself (decay, delta correction, rank-1 update, readout,
gated normalisation) lives here: the GPU path and the CPU oracle both take the
arrays produced below and nothing else from this file.

Generator.  A counter-based SplitMix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014): draw i of stream s
under seed x is mix64(key(x, s) + (i + 1) * 0x9E3779B97F4A7C15), with mix64 the
SplitMix64 finaliser and key(x, s) = mix64(x * 0x9E3779B97F4A7C15 + s).
Because every draw is a pure function of (seed, stream, index), any subset of
a tensor (say the state of a few pool slots) can be regenerated on its own.
Normals use Box-Muller on two 53-bit uniforms (draws 2i and 2i+1).

Workloads.  The shapes and value distributions mirror the serving shapes the
pages measure.  vLLM PR 57585 (SM90 launch tuning for recurrent KDA), section
"Microbenchmark and earlier serving limits": bf16 q/k/v, fp32 state,
K = V = 128, N in {1, 4, 32}, T in {1, 4}, H in {8, 16}; same page, "Retained
baseline trace attribution": launches at N = 1, 8, 16, 24, 32 over 8 local
heads, N = 32 dominating.  FlashInfer PR 4562 (H12 packed decode across the
SM100 family), description: 12 heads, packed requests, padding rows that the
kernel must skip.  Recipe:

  q, k    bf16, N(0,1) then L2-normalised per (token, head) in double
  v       bf16, N(0,1)
  g       fp32, -softplus(N(0,1)) per key channel (log-decay, already activated)
  beta    fp32, sigmoid(N(0,1)) per (token, value head)
  state   fp32, N(0, 0.05) in every pool slot (0.05 is the standard deviation)
  gate    bf16, N(0,1); norm weight bf16, 1 + N(0, 0.02); eps 1e-6
  scale   1/sqrt(K)

Raw-projection problems (``raw_gates=True``) carry the gate inputs before
activation instead of g and beta (FlashInfer PR 4562, inline review of the
binding: bf16 raw_gate and raw_beta, fp32 A_log and dt_bias):

  raw_gate  bf16, N(0,1) per key channel (the same draws as g's x above)
  raw_beta  bf16, N(0,1) per (token, value head) (the same draws as beta's)
  A_log     fp32, N(0, a_log_std) per value head
  dt_bias   fp32, N(0, dt_bias_std) per (value head, key channel)

The activation itself is the decode's business: this module only draws.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream ids, one per tensor, so tensors do not depend on generation order
STREAM_STATE, STREAM_SLOTS, STREAM_T, STREAM_PAD = 1, 2, 3, 4
STREAM_Q, STREAM_K, STREAM_V, STREAM_G, STREAM_BETA = 5, 6, 7, 8, 9
STREAM_GATE, STREAM_WEIGHT = 10, 11
STREAM_ALOG, STREAM_DTBIAS = 12, 13

SEED_BASE = 0x4B444100  # "KDA\0"


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        z = np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64) * _GAMMA + np.uint64(stream)
        return _mix64(z)[0]


def draws(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """Raw 64-bit draws at counter positions ``idx`` (uint64 array)."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(_key(seed, stream) + (idx + np.uint64(1)) * _GAMMA)


def uniform_open(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """Uniform doubles in (0, 1] from 53-bit draws."""
    d = draws(seed, stream, idx)
    return ((d >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)


def normal(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    """``n`` standard normals (float64), element i uses draws 2(offset+i) and +1."""
    i = np.arange(offset, offset + n, dtype=np.uint64)
    u1 = uniform_open(seed, stream, 2 * i)
    u2 = uniform_open(seed, stream, 2 * i + np.uint64(1))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A seeded permutation of range(n): sort indices by their draw."""
    keys = draws(seed, stream, np.arange(n, dtype=np.uint64))
    return np.argsort(keys, kind="stable").astype(np.int64)


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint16)
    r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_bf16_bits(x) -> np.ndarray:
    """float64 -> float32 (nearest) -> bf16 (nearest even)."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


# ---------------------------------------------------------------- problems
@dataclasses.dataclass
class Problem:
    """One decode call's inputs (host arrays).

    Token-major layouts, contiguous: q, k [tokens, H, K] bf16 bits; v
    [tokens, HV, V] bf16 bits; g [tokens, HV, K] fp32; beta [tokens, HV] fp32;
    gate [tokens, HV, V] bf16 bits or None; norm_weight [V] bf16 bits or None.
    Raw-projection problems have g = beta = None and instead raw_gate
    [tokens, HV, K] and raw_beta [tokens, HV] bf16 bits, A_log [HV] and
    dt_bias [HV, K] fp32.
    Request i owns tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 and pool slot
    slot_idx[i] (-1: inactive padding row).  The state pool is
    [num_slots, HV, K, V] fp32 and is generated on demand (``state_slots``).
    """

    name: str
    seed: int
    N: int
    H: int
    HV: int
    K: int
    V: int
    num_slots: int
    T: Optional[int]          # fixed tokens per request (step call) or None (packed)
    cu_seqlens: np.ndarray    # int32 [N+1]
    slot_idx: np.ndarray      # int32 [N]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: Optional[np.ndarray]
    beta: Optional[np.ndarray]
    gate: Optional[np.ndarray]
    norm_weight: Optional[np.ndarray]
    eps: float
    scale: float
    state_std: float = 0.05
    raw_gate: Optional[np.ndarray] = None
    raw_beta: Optional[np.ndarray] = None
    A_log: Optional[np.ndarray] = None
    dt_bias: Optional[np.ndarray] = None

    @property
    def raw(self) -> bool:
        return self.raw_gate is not None

    @property
    def tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def slot_elems(self) -> int:
        return self.HV * self.K * self.V

    def state_slots(self, slots) -> np.ndarray:
        """fp32 state of the given pool slots, shape [len(slots), HV, K, V]."""
        slots = np.asarray(slots, dtype=np.int64).reshape(-1)
        E = self.slot_elems
        out = np.empty((slots.size, E), dtype=np.float32)
        for j, s in enumerate(slots):
            out[j] = (self.state_std * normal(self.seed, STREAM_STATE, E, offset=int(s) * E)).astype(np.float32)
        return out.reshape(slots.size, self.HV, self.K, self.V)

    def state_pool(self) -> np.ndarray:
        """The whole fp32 pool [num_slots, HV, K, V]."""
        E = self.slot_elems
        flat = (self.state_std * normal(self.seed, STREAM_STATE, self.num_slots * E)).astype(np.float32)
        return flat.reshape(self.num_slots, self.HV, self.K, self.V)

    def live_requests(self) -> np.ndarray:
        s = self.slot_idx
        return np.nonzero((s >= 0) & (s < self.num_slots))[0]


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def make_problem(name: str, seed: int, N: int, H: int, HV: int, K: int, V: int,
                 num_slots: int, T: Optional[int] = None, t_max: int = 4,
                 n_pad: int = 0, norm: bool = False, first_slots: bool = False,
                 eps: float = 1e-6, raw_gates: bool = False, a_log_std: float = 0.5,
                 dt_bias_std: float = 0.5) -> Problem:
    """Draw one problem.  ``T`` fixed -> step call; ``T is None`` -> packed call
    with per-request T uniform on {1..t_max}.  ``n_pad`` requests (at seeded
    random positions) get slot -1.  Live requests get distinct pool slots, the
    first ones (``first_slots``) or a seeded random subset.  ``raw_gates``:
    raw projections for the fused gate activation instead of g and beta."""
    if HV % H:
        raise ValueError("HV must be a multiple of H")
    if T is not None:
        lens = np.full(N, T, dtype=np.int64)
    else:
        d = draws(seed, STREAM_T, np.arange(N, dtype=np.uint64))
        lens = ((d >> np.uint64(11)) % np.uint64(t_max)).astype(np.int64) + 1
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    tokens = int(cu[-1])

    pad = np.zeros(N, dtype=bool)
    if n_pad:
        pad[permutation(seed, STREAM_PAD, N)[:n_pad]] = True
    n_live = int(N - pad.sum())
    if n_live > num_slots:
        raise ValueError("more live requests than pool slots")
    if first_slots:
        live_slots = np.arange(n_live, dtype=np.int64)
    else:
        live_slots = permutation(seed, STREAM_SLOTS, num_slots)[:n_live]
    slot_idx = np.full(N, -1, dtype=np.int64)
    slot_idx[~pad] = live_slots

    q = _unit_rows(normal(seed, STREAM_Q, tokens * H * K).reshape(tokens, H, K))
    k = _unit_rows(normal(seed, STREAM_K, tokens * H * K).reshape(tokens, H, K))
    v = normal(seed, STREAM_V, tokens * HV * V).reshape(tokens, HV, V)
    x = normal(seed, STREAM_G, tokens * HV * K).reshape(tokens, HV, K)
    xb = normal(seed, STREAM_BETA, tokens * HV).reshape(tokens, HV)
    raw = {}
    if raw_gates:
        g = beta = None
        raw = dict(raw_gate=to_bf16_bits(x), raw_beta=to_bf16_bits(xb),
                   A_log=(a_log_std * normal(seed, STREAM_ALOG, HV)).astype(np.float32),
                   dt_bias=(dt_bias_std * normal(seed, STREAM_DTBIAS, HV * K)).astype(np.float32).reshape(HV, K))
    else:
        g = (-(np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0))).astype(np.float32)   # -softplus(x)
        beta = (1.0 / (1.0 + np.exp(-xb))).astype(np.float32)                            # sigmoid(x)
    gate = w = None
    if norm:
        gate = to_bf16_bits(normal(seed, STREAM_GATE, tokens * HV * V).reshape(tokens, HV, V))
        w = to_bf16_bits(1.0 + 0.02 * normal(seed, STREAM_WEIGHT, V))
    return Problem(
        name=name, seed=seed, N=N, H=H, HV=HV, K=K, V=V, num_slots=num_slots, T=T,
        cu_seqlens=cu.astype(np.int32), slot_idx=slot_idx.astype(np.int32),
        q=to_bf16_bits(q), k=to_bf16_bits(k), v=to_bf16_bits(v),
        g=g, beta=beta, gate=gate, norm_weight=w, eps=eps, scale=1.0 / math.sqrt(K), **raw)


# The five serving workloads, named by what they are.
WORKLOADS = {
    # one request, one token, 8 heads; slot 0 of a 4-slot pool
    "n1_t1_h8": dict(cid=0, N=1, H=8, HV=8, num_slots=4, T=1, first_slots=True),
    # the dominant serving shape: 32 requests, one token, 8 heads, 512-slot pool
    "n32_t1_h8": dict(cid=1, N=32, H=8, HV=8, num_slots=512, T=1),
    # four tokens per request recurred in one call, 8 heads (N swept)
    **{f"n{n}_t4_h8": dict(cid=2, N=n, H=8, HV=8, num_slots=512, T=4) for n in (1, 8, 16, 24, 32)},
    # 16 heads with the fused gated RMSNorm epilogue
    "n32_t1_h16_norm": dict(cid=3, N=32, H=16, HV=16, num_slots=512, T=1, norm=True),
    # packed varlen: 256 requests, 12 heads, T_i in {1..4}, 26 padding rows, 2048-slot pool
    "packed_n256_h12": dict(cid=4, N=256, H=12, HV=12, num_slots=2048, T=None, n_pad=26),
    # the dominant shape and the packed batch with the gate activation fused
    # into the decode: raw projections instead of activated g and beta
    "n32_t1_h8_rawgate": dict(cid=1, N=32, H=8, HV=8, num_slots=512, T=1, raw_gates=True),
    "packed_n256_h12_rawgate": dict(cid=4, N=256, H=12, HV=12, num_slots=2048, T=None, n_pad=26, raw_gates=True),
}


def workload(name: str) -> Problem:
    spec = dict(WORKLOADS[name])
    cid = spec.pop("cid")
    seed = SEED_BASE + cid + (spec["N"] if cid == 2 else 0)
    return make_problem(name, seed, K=128, V=128, **spec)

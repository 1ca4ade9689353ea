"""ctypes front end of the CPU oracle for recurrent KDA decode.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here imports the GPU package
and the GPU package never imports this one.

The arithmetic lives in ``kda_oracle.c`` (double precision, sequential); this
file only builds the library with gcc, loads it and marshals numpy arrays.
The recurrence, its step order and the readings of the pages it rests on are
stated at the top of ``kda_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "kda_oracle.c")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]
# KDA_ORACLE_SANITIZE=1 (the test suite's sanitizer tier, in a process that
# preloads the sanitizer runtimes): the oracle is built and loaded with
# AddressSanitizer and UndefinedBehaviorSanitizer, any finding fatal
SANITIZE = os.environ.get("KDA_ORACLE_SANITIZE") == "1"
SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
if SANITIZE:
    CFLAGS = CFLAGS + SANITIZE_FLAGS
LIB = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")

_lib = None


def build() -> str:
    """Compile ``liboracle.so`` with gcc (always recompiles)."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.kda_oracle_decode.restype = ctypes.c_int
    lib.kda_oracle_decode.argtypes = [
        i64, i64, i64, i64, i64, p,
        p, i64, p, i64, p, i64, p, i64, p, i64,
        p, i64, i64, p, ctypes.c_double,
        p, i64, p, ctypes.c_double, p, i64, p, i64,
        p, i64, p, i64, p, p]
    lib.kda_oracle_gate_activation.restype = ctypes.c_int
    lib.kda_oracle_gate_activation.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, p]
    lib.kda_oracle_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_oracle_gated_rmsnorm.argtypes = [i64, i64, p, p, p, ctypes.c_double, p]
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _tok_stride(a: np.ndarray, inner: int) -> int:
    """Token stride in elements of a [tokens, ...] view whose inner dims are dense."""
    item = a.itemsize
    expect = item
    for d in range(a.ndim - 1, 0, -1):
        if a.shape[d] > 1 and a.strides[d] != expect:
            raise ValueError("inner dimensions must be contiguous")
        expect *= a.shape[d]
    if a.shape[0] <= 1:
        return inner
    if a.strides[0] % item or a.strides[0] < 0:
        raise ValueError("token stride must be a non-negative whole number of elements")
    return a.strides[0] // item


def _raw_gate_args(raw_gate, raw_beta, A_log, dt_bias, tokens, HV, K):
    """Validate the raw-projection inputs of the gate activation."""
    if raw_gate.dtype != np.uint16 or raw_beta.dtype != np.uint16:
        raise ValueError("raw_gate and raw_beta are bf16 bits (uint16)")
    if raw_gate.shape != (tokens, HV, K) or raw_beta.shape != (tokens, HV):
        raise ValueError("raw_gate must be [tokens, HV, K] and raw_beta [tokens, HV]")
    A_log = np.ascontiguousarray(A_log, dtype=np.float32)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    if A_log.shape != (HV,) or dt_bias.reshape(-1).shape != (HV * K,):
        raise ValueError("A_log must be [HV] and dt_bias [HV, K]")
    return A_log, dt_bias


def gate_activation(raw_gate, raw_beta, A_log, dt_bias):
    """Step 0 alone: raw_gate uint16 [tokens, HV, K], raw_beta uint16
    [tokens, HV], A_log float32 [HV], dt_bias float32 [HV, K] ->
    (g float64 [tokens, HV, K], beta float64 [tokens, HV])."""
    lib = _load()
    tokens, HV, K = raw_gate.shape
    A_log, dt_bias = _raw_gate_args(raw_gate, raw_beta, A_log, dt_bias, tokens, HV, K)
    g = np.empty((tokens, HV, K), dtype=np.float64)
    beta = np.empty((tokens, HV), dtype=np.float64)
    rc = lib.kda_oracle_gate_activation(
        tokens, HV, K, _ptr(raw_gate), _tok_stride(raw_gate, HV * K), _ptr(raw_beta),
        _tok_stride(raw_beta, HV), _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(beta))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return g, beta


def decode_packed(q, k, v, g, beta, state, slot_idx, cu_seqlens, scale, *,
                  gate=None, norm_weight=None, eps=1e-6, out=None, inter_state=None,
                  raw_gate=None, raw_beta=None, A_log=None, dt_bias=None):
    """Run the oracle over a packed batch.

    q, k: uint16 bf16 bits [tokens, H, K]; v: uint16 [tokens, HV, V];
    g: float32 [tokens, HV, K]; beta: float32 [tokens, HV];
    state: float64 [num_slots, HV, K, V], updated in place;
    slot_idx: int32 [N]; cu_seqlens: int32 [N+1];
    gate: uint16 [tokens, HV, V] or None; norm_weight: uint16 [V].
    Returns out, float64 [tokens, HV, V] (NaN where a request was skipped,
    unless ``out`` is given, which is then left untouched there).
    inter_state: None, or float64 [tokens, HV, K, V] that receives the state
    after each token of each live request.
    raw_gate (uint16 [tokens, HV, K]), raw_beta (uint16 [tokens, HV]), A_log
    (float32 [HV]), dt_bias (float32 [HV, K]): all four or none; with them
    the log-decay and beta are activated from these and g, beta may be None.
    """
    lib = _load()
    tokens, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise ValueError("state must be a C-contiguous float64 pool")
    num_slots = state.shape[0]
    slot_stride = int(np.prod(state.shape[1:]))
    if state.shape[1:] != (HV, K, V):
        raise ValueError("state pool must be [num_slots, HV, K, V]")
    slot_idx = np.ascontiguousarray(slot_idx, dtype=np.int32)
    cu_seqlens = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = slot_idx.shape[0]
    if cu_seqlens.shape[0] != N + 1 or cu_seqlens[-1] > tokens or cu_seqlens[0] < 0:
        raise ValueError("cu_seqlens must be [N+1] within the token range")
    if out is None:
        out = np.full((tokens, HV, V), np.nan, dtype=np.float64)
    if out.dtype != np.float64 or out.shape != (tokens, HV, V) or not out.flags.c_contiguous:
        raise ValueError("out must be C-contiguous float64 [tokens, HV, V]")
    if (gate is None) != (norm_weight is None):
        raise ValueError("gate and norm_weight go together")
    raw = raw_gate is not None
    if raw != (raw_beta is not None) or raw != (A_log is not None) or raw != (dt_bias is not None):
        raise ValueError("raw_gate, raw_beta, A_log and dt_bias go together")
    if raw:
        A_log, dt_bias = _raw_gate_args(raw_gate, raw_beta, A_log, dt_bias, tokens, HV, K)
        g_args = (None, HV * K, None, HV)
        raw_args = (_ptr(raw_gate), _tok_stride(raw_gate, HV * K), _ptr(raw_beta), _tok_stride(raw_beta, HV),
                    _ptr(A_log), _ptr(dt_bias))
    else:
        if g is None or beta is None or g.dtype != np.float32 or beta.dtype != np.float32:
            raise ValueError("g and beta must be float32 arrays")
        g_args = (_ptr(g), _tok_stride(g, HV * K), _ptr(beta), _tok_stride(beta, HV))
        raw_args = (None, 0, None, 0, None, None)
    for a, dt in ((q, np.uint16), (k, np.uint16), (v, np.uint16)):
        if a.dtype != dt:
            raise ValueError(f"dtype {a.dtype}, expected {dt}")
    if gate is not None:
        norm_weight = np.ascontiguousarray(norm_weight, dtype=np.uint16)
    if inter_state is not None and (inter_state.dtype != np.float64 or not inter_state.flags.c_contiguous
                                    or inter_state.shape != (tokens, HV, K, V)):
        raise ValueError("inter_state must be C-contiguous float64 [tokens, HV, K, V]")
    rc = lib.kda_oracle_decode(
        N, H, HV, K, V, _ptr(cu_seqlens),
        _ptr(q), _tok_stride(q, H * K), _ptr(k), _tok_stride(k, H * K),
        _ptr(v), _tok_stride(v, HV * V), *g_args,
        _ptr(state), num_slots, slot_stride, _ptr(slot_idx), float(scale),
        _ptr(gate), 0 if gate is None else _tok_stride(gate, HV * V),
        _ptr(norm_weight), float(eps), _ptr(out), HV * V,
        _ptr(inter_state), HV * K * V, *raw_args)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out


def decode_step(q, k, v, g, beta, state, slot_idx, T, scale, **kw):
    """Every request has exactly ``T`` tokens, request-major ([N*T, ...])."""
    N = int(np.asarray(slot_idx).shape[0])
    cu = (np.arange(N + 1, dtype=np.int64) * int(T)).astype(np.int32)
    return decode_packed(q, k, v, g, beta, state, slot_idx, cu, scale, **kw)


def gated_rmsnorm(x, gate, norm_weight, eps):
    """x, gate: uint16 bf16 bits [rows, V]; norm_weight: uint16 [V] -> float64 [rows, V]."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    gate = np.ascontiguousarray(gate, dtype=np.uint16)
    norm_weight = np.ascontiguousarray(norm_weight, dtype=np.uint16)
    rows, V = x.shape
    if gate.shape != x.shape or norm_weight.shape != (V,):
        raise ValueError("shape mismatch")
    y = np.empty((rows, V), dtype=np.float64)
    rc = lib.kda_oracle_gated_rmsnorm(rows, V, _ptr(x), _ptr(gate), _ptr(norm_weight), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return y

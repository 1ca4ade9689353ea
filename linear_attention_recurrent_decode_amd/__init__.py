"""Recurrent KDA decode on MI355X (gfx950): Python binding of libkda.so.

This module only marshals arguments: it turns torch tensors into the plain
pointers, sizes and strides of the C ABI in ``include/kda.h`` and raises on
an error status.  Every step of the decode runs in the HIP kernels of
``csrc/kda_decode.hip``.  There is no fallback: without the built library
every call raises.

torch supplies device memory and the current stream.  It is imported before
the library is loaded so that libkda.so binds to the HIP runtime torch
already loaded.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "KdaError", "KdaDecodeArgs", "library", "library_path",
    "kda_decode_step", "kda_decode_packed", "kda_gated_rmsnorm",
    "kda_decode_plan", "KDA_PLAN_NORM", "KDA_PLAN_STATE_BF16", "KDA_PLAN_PACKED", "KDA_PLAN_LAYOUT",
    "KDA_PLAN_RAW_GATE",
    "KDA_LAYOUT_WIDE", "KDA_LAYOUT_QUARTER", "KDA_LAYOUT_SPLIT", "kda_status_string",
    "decode_args", "KDA_FLAG_VTILE", "KDA_FLAG_KERNEL", "KDA_FLAG_ORDER", "KDA_FLAG_STATE_BF16",
    "KDA_FLAG_VALIDATE", "KDA_DEVICE_STATUS",
    "KDA_KERNEL_WIDE", "KDA_KERNEL_QUARTER2", "KDA_KERNEL_QUARTER4", "KDA_KERNEL_QUARTER8", "KDA_KERNEL_SPLIT",
    "KDA_ORDER_TILE_FIRST", "KDA_ORDER_INPUTS_FIRST", "KDA_FLAG_PLACEMENT", "KDA_PLACEMENT_HEAD_XCD",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libkda.so")
# the benchmark's tile-stream reference (include/kda_stream.h); not the decode path
stream_library_path = os.path.join(_PKG, "libkda_stream.so")

KDA_STATUS = {
    0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_ALIGN",
    4: "KDA_ERR_ALIAS", 5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_DEVICE", 7: "KDA_ERR_LAUNCH",
}
KDA_FLAG_STATE_BF16 = 1 << 0
KDA_FLAG_VALIDATE = 1 << 1
KDA_DEVICE_STATUS = {0: "KDA_DEVICE_OK", 1: "KDA_DEVICE_ERR_SLOT_RANGE", 2: "KDA_DEVICE_ERR_SLOT_DUP",
                     3: "KDA_DEVICE_ERR_CU_SEQLENS"}
KDA_FLAG_VTILE_SHIFT = 8
KDA_FLAG_KERNEL_SHIFT = 12
KDA_FLAG_ORDER_SHIFT = 16
KDA_FLAG_PLACEMENT_SHIFT = 18
KDA_KERNEL_WIDE, KDA_KERNEL_QUARTER2, KDA_KERNEL_QUARTER4, KDA_KERNEL_QUARTER8 = 1, 2, 3, 4
KDA_KERNEL_SPLIT = 5
KDA_ORDER_TILE_FIRST, KDA_ORDER_INPUTS_FIRST = 1, 2
KDA_PLACEMENT_HEAD_XCD = 1


def KDA_FLAG_VTILE(width: int) -> int:
    """Flag bits forcing a value-tile width of 32, 64 or 128 columns."""
    code = {32: 1, 64: 2, 128: 3}[width]
    return code << KDA_FLAG_VTILE_SHIFT


def KDA_FLAG_KERNEL(code: int) -> int:
    """Flag bits forcing a kernel (a KDA_KERNEL_* code)."""
    return (int(code) & 15) << KDA_FLAG_KERNEL_SHIFT


def KDA_FLAG_ORDER(code: int) -> int:
    """Flag bits forcing a load order (KDA_ORDER_TILE_FIRST or KDA_ORDER_INPUTS_FIRST)."""
    return (int(code) & 3) << KDA_FLAG_ORDER_SHIFT


def KDA_FLAG_PLACEMENT(code: int) -> int:
    """Flag bits forcing a workgroup placement (KDA_PLACEMENT_HEAD_XCD)."""
    return (int(code) & 3) << KDA_FLAG_PLACEMENT_SHIFT


class KdaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        self.name = KDA_STATUS.get(status, str(status))
        super().__init__(f"{what}: {self.name} ({kda_status_string(status)})")


class KdaDecodeArgs(ctypes.Structure):
    """Mirror of ``kda_decode_args`` in include/kda.h."""
    _fields_ = [
        ("N", ctypes.c_int32), ("H", ctypes.c_int32), ("HV", ctypes.c_int32),
        ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_stride", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("k_stride", ctypes.c_int64),
        ("v", ctypes.c_void_p), ("v_stride", ctypes.c_int64),
        ("g", ctypes.c_void_p), ("g_stride", ctypes.c_int64),
        ("beta", ctypes.c_void_p), ("beta_stride", ctypes.c_int64),
        ("state", ctypes.c_void_p), ("num_slots", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
        ("slot_idx", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("out_stride", ctypes.c_int64),
        ("gate", ctypes.c_void_p), ("gate_stride", ctypes.c_int64),
        ("norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("device_status", ctypes.c_void_p),
        ("inter_state", ctypes.c_void_p), ("inter_stride", ctypes.c_int64),
        ("raw_gate", ctypes.c_void_p), ("raw_gate_stride", ctypes.c_int64),
        ("raw_beta", ctypes.c_void_p), ("raw_beta_stride", ctypes.c_int64),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
    ]


_lib = None


def _open(path: str) -> ctypes.CDLL:
    """Load a build of the C ABI from ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(KdaDecodeArgs)
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [P, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p]
    lib.kda_decode_packed.restype = ctypes.c_int
    lib.kda_decode_packed.argtypes = [P, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    lib.kda_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_gated_rmsnorm.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
    lib.kda_decode_plan.restype = ctypes.c_int32
    lib.kda_decode_plan.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    return lib


def library() -> ctypes.CDLL:
    """Load libkda.so (built in place by ``build.py``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is not built: run linear_attention_recurrent_decode_amd.build.build()")
    _lib = _open(library_path)
    return _lib


_stream_lib = None


def stream_library() -> ctypes.CDLL:
    """Load libkda_stream.so, the tile-stream reference the benchmark times
    beside the decode (it moves a call's state bytes in place and computes
    nothing); raise if it is missing."""
    global _stream_lib
    if _stream_lib is not None:
        return _stream_lib
    if not os.path.exists(stream_library_path):
        raise RuntimeError(f"{stream_library_path} is not built: run linear_attention_recurrent_decode_amd.build.build()")
    lib = ctypes.CDLL(stream_library_path)
    lib.kda_stream_tiles.restype = ctypes.c_int
    lib.kda_stream_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    _stream_lib = lib
    return lib


def kda_status_string(status: int) -> str:
    return library().kda_status_string(int(status)).decode()


KDA_PLAN_NORM = 1
KDA_PLAN_STATE_BF16 = 2
KDA_PLAN_PACKED = 4
KDA_PLAN_LAYOUT = 8
KDA_PLAN_RAW_GATE = 16
KDA_LAYOUT_WIDE = 0
KDA_LAYOUT_QUARTER = 1
KDA_LAYOUT_SPLIT = 2


def kda_decode_plan(units: int, T: int = 1, has_norm: bool = False, bf16_state: bool = False,
                    packed: bool = False, layout: bool = False, raw_gate: bool = False) -> int:
    """Columns per workgroup the library picks, or with layout=True its lane
    layout, a KDA_LAYOUT_* value (include/kda.h, kda_decode_plan)."""
    options = ((KDA_PLAN_NORM if has_norm else 0) | (KDA_PLAN_STATE_BF16 if bf16_state else 0)
               | (KDA_PLAN_PACKED if packed else 0) | (KDA_PLAN_LAYOUT if layout else 0)
               | (KDA_PLAN_RAW_GATE if raw_gate else 0))
    return int(library().kda_decode_plan(int(units), int(T), options))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _current_device() -> torch.device:
    """The GPU every tensor of a call must live on: torch's current device."""
    return torch.device("cuda", torch.cuda.current_device())


def _on_device(t: torch.Tensor, name: str, device: Optional[torch.device]):
    """Raise unless ``t`` lives on ``device`` (None: torch's current GPU).  A
    host tensor's data_ptr() is a host address; handed to a kernel it would
    fault the GPU, so it is refused here, before any library call."""
    if device is None:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
        device = _current_device()
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, device: Optional[torch.device] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    _on_device(t, name, device)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    # inner dimensions dense; the leading (token / slot) dimension may be strided
    expect = 1
    for d in range(ndim - 1, 0, -1):
        if t.shape[d] > 1 and t.stride(d) != expect:
            raise ValueError(f"{name}: inner dimensions must be contiguous")
        expect *= t.shape[d]


def _lead_stride(t: torch.Tensor) -> int:
    inner = 1
    for d in t.shape[1:]:
        inner *= d
    return t.stride(0) if t.shape[0] > 1 else inner


def _state_flag(state: torch.Tensor, flags: int) -> int:
    """The state pool's dtype selects the bf16-state flag."""
    flags = int(flags) & ~KDA_FLAG_STATE_BF16
    return flags | (KDA_FLAG_STATE_BF16 if state.dtype == torch.bfloat16 else 0)


def decode_args(q, k, v, g, beta, state, slot_idx, out, scale, gate=None, norm_weight=None,
                eps: float = 1e-6, device_status=None, inter_state=None, raw_gate=None, raw_beta=None,
                A_log=None, dt_bias=None) -> KdaDecodeArgs:
    """Marshal tensors into a ``kda_decode_args`` struct (no validation of
    values; the library validates sizes, alignment and overlap).  The gate
    inputs come either activated (g, beta) or raw (raw_gate, raw_beta, A_log,
    dt_bias, with g = beta = None): the kernel then activates them.  Every
    tensor must live on torch's current GPU (ValueError otherwise)."""
    return _marshal_args(q, k, v, g, beta, state, slot_idx, out, scale, gate, norm_weight, eps, device_status,
                         inter_state, raw_gate, raw_beta, A_log, dt_bias, device=None)


def _marshal_args(q, k, v, g, beta, state, slot_idx, out, scale, gate, norm_weight, eps, device_status,
                  inter_state, raw_gate, raw_beta, A_log, dt_bias, *, device) -> KdaDecodeArgs:
    """decode_args with the device every tensor must be on made explicit
    (None: torch's current GPU, the only value the library calls use)."""
    if device is None:
        _on_device(q, "q", None)   # a host tensor is refused before any device query
        device = _current_device()
    _check(q, "q", torch.bfloat16, 3, device)
    _check(k, "k", torch.bfloat16, 3, device)
    _check(v, "v", torch.bfloat16, 3, device)
    _check(state, "state", state.dtype if state.dtype in (torch.float32, torch.bfloat16) else torch.float32, 4, device)
    _check(slot_idx, "slot_idx", torch.int32, 1, device)
    _check(out, "out", torch.bfloat16, 3, device)
    tokens, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != tokens or out.shape != (tokens, HV, V) or state.shape[1:] != (HV, K, V):
        raise ValueError("inconsistent shapes")
    raw = raw_gate is not None
    if any((t is not None) != raw for t in (raw_beta, A_log, dt_bias)) or (raw and (g is not None or beta is not None)):
        raise ValueError("give either g and beta, or raw_gate, raw_beta, A_log and dt_bias")
    a = KdaDecodeArgs()
    a.N, a.H, a.HV, a.K, a.V = slot_idx.shape[0], H, HV, K, V
    a.scale = float(scale)
    a.q, a.q_stride = q.data_ptr(), _lead_stride(q)
    a.k, a.k_stride = k.data_ptr(), _lead_stride(k)
    a.v, a.v_stride = v.data_ptr(), _lead_stride(v)
    if raw:
        _check(raw_gate, "raw_gate", torch.bfloat16, 3, device)
        _check(raw_beta, "raw_beta", torch.bfloat16, 2, device)
        _check(A_log, "A_log", torch.float32, 1, device)
        _check(dt_bias, "dt_bias", torch.float32, 2, device)
        if raw_gate.shape != (tokens, HV, K) or raw_beta.shape != (tokens, HV) or A_log.shape != (HV,) or \
                dt_bias.shape != (HV, K):
            raise ValueError("inconsistent raw gate shapes")
        a.raw_gate, a.raw_gate_stride = raw_gate.data_ptr(), _lead_stride(raw_gate)
        a.raw_beta, a.raw_beta_stride = raw_beta.data_ptr(), _lead_stride(raw_beta)
        a.A_log, a.dt_bias = A_log.data_ptr(), dt_bias.data_ptr()
    else:
        _check(g, "g", torch.float32, 3, device)
        _check(beta, "beta", torch.float32, 2, device)
        if g.shape != (tokens, HV, K) or beta.shape != (tokens, HV):
            raise ValueError("inconsistent shapes")
        a.g, a.g_stride = g.data_ptr(), _lead_stride(g)
        a.beta, a.beta_stride = beta.data_ptr(), _lead_stride(beta)
    a.state, a.num_slots, a.slot_stride = state.data_ptr(), state.shape[0], _lead_stride(state)
    a.slot_idx = slot_idx.data_ptr()
    a.out, a.out_stride = out.data_ptr(), _lead_stride(out)
    if (gate is None) != (norm_weight is None):
        raise ValueError("gate and norm_weight go together")
    if gate is not None:
        _check(gate, "gate", torch.bfloat16, 3, device)
        _check(norm_weight, "norm_weight", torch.bfloat16, 1, device)
        if gate.shape != out.shape or norm_weight.shape != (V,):
            raise ValueError("inconsistent gate / norm_weight shapes")
        a.gate, a.gate_stride = gate.data_ptr(), _lead_stride(gate)
        a.norm_weight = norm_weight.data_ptr()
    a.norm_eps = float(eps)
    if device_status is not None:
        _check(device_status, "device_status", torch.int32, 1, device)
        a.device_status = device_status.data_ptr()
    if inter_state is not None:
        _check(inter_state, "inter_state", state.dtype, 4, device)
        if inter_state.shape != (tokens, HV, K, V):
            raise ValueError("inter_state must be [tokens, HV, K, V]")
        a.inter_state, a.inter_stride = inter_state.data_ptr(), _lead_stride(inter_state)
    return a


def kda_decode_step(q, k, v, g, beta, state, slot_idx, out, *, T: int, scale: float,
                    gate=None, norm_weight=None, eps: float = 1e-6, flags: int = 0, stream=None,
                    device_status=None, inter_state=None, raw_gate=None, raw_beta=None, A_log=None,
                    dt_bias=None):
    """Decode T tokens for each of N requests (tokens request-major, N*T rows);
    updates ``state`` in place and writes ``out`` for live requests.  With
    ``device_status`` (an int32 device tensor of one element) the device
    metadata is validated first, all or nothing (KDA_FLAG_VALIDATE).  With
    ``inter_state`` ([tokens, HV, K, V], the pool's dtype) the state after
    every token is written too (speculative decoding).  With ``raw_gate``
    (bf16 [tokens, HV, K]), ``raw_beta`` (bf16 [tokens, HV]), ``A_log`` (fp32
    [HV]) and ``dt_bias`` (fp32 [HV, K]) instead of g and beta (both None)
    the kernel activates the gates itself."""
    a = decode_args(q, k, v, g, beta, state, slot_idx, out, scale, gate, norm_weight, eps, device_status,
                    inter_state, raw_gate, raw_beta, A_log, dt_bias)
    if device_status is not None:
        flags = int(flags) | KDA_FLAG_VALIDATE
    if q.shape[0] != a.N * int(T):
        raise ValueError("step call needs N*T token rows")
    flags = _state_flag(state, flags)
    st = library().kda_decode_step(ctypes.byref(a), int(T), int(flags), _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_decode_step")
    return out


def kda_decode_packed(q, k, v, g, beta, state, slot_idx, cu_seqlens, out, *, scale: float,
                      gate=None, norm_weight=None, eps: float = 1e-6, flags: int = 0, stream=None,
                      device_status=None, inter_state=None, raw_gate=None, raw_beta=None, A_log=None,
                      dt_bias=None):
    """Packed variable-length decode: request n owns token rows
    cu_seqlens[n] .. cu_seqlens[n+1]-1.  ``device_status``, ``inter_state``
    and the raw gate inputs as for kda_decode_step."""
    a = decode_args(q, k, v, g, beta, state, slot_idx, out, scale, gate, norm_weight, eps, device_status,
                    inter_state, raw_gate, raw_beta, A_log, dt_bias)
    if device_status is not None:
        flags = int(flags) | KDA_FLAG_VALIDATE
    _check(cu_seqlens, "cu_seqlens", torch.int32, 1, q.device)
    if cu_seqlens.shape[0] != a.N + 1:
        raise ValueError("cu_seqlens must hold N+1 entries")
    flags = _state_flag(state, flags)
    st = library().kda_decode_packed(ctypes.byref(a), cu_seqlens.data_ptr(), q.shape[0], int(flags), _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_decode_packed")
    return out


def kda_gated_rmsnorm(x, gate, weight, y, eps: float = 1e-6, stream=None):
    """y = x / sqrt(mean(x^2) + eps) * weight * silu(gate) over the last dim."""
    _on_device(x, "x", None)
    device = _current_device()
    for t, n in ((x, "x"), (gate, "gate"), (y, "y"), (weight, "weight")):
        _on_device(t, n, device)
    for t, n in ((x, "x"), (gate, "gate"), (y, "y")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous bf16 tensor")
    if weight.dtype != torch.bfloat16 or weight.dim() != 1 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous bf16 vector")
    V = x.shape[-1]
    if gate.shape != x.shape or y.shape != x.shape or weight.shape[0] != V:
        raise ValueError("shape mismatch")
    rows = x.numel() // V if V else 0
    st = library().kda_gated_rmsnorm(x.data_ptr(), gate.data_ptr(), weight.data_ptr(), y.data_ptr(),
                                     rows, V, float(eps), _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_gated_rmsnorm")
    return y

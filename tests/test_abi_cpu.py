"""Host-side checks of the C ABI: the library loads, exports what kda.h
declares, the ctypes struct matches the C layout, and every validation path
returns its status before any device work.  The pointers used here are fake
addresses: each call below is rejected by host validation, so nothing is
dereferenced and no kernel is launched.  On a machine with a GPU the whole
module is skipped, so that a call that wrongly passed validation could never
reach a kernel with fake pointers."""
import ctypes
import os
import re
import subprocess

import pytest

import torch

import linear_attention_recurrent_decode_amd as kda

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake device pointers are only used where no GPU exists")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)) - {"kda_decode_args"})


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert names == ["kda_decode_packed", "kda_decode_plan", "kda_decode_step",
                     "kda_gated_rmsnorm", "kda_status_string"]
    lib = kda.library()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kda.library_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)", out))
    assert set(names) <= exported


def test_stream_reference_exports_and_host_checks():
    """The benchmark's tile-stream reference (include/kda_stream.h): the
    library exports what the header declares, and every argument check
    answers before any launch (fake pointers, never dereferenced)."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kda_stream.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))
    assert names == ["kda_stream_tiles"]
    out = subprocess.run(["nm", "-D", "--defined-only", kda.stream_library_path], capture_output=True,
                         text=True).stdout
    assert set(names) <= set(re.findall(r"\bT (kda_\w+)", out))
    lib = kda.stream_library()
    st, idx, tile = 0x10000, 0x20000, 128 * 128
    assert lib.kda_stream_tiles(None, 4, 8, 8 * tile, idx, 2, 8, None) == 1          # KDA_ERR_NULL
    assert lib.kda_stream_tiles(st, 4, 8, 8 * tile, None, 2, 8, None) == 1
    assert lib.kda_stream_tiles(st, 3, 8, 8 * tile, idx, 2, 8, None) == 2            # KDA_ERR_SHAPE
    assert lib.kda_stream_tiles(st, 4, 8, 8 * tile - 1, idx, 2, 8, None) == 2
    assert lib.kda_stream_tiles(st, 4, 8, 8 * tile, idx, 65536, 8, None) == 2
    assert lib.kda_stream_tiles(st, 4, 8, 8 * tile, idx, -1, 8, None) == 2
    assert lib.kda_stream_tiles(st, 4, 8, 8 * tile, idx, 2, 0, None) == 2
    assert lib.kda_stream_tiles(st + 8, 4, 8, 8 * tile, idx, 2, 8, None) == 3        # KDA_ERR_ALIGN
    assert lib.kda_stream_tiles(st, 2, 8, 8 * tile + 1, idx, 2, 8, None) == 3
    assert lib.kda_stream_tiles(st, 4, 8, 8 * tile, idx + 2, 2, 8, None) == 3
    assert lib.kda_stream_tiles(st, 4, 8, 8 * tile, idx, 0, 8, None) == 0            # nothing to do


def test_struct_layout_matches_c(tmp_path):
    fields = [f[0] for f in kda.KdaDecodeArgs._fields_]
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kda.h"', 'int main(void) {',
             '  printf("size %zu\\n", sizeof(kda_decode_args));']
    for f in fields:
        lines.append(f'  printf("{f} %zu\\n", offsetof(kda_decode_args, {f}));')
    lines.append("  return 0; }")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), "-o", str(exe), str(src)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(kda.KdaDecodeArgs)
    for f in fields:
        assert int(got[f]) == getattr(kda.KdaDecodeArgs, f).offset, f


def test_status_strings_and_plan():
    for code in range(8):
        assert kda.kda_status_string(code)
    assert kda.kda_status_string(99) == "unknown status"
    for units in (1, 8, 64, 127, 128, 255, 256, 3072, 1 << 20):
        for T in (1, 2, 4):
            assert kda.kda_decode_plan(units, T, False) in (32, 64, 128)
            assert kda.kda_decode_plan(units, T, True) == 128
    # the launch table of fp32 step calls without the norm: with one token,
    # split-key 16-column waves (32 columns) up to 128 tiles, 32-column waves
    # (32 or 64 columns) to 256, four 16-column waves (64 columns) to 384,
    # eight (128 columns) beyond;
    # with two or more tokens split-key waves up to 320 tiles, four
    # 16-column waves (64 columns) to 576 (512 with
    # two tokens), 32-column waves to 768 (64 columns with two tokens, else
    # 128), four 16-column waves to 1536, eight beyond
    W, Q, S = kda.KDA_LAYOUT_WIDE, kda.KDA_LAYOUT_QUARTER, kda.KDA_LAYOUT_SPLIT
    expect = {(1, 1): (32, S), (8, 1): (32, S), (64, 1): (32, S), (128, 1): (32, S), (129, 1): (32, W),
              (192, 1): (32, W), (255, 1): (32, W), (256, 1): (64, W), (257, 1): (64, Q), (384, 1): (64, Q),
              (385, 1): (128, Q),
              (512, 1): (128, Q), (1024, 1): (128, Q),
              (128, 2): (32, S), (256, 2): (32, S), (320, 2): (32, S), (321, 2): (64, Q), (512, 2): (64, Q),
              (513, 2): (64, W), (576, 2): (64, W), (768, 2): (64, W), (769, 2): (64, Q), (1536, 2): (64, Q),
              (1537, 2): (128, Q), (4096, 2): (128, Q),
              (192, 3): (32, S), (320, 3): (32, S), (321, 3): (64, Q), (576, 3): (64, Q), (577, 3): (128, W),
              (768, 3): (128, W), (769, 3): (64, Q),
              (8, 4): (32, S), (256, 4): (32, S), (320, 4): (32, S), (321, 4): (64, Q), (512, 4): (64, Q), (576, 4): (64, Q),
              (577, 4): (128, W), (768, 4): (128, W), (769, 4): (64, Q), (1536, 4): (64, Q), (1537, 4): (128, Q),
              (384, 9): (64, Q), (192, 9): (32, S), (320, 9): (32, S), (321, 9): (64, Q), (700, 9): (128, W)}
    for (units, T), (width, layout) in expect.items():
        assert kda.kda_decode_plan(units, T, False) == width, (units, T)
        assert kda.kda_decode_plan(units, T, False, layout=True) == layout, (units, T)
    # the fused gate activation: one-token calls take two 16-column waves
    # (32 columns) up to 64 tiles instead of the split-key waves; the rest of
    # the table is the same
    raw = {(1, 1): (32, Q), (64, 1): (32, Q), (65, 1): (32, W), (128, 1): (32, W), (256, 1): (64, W),
           (300, 1): (64, Q), (384, 1): (64, Q),
           (385, 1): (128, Q), (512, 1): (128, Q), (8, 4): (32, S), (192, 2): (32, S), (300, 4): (32, S), (321, 4): (64, Q)}
    for (units, T), (width, layout) in raw.items():
        assert kda.kda_decode_plan(units, T, raw_gate=True) == width, (units, T)
        assert kda.kda_decode_plan(units, T, raw_gate=True, layout=True) == layout, (units, T)
    # packed fp32 calls: four 16-column waves up to 1024 tiles, eight beyond
    for units, width in ((8, 64), (192, 64), (1024, 64), (1025, 128), (3072, 128)):
        for r in (False, True):
            assert kda.kda_decode_plan(units, 4, packed=True, raw_gate=r) == width
            assert kda.kda_decode_plan(units, 4, packed=True, layout=True, raw_gate=r) == Q
    # bf16 pool without the norm: split-key waves for calls of two or more
    # tokens up to 32 tiles and for one-token calls with activated gates up
    # to 24 tiles, else four 16-column waves (64 columns); with the norm eight
    for units in (1, 8, 24, 25, 32, 33, 256, 511, 512, 3072):
        for T in (1, 2, 4):
            small = units <= 32 and T >= 2 or units <= 24 and T == 1
            assert kda.kda_decode_plan(units, T, bf16_state=True) == (32 if small else 64)
            assert kda.kda_decode_plan(units, T, bf16_state=True, layout=True) == (S if small else Q)
            small_raw = units <= 32 and T >= 2
            assert kda.kda_decode_plan(units, T, bf16_state=True, raw_gate=True, layout=True) == (S if small_raw else Q)
            assert kda.kda_decode_plan(units, T, bf16_state=True, packed=True) == 64
            assert kda.kda_decode_plan(units, T, bf16_state=True, packed=True, layout=True) == Q
            assert kda.kda_decode_plan(units, T, True, bf16_state=True) == 128
            assert kda.kda_decode_plan(units, T, True, bf16_state=True, layout=True) == Q
    # the norm with an fp32 pool: eight 16-column waves for step calls of two
    # or more tokens up to 512 tiles and for one-token calls from 512, else
    # 32-column waves of 128 columns
    for (units, T), layout in {(8, 1): W, (511, 1): W, (512, 1): Q, (2048, 1): Q, (8, 2): Q, (512, 4): Q,
                               (513, 4): W}.items():
        assert kda.kda_decode_plan(units, T, True, layout=True) == layout, (units, T)
    assert kda.kda_decode_plan(8, 4, True, packed=True, layout=True) == W


BASE = 0x7F0000000000


def _valid_args(N=4, H=2, HV=4, T=1):
    """Fake, well-formed device addresses: disjoint 64 MiB regions."""
    a = kda.KdaDecodeArgs()
    a.N, a.H, a.HV, a.K, a.V, a.scale = N, H, HV, 128, 128, 0.088
    region = iter(range(BASE, BASE + 64 * (1 << 26), 1 << 26))
    a.q, a.q_stride = next(region), H * 128
    a.k, a.k_stride = next(region), H * 128
    a.v, a.v_stride = next(region), HV * 128
    a.g, a.g_stride = next(region), HV * 128
    a.beta, a.beta_stride = next(region), HV
    a.state, a.num_slots, a.slot_stride = next(region), 8, HV * 128 * 128
    a.slot_idx = next(region)
    a.out, a.out_stride = next(region), HV * 128
    a.gate, a.gate_stride, a.norm_weight, a.norm_eps = 0, 0, 0, 1e-6
    return a, next(region)


def _step(a, T=1, flags=0):
    return kda.library().kda_decode_step(ctypes.byref(a), T, flags, None)


def _packed(a, cu, tokens, flags=0):
    return kda.library().kda_decode_packed(ctypes.byref(a), cu, tokens, flags, None)


NULL, SHAPE, ALIGN, ALIAS, UNSUP, DEVICE = 1, 2, 3, 4, 5, 6


def test_null_pointers():
    assert kda.library().kda_decode_step(None, 1, 0, None) == NULL
    for f in ("q", "k", "v", "g", "beta", "state", "slot_idx", "out"):
        a, _ = _valid_args()
        setattr(a, f, 0)
        assert _step(a) == NULL, f
    a, cu = _valid_args()
    assert _packed(a, None, 4) == NULL
    a, _ = _valid_args()
    a.gate, a.gate_stride = BASE + 40 * (1 << 26), 4 * 128
    assert _step(a) == NULL                      # gate without weight


def test_shapes():
    for field, value in (("K", 64), ("V", 256), ("H", 3), ("HV", 0), ("HV", 65536), ("N", -1), ("num_slots", -1),
                         ("slot_stride", 4 * 128 * 128 - 4), ("q_stride", 128), ("out_stride", 4),
                         ("beta_stride", 3), ("norm_eps", -1.0), ("norm_eps", float("nan"))):
        a, _ = _valid_args()
        setattr(a, field, value)
        assert _step(a) == SHAPE, field
    a, _ = _valid_args()
    assert _step(a, T=0) == SHAPE


def test_alignment():
    for field, value in (("q", BASE + 8), ("k", BASE + (1 << 26) + 2), ("v", BASE + 2 * (1 << 26) + 4),
                         ("g", BASE + 3 * (1 << 26) + 8), ("state", BASE + 5 * (1 << 26) + 4),
                         ("out", BASE + 7 * (1 << 26) + 2)):
        a, _ = _valid_args()
        setattr(a, field, value)
        assert _step(a) == ALIGN, field
    for field, value in (("q_stride", 2 * 128 + 4), ("v_stride", 4 * 128 + 2), ("g_stride", 4 * 128 + 2),
                         ("slot_stride", 4 * 128 * 128 + 2), ("out_stride", 4 * 128 + 2)):
        a, _ = _valid_args()
        setattr(a, field, value)
        assert _step(a) == ALIGN, field


def test_bf16_state_flag():
    a, _ = _valid_args()
    a.state += 8                                   # 8-byte aligned: enough for bf16 rows only
    assert _step(a) == ALIGN
    assert _step(a, flags=kda.KDA_FLAG_STATE_BF16) == DEVICE
    a, _ = _valid_args()
    # a bf16 pool is half as long: out may start right after it
    a.out = a.state + 8 * 4 * 128 * 128 * 2
    assert _step(a) == ALIAS
    assert _step(a, flags=kda.KDA_FLAG_STATE_BF16) == DEVICE


def test_validate_flag_needs_a_status_word():
    V = kda.KDA_FLAG_VALIDATE
    a, _ = _valid_args()
    assert _step(a, flags=V) == NULL
    a, spare = _valid_args()
    a.device_status = spare + 2
    assert _step(a, flags=V) == ALIGN
    a, _ = _valid_args()
    a.device_status = a.slot_idx + 4                 # inside the slot indices
    assert _step(a, flags=V) == ALIAS
    a, _ = _valid_args()
    a.device_status = a.state + 1024                 # inside the pool
    assert _step(a, flags=V) == ALIAS
    a, spare = _valid_args()
    a.device_status = spare
    assert _step(a, flags=V) == DEVICE
    a, _ = _valid_args()
    a.device_status = a.q                            # ignored without the flag
    assert _step(a) == DEVICE


def test_intermediate_state_buffer():
    a, spare = _valid_args()
    a.inter_state, a.inter_stride = spare, 4 * 128 * 128
    assert _step(a) == DEVICE
    a.inter_state = spare + 8
    assert _step(a) == ALIGN
    assert _step(a, flags=kda.KDA_FLAG_STATE_BF16) == DEVICE     # 8 bytes is enough for bf16
    a.inter_state, a.inter_stride = spare, 4 * 128 * 128 - 4
    assert _step(a) == SHAPE
    a.inter_stride = 4 * 128 * 128 + 2
    assert _step(a) == ALIGN
    a, _ = _valid_args()
    a.inter_state, a.inter_stride = a.state + (1 << 20), 4 * 128 * 128   # inside the pool
    assert _step(a) == ALIAS
    a, _ = _valid_args()
    a.inter_state, a.inter_stride = a.out, 4 * 128 * 128
    assert _step(a) == ALIAS
    a, _ = _valid_args()
    a.inter_state, a.inter_stride = a.g, 4 * 128 * 128
    assert _step(a) == ALIAS


def _raw_args():
    """Valid fake arguments with the raw gate form (g and beta cleared)."""
    a, spare = _valid_args()
    a.raw_gate, a.raw_gate_stride = a.g, 4 * 128          # reuse g's region (bf16 needs less)
    a.raw_beta, a.raw_beta_stride = a.beta, 4
    a.A_log = spare
    a.dt_bias = spare + 4096
    a.g = a.beta = 0
    return a


def test_raw_gate_form():
    a = _raw_args()
    assert _step(a) == DEVICE                              # passes host validation
    for f in ("raw_beta", "A_log", "dt_bias"):
        a = _raw_args()
        setattr(a, f, 0)
        assert _step(a) == NULL, f
    # mixed forms
    a = _raw_args()
    a.g = BASE + 50 * (1 << 26)
    assert _step(a) == UNSUP
    a = _raw_args()
    a.beta = BASE + 50 * (1 << 26)
    assert _step(a) == UNSUP
    a, spare = _valid_args()
    a.A_log = spare                                        # activated form plus a raw field
    assert _step(a) == UNSUP
    # strides and alignment
    for field, value, status in (("raw_gate_stride", 4 * 128 - 8, SHAPE), ("raw_beta_stride", 3, SHAPE),
                                 ("raw_gate_stride", 4 * 128 + 4, ALIGN)):
        a = _raw_args()
        setattr(a, field, value)
        assert _step(a) == status, field
    for field, offset in (("raw_gate", 8), ("raw_beta", 1), ("A_log", 2), ("dt_bias", 8)):
        a = _raw_args()
        setattr(a, field, getattr(a, field) + offset)
        assert _step(a) == ALIGN, field
    # written buffers may not overlap the raw inputs
    a = _raw_args()
    a.out = a.dt_bias + 1024
    assert _step(a) == ALIAS
    a = _raw_args()
    a.state = a.A_log
    assert _step(a) == ALIAS
    # no requests: nothing is read, every pointer may be NULL
    a = _raw_args()
    a.N = 0
    a.q = a.k = a.v = a.out = a.raw_gate = 0
    a.raw_beta = a.A_log = a.dt_bias = 0
    assert _step(a) == 0


def test_aliasing():
    a, _ = _valid_args()
    a.out = a.q + 256                              # out inside q
    assert _step(a) == ALIAS
    a, _ = _valid_args()
    a.state = a.g                                  # state on g
    assert _step(a) == ALIAS
    a, _ = _valid_args()
    a.out = a.state + 8 * 4 * 128 * 128 * 4 - 64   # out starts in the last pool slot
    a.out -= a.out % 8
    assert _step(a) == ALIAS
    a, _ = _valid_args()
    a.slot_idx = a.state + 64                      # metadata inside the pool
    assert _step(a) == ALIAS
    a, cu = _valid_args()
    a.out = cu                                     # out over cu_seqlens
    assert _packed(a, cu, 4) == ALIAS
    # inputs may overlap each other: q and k as views of one projection
    a, _ = _valid_args()
    a.k = a.q + 2 * 128 * 2
    a.q_stride = a.k_stride = 4 * 128
    assert _step(a) == DEVICE                      # passes validation, stops at the device check


def test_unknown_flags():
    for flags in (4, 1 << 10, 1 << 20, 1 << 31, kda.KDA_FLAG_KERNEL(6), kda.KDA_FLAG_KERNEL(15),
                  kda.KDA_FLAG_ORDER(3), kda.KDA_FLAG_PLACEMENT(2), kda.KDA_FLAG_PLACEMENT(3)):
        a, _ = _valid_args()
        assert _step(a, T=2, flags=flags) == UNSUP, hex(flags)
    a, _ = _valid_args()
    a.gate, a.gate_stride, a.norm_weight = BASE + 40 * (1 << 26), 4 * 128, BASE + 41 * (1 << 26)
    assert _step(a, flags=kda.KDA_FLAG_VTILE(32)) == UNSUP      # the norm needs 128 columns


def _norm_args():
    a, cu = _valid_args()
    a.gate, a.gate_stride, a.norm_weight = BASE + 40 * (1 << 26), 4 * 128, BASE + 41 * (1 << 26)
    return a, cu


K, O, P = kda.KDA_FLAG_KERNEL, kda.KDA_FLAG_ORDER, kda.KDA_FLAG_PLACEMENT
XCD = P(kda.KDA_PLACEMENT_HEAD_XCD)


@pytest.mark.parametrize("make,T,flags,expect", [
    # forced kernels the library provides: validation passes, the device check stops the call
    (_valid_args, 1, K(kda.KDA_KERNEL_WIDE), DEVICE),
    (_valid_args, 2, K(kda.KDA_KERNEL_WIDE) | kda.KDA_FLAG_VTILE(64), DEVICE),
    (_valid_args, 1, K(kda.KDA_KERNEL_QUARTER4), DEVICE),
    (_valid_args, 3, K(kda.KDA_KERNEL_QUARTER8) | O(kda.KDA_ORDER_INPUTS_FIRST), DEVICE),
    (_valid_args, 4, K(kda.KDA_KERNEL_SPLIT) | O(kda.KDA_ORDER_TILE_FIRST), DEVICE),
    (_valid_args, 2, O(kda.KDA_ORDER_INPUTS_FIRST), DEVICE),    # the library's kernel, forced order
    (_norm_args, 2, K(kda.KDA_KERNEL_QUARTER8), DEVICE),
    (_norm_args, 1, K(kda.KDA_KERNEL_WIDE), DEVICE),
    (_valid_args, 4, K(kda.KDA_KERNEL_SPLIT) | XCD, DEVICE),   # a head's value tiles on one XCD
    (_valid_args, 2, XCD, DEVICE),                             # the library's split-key kernel, placed so
    (_valid_args, 3, K(kda.KDA_KERNEL_SPLIT) | O(kda.KDA_ORDER_INPUTS_FIRST) | XCD, DEVICE),
    # combinations no kernel provides
    (_valid_args, 2, K(kda.KDA_KERNEL_QUARTER4) | kda.KDA_FLAG_VTILE(64), UNSUP),   # a width is for WIDE only
    (_norm_args, 2, K(kda.KDA_KERNEL_QUARTER4), UNSUP),         # the norm: 128 columns per workgroup
    (_norm_args, 2, K(kda.KDA_KERNEL_SPLIT), UNSUP),
    (_norm_args, 1, K(kda.KDA_KERNEL_WIDE) | kda.KDA_FLAG_VTILE(64), UNSUP),
    (_valid_args, 1, K(kda.KDA_KERNEL_QUARTER2), UNSUP),        # two waves: one-token fused-gate calls only
    (_valid_args, 1, K(kda.KDA_KERNEL_WIDE) | O(kda.KDA_ORDER_TILE_FIRST), UNSUP),   # the body fixes the order
    (_valid_args, 1, K(kda.KDA_KERNEL_SPLIT) | O(kda.KDA_ORDER_INPUTS_FIRST), UNSUP),   # one token: tile first
    (_valid_args, 2, K(kda.KDA_KERNEL_SPLIT) | O(kda.KDA_ORDER_INPUTS_FIRST) | kda.KDA_FLAG_STATE_BF16, UNSUP),
    (_valid_args, 1, K(kda.KDA_KERNEL_SPLIT) | XCD, UNSUP),    # placement: multi-token split-key calls only
    (_valid_args, 2, K(kda.KDA_KERNEL_QUARTER4) | XCD, UNSUP),
    (_valid_args, 2, K(kda.KDA_KERNEL_SPLIT) | XCD | kda.KDA_FLAG_STATE_BF16, UNSUP),
])
def test_forced_kernels(make, T, flags, expect):
    a, _ = make()
    a.N = 2 if T > 2 else a.N
    assert _step(a, T=T, flags=flags) == expect


def test_forced_split_kernel_refuses_packed_calls():
    a, cu = _valid_args()
    assert _packed(a, cu, 4, flags=K(kda.KDA_KERNEL_SPLIT)) == UNSUP
    assert _packed(a, cu, 4, flags=XCD) == UNSUP
    assert _packed(a, cu, 4, flags=K(kda.KDA_KERNEL_QUARTER4)) == DEVICE


def test_zero_requests_is_a_no_op():
    a, _ = _valid_args(N=0)
    a.q = a.k = a.v = a.g = a.beta = a.out = 0
    assert _step(a) == 0


def test_gated_rmsnorm_validation():
    f = kda.library().kda_gated_rmsnorm
    x, z, w, y = BASE, BASE + (1 << 26), BASE + 2 * (1 << 26), BASE + 3 * (1 << 26)
    assert f(None, z, w, y, 4, 128, 1e-6, None) == NULL
    assert f(x, z, w, y, 4, 127, 1e-6, None) == SHAPE
    assert f(x, z, w, y, 4, 0, 1e-6, None) == SHAPE
    assert f(x, z, w, y, 4, 128, -1.0, None) == SHAPE
    assert f(x + 2, z, w, y, 4, 128, 1e-6, None) == ALIGN
    assert f(x, z, w, x + 256, 4, 128, 1e-6, None) == ALIAS     # partial overlap
    assert f(x, z, w, z, 4, 128, 1e-6, None) == ALIAS
    assert f(x, z, w, x, 0, 128, 1e-6, None) == 0                # in place, no rows


def test_valid_call_without_gpu_reports_device():
    a, _ = _valid_args()
    assert _step(a) == DEVICE

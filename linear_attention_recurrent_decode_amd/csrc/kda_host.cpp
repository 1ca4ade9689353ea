// kda_host.cpp -- host layer of libkda.so: the C ABI entry points declared
// in kda.h, the O(1) argument validation every call passes before anything
// is launched, and the launch plan (which kernel, how many waves, which
// load order) keyed on the call's (request, value head) count N*HV, its
// tokens per request and its options.  No HIP types: the kernels and their
// launches are behind kda_launch.h.

#include <string.h>

#include "kda_launch.h"

namespace kda_internal {
namespace {

struct ByteRange {
    uintptr_t lo = 0, hi = 0;   // [lo, hi), empty when lo == hi
};

// Bounding byte range of a strided [rows][inner] tensor.
ByteRange span(const void *ptr, int64_t rows, int64_t stride, int64_t inner, int64_t elem)
{
    ByteRange r;
    if (!ptr || rows <= 0 || inner <= 0)
        return r;
    r.lo = reinterpret_cast<uintptr_t>(ptr);
    r.hi = r.lo + (uintptr_t)(((rows - 1) * stride + inner) * elem);
    return r;
}

bool overlaps(ByteRange a, ByteRange b)
{
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t bytes)
{
    return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

int vtile_from_flags(uint32_t flags)
{
    switch ((flags & KDA_FLAG_VTILE_MASK) >> KDA_FLAG_VTILE_SHIFT) {
    case 1: return 32;
    case 2: return 64;
    case 3: return 128;
    default: return 0;
    }
}

constexpr uint32_t KNOWN_FLAGS = KDA_FLAG_STATE_BF16 | KDA_FLAG_VALIDATE | KDA_FLAG_VTILE_MASK |
                                 KDA_FLAG_KERNEL_MASK | KDA_FLAG_ORDER_MASK | KDA_FLAG_PLACEMENT_MASK;

// Sizes, null pointers, alignment and overlap of a decode call (the rules of
// kda.h, "One decode call").
kda_status validate(const kda_decode_args *a, int64_t tokens, const int32_t *cu_seqlens, uint32_t flags)
{
    if (flags & ~KNOWN_FLAGS)
        return KDA_ERR_UNSUPPORTED;
    const int64_t state_elem = (flags & KDA_FLAG_STATE_BF16) ? 2 : 4;
    if (a->N < 0 || a->H < 1 || a->HV < 1 || a->HV > 65535 || a->HV % a->H != 0 || tokens < 0)
        return KDA_ERR_SHAPE;
    if (a->K != KD || a->V != VD)
        return KDA_ERR_SHAPE;
    // the gate inputs come in one form: activated (g, beta) or raw
    const bool raw = a->raw_gate != nullptr;
    if (raw ? (a->g || a->beta) : (a->raw_beta || a->A_log || a->dt_bias))
        return KDA_ERR_UNSUPPORTED;
    if (a->N == 0)
        return KDA_OK;
    // per-token tensors may be NULL only when the call holds no token rows
    if (tokens > 0 && (!a->q || !a->k || !a->v || !a->out || (!raw && (!a->g || !a->beta))))
        return KDA_ERR_NULL;
    if (raw && (!a->raw_beta || !a->A_log || !a->dt_bias))
        return KDA_ERR_NULL;
    if (!a->state || !a->slot_idx)
        return KDA_ERR_NULL;
    if (!a->norm_weight && a->gate)
        return KDA_ERR_NULL;
    const int64_t hk = (int64_t)a->H * a->K, hvk = (int64_t)a->HV * a->K, hvv = (int64_t)a->HV * a->V;
    if (a->num_slots < 0 || a->slot_stride < hvk * a->V)
        return KDA_ERR_SHAPE;
    if (a->q_stride < hk || a->k_stride < hk || a->v_stride < hvv || a->out_stride < hvv ||
        (a->gate && a->gate_stride < hvv))
        return KDA_ERR_SHAPE;
    if (raw ? (a->raw_gate_stride < hvk || a->raw_beta_stride < a->HV)
            : (a->g_stride < hvk || a->beta_stride < a->HV))
        return KDA_ERR_SHAPE;
    if (!(a->norm_eps >= 0.0f))
        return KDA_ERR_SHAPE;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || a->q_stride % 8 || a->k_stride % 8 ||
        !aligned(a->v, 8) || a->v_stride % 4 ||
        (raw ? (!aligned(a->raw_gate, 16) || a->raw_gate_stride % 8 || !aligned(a->raw_beta, 2) ||
                !aligned(a->A_log, 4) || !aligned(a->dt_bias, 16))
             : (!aligned(a->g, 16) || a->g_stride % 4 || !aligned(a->beta, 4))) ||
        !aligned(a->state, 4 * state_elem) || a->slot_stride % 4 ||
        !aligned(a->out, 8) || a->out_stride % 4 || !aligned(a->slot_idx, 4) ||
        (cu_seqlens && !aligned(cu_seqlens, 4)) ||
        (a->gate && (!aligned(a->gate, 8) || a->gate_stride % 4 || !aligned(a->norm_weight, 8))))
        return KDA_ERR_ALIGN;

    const ByteRange out = span(a->out, tokens, a->out_stride, hvv, 2);
    const ByteRange state = span(a->state, a->num_slots, a->slot_stride, hvk * a->V, state_elem);
    const ByteRange inputs[] = {
        span(a->q, tokens, a->q_stride, hk, 2),
        span(a->k, tokens, a->k_stride, hk, 2),
        span(a->v, tokens, a->v_stride, hvv, 2),
        span(a->g, tokens, a->g_stride, hvk, 4),
        span(a->beta, tokens, a->beta_stride, a->HV, 4),
        span(a->slot_idx, 1, 0, a->N, 4),
        span(cu_seqlens, 1, 0, (int64_t)a->N + 1, 4),
        span(a->gate, tokens, a->gate_stride, hvv, 2),
        span(a->norm_weight, 1, 0, a->V, 2),
        span(a->raw_gate, tokens, a->raw_gate_stride, hvk, 2),
        span(a->raw_beta, tokens, a->raw_beta_stride, a->HV, 2),
        span(a->A_log, 1, 0, a->HV, 4),
        span(a->dt_bias, 1, 0, hvk, 4),
    };
    if (overlaps(out, state))
        return KDA_ERR_ALIAS;
    for (const ByteRange &in : inputs)
        if (overlaps(out, in) || overlaps(state, in))
            return KDA_ERR_ALIAS;
    ByteRange inter;
    if (a->inter_state) {
        if (!aligned(a->inter_state, 4 * state_elem) || a->inter_stride % 4)
            return KDA_ERR_ALIGN;
        if (a->inter_stride < hvk * a->V)
            return KDA_ERR_SHAPE;
        inter = span(a->inter_state, tokens, a->inter_stride, hvk * a->V, state_elem);
        if (overlaps(inter, out) || overlaps(inter, state))
            return KDA_ERR_ALIAS;
        for (const ByteRange &in : inputs)
            if (overlaps(inter, in))
                return KDA_ERR_ALIAS;
    }
    if (flags & KDA_FLAG_VALIDATE) {
        if (!a->device_status)
            return KDA_ERR_NULL;
        if (!aligned(a->device_status, 4))
            return KDA_ERR_ALIGN;
        const ByteRange st = span(a->device_status, 1, 0, 1, 4);
        if (overlaps(st, out) || overlaps(st, state) || overlaps(st, inter))
            return KDA_ERR_ALIAS;
        for (const ByteRange &in : inputs)
            if (overlaps(st, in))
                return KDA_ERR_ALIAS;
    }
    return KDA_OK;
}

// ------------------------------------------------------------------ plan
//
// What a call looks like to the plan: its (request, value head) tile count
// `units` = N*HV, its tokens per request (0 for a packed call), and its
// options.
struct CallShape {
    int64_t units;
    int32_t T;      // 0: packed
    bool bf16, norm, raw;
};

// Value-tile width of the 32-column kernel from the tile count, tuned on
// MI355X with cold caches (256 compute units; A/B blocks as below):
//   fewer tiles than compute units: 32 columns, one wave per workgroup, the
//     most workgroups in flight for a latency-bound call (N20/T1 5.08 vs
//     5.63 us at 64 columns, N24/T1 5.39 vs 5.80);
//   one token per request, 256 .. 1023 tiles: 64 columns (N32/T1 6.69 vs
//     6.95 at 32 and 7.06 at 128, N40/T1 8.26 vs 8.62 and 11.07);
//   two tokens per request (the kernel serves them at 513 .. 768 tiles): 64
//     columns (N80/T2 15.10 vs 16.18, N96/T2 18.65 vs 20.16 at 128);
//   three or more tokens, or 1024 tiles and up: 128 columns (N80/T4 18.28
//     vs 19.37, N88/T3 16.94 vs 17.79 at 64).
// The norm epilogue needs all 128 columns in one workgroup.
int32_t plan_vtile(int64_t units, int32_t T, bool norm)
{
    if (norm)
        return 128;
    if (units < 256)
        return 32;
    if ((T <= 1 && units < 1024) || T == 2)
        return 64;
    return 128;
}

// The 32-column kernel's body: packed batches the staged body; step calls
// with several tokens per request, fewer than 512 tiles (two per compute
// unit), the fused gate activation or a bf16 pool the peeled body (its
// straight-line first token also lets the activation run while the tile is
// in flight, and at 144 VGPRs it runs three waves per SIMD, which the
// half-size bf16 tiles need); otherwise the prefetching loop (measured on
// MI355X, cold caches).
int32_t plan_body(const CallShape &c)
{
    if (c.T == 0)
        return BODY_STAGED;
    return (c.T > 1 || c.units < 512 || c.raw || c.bf16) ? BODY_PEELED : BODY_LOOP;
}

// The 16-column layouts: 0 = the 32-column kernel, PLAN_SPLIT = the
// split-key kernel, else kda_decode_q_kernel's waves per workgroup (2, 4 or
// 8).  Every boundary below is an A/B measurement on MI355X (bench.py
// --flags-b: the two choices in alternating A B B A blocks of 200 cold
// calls in one process; H = 8 unless noted; us per call, block spread
// +-0.2 to 0.5%):
//   fp32, one token: split-key waves up to 128 tiles (N16: 4.54 vs 4.75 on
//     the 32-column kernel), the 32-column kernel from there (N20 5.12 vs
//     5.21, N24 5.42 vs 5.96 on four 16-column waves) to 256 tiles (N32 6.53
//     vs 7.12), four 16-column waves to 384 (N33 7.38 vs 7.67, N36 7.49 vs
//     7.92, N48 9.13 vs 9.62 and 9.95 on eight; fused gate N33 7.60 vs 7.98,
//     N48 9.20 vs 9.70), eight 16-column waves beyond (N50 10.12 vs 11.34,
//     N52 10.32 vs 12.20 on four, N64 11.91 vs 12.86); with the fused gate
//     two 16-column waves up to 64 tiles (N8 3.80 vs 3.91 split-key, 4.06
//     32-column; N9 4.24 on the 32-column kernel vs 4.36);
//   fp32, two or more tokens: split-key waves up to 320 tiles (N32/T4 8.46
//     vs 8.76 on four 16-column waves, N36/T4 9.21 vs 9.56, N40/T4 9.48 vs
//     9.71, N40/T2 8.49 vs 8.59, N40/T3 8.81 vs 8.98; N44/T3 9.84 vs 9.08
//     and N48/T4 10.75 vs 10.35 the other way); four 16-column waves to 576
//     tiles, 512 with two tokens
//     (N64/T2 12.30 vs 13.27 on the 32-column kernel, N72/T4 17.51 vs 19.70;
//     but N72/T2 17.21 vs 14.90); the 32-column kernel to 768 (N80/T4 18.65
//     vs 18.89, N96/T4 20.33 vs 22.33, N88/T3 16.93 vs 20.83, N96/T2 18.65
//     vs 21.55); four 16-column waves again to 1536 (N104/T4 24.70 vs 27.70,
//     N112/T2 24.35 vs 25.57, N104/T3 23.65 vs 25.34, N128/T2 26.84 vs
//     29.04, N160/T4 35.67 vs 37.10 and 37.20 on eight), eight beyond
//     (N256/T4 54.41 vs 55.37 on four and 57.45 on the 32-column kernel,
//     N256/T2 53.22 vs 54.20);
//   fp32, packed (1 to 4 tokens per request): four 16-column waves up to
//     1024 tiles (N8: 5.63 vs 7.64 on the 32-column kernel, N24 7.69 vs
//     9.28 and 8.75 on eight waves, N32 8.14 vs 9.40, N48 10.20 vs 12.48,
//     N96 22.7 vs 24.4, N128 29.25 vs 29.17), eight beyond (N256 51.3 vs
//     54.8, the H12 batch 67.6 vs 73.3 and 69.7 on the 32-column kernel);
//   bf16 pool, no norm: four 16-column waves (full 128-byte row pieces of
//     bf16) at every size (N32/T1 5.15 vs 5.81 on the 32-column kernel and
//     5.68 on eight waves, N128/T1 15.3 vs 16.3 on eight), the split-key
//     waves with two or more tokens up to 32 tiles (N4/T4 4.85 vs 5.00) and
//     for one-token calls with activated gates up to 24 tiles (N1 3.03 vs
//     3.23, N2 3.11 vs 3.29, N3 3.24 vs 3.31; N4 3.34 both, N6 3.61 vs 3.45
//     the other way; with the fused gate equal at N1 and N2, N4 3.57 vs
//     3.41 the other way);
//   the norm epilogue (the head's 128 columns in one workgroup: eight
//     16-column waves or the 32-column kernel at 128 columns): eight waves
//     for every bf16-pool call, fp32 calls of two or more tokens up to 512
//     tiles (N8/H16/T4 9.72 vs 10.58) and fp32 one-token calls from 512
//     (N32/H16 12.35 vs 12.61, N48/H16 20.3 vs 21.5; N16/H16 8.56 vs 7.83
//     the other way).
constexpr int32_t PLAN_SPLIT = 1;

int32_t plan_quarter_waves(const CallShape &c)
{
    if (c.norm) {
        if (c.bf16)
            return 8;
        return (c.T >= 2 ? c.units <= 512 : c.T == 1 && c.units >= 512) ? 8 : 0;
    }
    if (c.bf16)
        return ((c.T >= 2 && c.units <= 32) || (c.T == 1 && !c.raw && c.units <= 24)) ? PLAN_SPLIT : 4;
    if (c.T == 0)
        return c.units <= 1024 ? 4 : 8;
    if (c.T == 1) {
        if (c.units > 384)
            return 8;
        if (c.units > 256)
            return 4;
        if (c.raw)
            return c.units <= 64 ? 2 : 0;
        return c.units <= 128 ? PLAN_SPLIT : 0;
    }
    if (c.units <= 320)
        return PLAN_SPLIT;
    if (c.units <= (c.T == 2 ? 512 : 576))
        return 4;
    if (c.units <= 768)
        return 0;
    return c.units <= 1536 ? 4 : 8;
}

// The load order of a 16-column-wave launch: the first token's inputs
// before the state tile (so that their state-free part runs while the tile
// is in flight) for fp32-pool calls from 192 tiles with two or more tokens
// per request, or packed on eight waves: eight waves always, split-key
// waves up to 256 tiles, four waves with three or more tokens; otherwise
// the tile first.  Measured as above: split-key N24/T4 7.49 vs 7.62 tile
// first, N33/T2 7.33 tile first vs 7.72 on four waves, N36/T2 7.52 tile
// first vs 8.24 inputs first; four waves N32/T4 8.78 vs 8.95 tile first,
// N48/T4 10.31 vs 10.72, N64/T4 12.76 vs 13.09, N70/T4 17.18 vs 17.78;
// packed, eight waves: the H12 batch 67.7 vs 68.8 tile first; four waves:
// N24 7.58 tile first vs 7.69, N64 13.43 vs 13.53.  With one token the tile
// first wins at every size (N1 3.04 vs 3.54 us, N64 12.2 vs 12.9), and with
// a bf16 pool, whose tiles are half the bytes.
bool plan_early(const CallShape &c, int32_t waves, bool split)
{
    if (c.bf16 || c.T == 1 || c.units < 192)
        return false;
    if (c.T == 0 || waves == 8)
        return waves == 8;
    if (split)
        return c.units <= 256;
    return c.T >= 3;
}

// The library's plan for a call.
Plan library_plan(const CallShape &c)
{
    Plan p;
    const int32_t nq = plan_quarter_waves(c);
    if (nq == PLAN_SPLIT) {
        p.kernel = KERNEL_SPLIT;
        p.waves = 4;
        p.early = plan_early(c, 4, true);
    } else if (nq) {
        p.kernel = KERNEL_QUARTER;
        p.waves = c.norm ? 8 : nq;
        p.early = plan_early(c, p.waves, false);
    } else {
        p.kernel = KERNEL_WIDE;
        p.waves = plan_vtile(c.units, c.T, c.norm) / 32;
        p.body = plan_body(c);
    }
    return p;
}

// The plan a call's flags force (KDA_FLAG_VTILE, KDA_FLAG_KERNEL,
// KDA_FLAG_ORDER), or the library's; KDA_ERR_UNSUPPORTED for a combination
// no kernel provides.
kda_status call_plan(const CallShape &c, uint32_t flags, Plan &out)
{
    const int vtile = vtile_from_flags(flags);
    int code = (int)((flags & KDA_FLAG_KERNEL_MASK) >> KDA_FLAG_KERNEL_SHIFT);
    const int order = (int)((flags & KDA_FLAG_ORDER_MASK) >> KDA_FLAG_ORDER_SHIFT);
    const int placement = (int)((flags & KDA_FLAG_PLACEMENT_MASK) >> KDA_FLAG_PLACEMENT_SHIFT);
    if (code == 0 && vtile)
        code = KDA_KERNEL_WIDE;
    if (vtile && code != KDA_KERNEL_WIDE)
        return KDA_ERR_UNSUPPORTED;
    if (placement > KDA_PLACEMENT_HEAD_XCD)
        return KDA_ERR_UNSUPPORTED;
    Plan p = library_plan(c);
    if (code == 0 && order == 0 && placement == 0) {
        out = p;
        return KDA_OK;
    }
    switch (code) {
    case 0:
        break;
    case KDA_KERNEL_WIDE:
        p = Plan();
        p.kernel = KERNEL_WIDE;
        p.waves = (vtile ? vtile : plan_vtile(c.units, c.T, c.norm)) / 32;
        p.body = plan_body(c);
        break;
    case KDA_KERNEL_QUARTER2:
    case KDA_KERNEL_QUARTER4:
    case KDA_KERNEL_QUARTER8:
        p = Plan();
        p.kernel = KERNEL_QUARTER;
        p.waves = code == KDA_KERNEL_QUARTER2 ? 2 : code == KDA_KERNEL_QUARTER4 ? 4 : 8;
        p.early = plan_early(c, p.waves, false);
        break;
    case KDA_KERNEL_SPLIT:
        p = Plan();
        p.kernel = KERNEL_SPLIT;
        p.waves = 4;
        p.early = plan_early(c, 4, true);
        break;
    default:
        return KDA_ERR_UNSUPPORTED;
    }
    if (order) {
        if (order > KDA_ORDER_INPUTS_FIRST || (p.kernel != KERNEL_QUARTER && p.kernel != KERNEL_SPLIT))
            return KDA_ERR_UNSUPPORTED;   // the 32-column kernel's body fixes its order
        p.early = order == KDA_ORDER_INPUTS_FIRST;
    }
    // what the kernels provide
    if (c.norm && !((p.kernel == KERNEL_WIDE && p.waves == 4) || (p.kernel == KERNEL_QUARTER && p.waves == 8)))
        return KDA_ERR_UNSUPPORTED;
    if (p.kernel == KERNEL_SPLIT && c.T == 0)
        return KDA_ERR_UNSUPPORTED;
    if (p.kernel == KERNEL_QUARTER && p.waves == 2 && !(c.raw && !c.bf16 && c.T == 1 && !c.norm))
        return KDA_ERR_UNSUPPORTED;
    if (p.early && (c.bf16 || c.T == 1))
        return KDA_ERR_UNSUPPORTED;
    if (placement) {
        // the head-per-XCD order exists for the multi-token fp32 split-key kernels
        if (p.kernel != KERNEL_SPLIT || c.T < 2 || c.bf16)
            return KDA_ERR_UNSUPPORTED;
        p.head_xcd = true;
    }
    out = p;
    return KDA_OK;
}

kda_status run_decode(const kda_decode_args *a, int32_t T, const int32_t *cu_seqlens, int64_t tokens,
                      uint32_t flags, void *stream)
{
    if (!a)
        return KDA_ERR_NULL;
    kda_status st = validate(a, tokens, cu_seqlens, flags);
    if (st != KDA_OK)
        return st;
    if (a->N == 0)
        return KDA_OK;
    DecodeCall call;
    call.args = a;
    call.T = cu_seqlens ? 0 : T;
    call.cu_seqlens = cu_seqlens;
    call.tokens = tokens;
    call.bf16_state = (flags & KDA_FLAG_STATE_BF16) != 0;
    call.validate = (flags & KDA_FLAG_VALIDATE) != 0;
    const CallShape shape{(int64_t)a->N * a->HV, call.T, call.bf16_state, a->gate != nullptr, a->raw_gate != nullptr};
    st = call_plan(shape, flags, call.plan);
    if (st != KDA_OK)
        return st;
    const uint64_t qk_magic = (uint64_t(1) << 32) / (uint64_t)(a->HV / a->H) + 1;
    call.qk_magic = (uint32_t)qk_magic;
    call.qk_magic_hi = (uint32_t)(qk_magic >> 32);
    call.stream = stream;
    st = device_ready();
    if (st != KDA_OK)
        return st;
    return launch_decode(call);
}

}  // namespace
}  // namespace kda_internal

using namespace kda_internal;

extern "C" {

kda_status kda_decode_step(const kda_decode_args *args, int32_t T, uint32_t flags, void *stream)
{
    if (!args)
        return KDA_ERR_NULL;
    if (T < 1)
        return KDA_ERR_SHAPE;
    return run_decode(args, T, nullptr, (int64_t)args->N * T, flags, stream);
}

kda_status kda_decode_packed(const kda_decode_args *args, const int32_t *cu_seqlens, int64_t total_tokens,
                             uint32_t flags, void *stream)
{
    if (!args || !cu_seqlens)
        return KDA_ERR_NULL;
    return run_decode(args, 0, cu_seqlens, total_tokens, flags, stream);
}

kda_status kda_gated_rmsnorm(const void *x, const void *gate, const void *weight, void *y, int64_t rows,
                             int32_t V, float eps, void *stream)
{
    if (!x || !gate || !weight || !y)
        return KDA_ERR_NULL;
    if (rows < 0 || V < 2 || V > 8192 || V % 2 || !(eps >= 0.0f))
        return KDA_ERR_SHAPE;
    if (!aligned(x, 4) || !aligned(gate, 4) || !aligned(weight, 4) || !aligned(y, 4))
        return KDA_ERR_ALIGN;
    const ByteRange yr = span(y, rows, V, V, 2);
    if (y != x && overlaps(yr, span(x, rows, V, V, 2)))
        return KDA_ERR_ALIAS;
    if (overlaps(yr, span(gate, rows, V, V, 2)) || overlaps(yr, span(weight, 1, 0, V, 2)))
        return KDA_ERR_ALIAS;
    if (rows == 0)
        return KDA_OK;
    if ((rows + 3) / 4 > 0x7FFFFFFF)
        return KDA_ERR_SHAPE;
    const kda_status st = device_ready();
    if (st != KDA_OK)
        return st;
    return launch_gated_rmsnorm(x, gate, weight, y, rows, V, eps, stream);
}

int32_t kda_decode_plan(int64_t units, int32_t T, uint32_t options)
{
    const bool packed = (options & KDA_PLAN_PACKED) != 0;
    const CallShape c{units, packed ? 0 : (T < 1 ? 1 : T), (options & KDA_PLAN_STATE_BF16) != 0,
                      (options & KDA_PLAN_NORM) != 0, (options & KDA_PLAN_RAW_GATE) != 0};
    const Plan p = library_plan(c);
    if (options & KDA_PLAN_LAYOUT)
        return p.kernel;
    return p.columns();
}

const char *kda_status_string(kda_status status)
{
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range or unsupported";
    case KDA_ERR_ALIGN: return "a pointer or stride breaks the alignment rules";
    case KDA_ERR_ALIAS: return "a written buffer overlaps another buffer of the call";
    case KDA_ERR_UNSUPPORTED: return "unsupported flag or mode";
    case KDA_ERR_DEVICE: return "the current device is not gfx950, or a HIP query failed";
    case KDA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"

// kda_launch.h -- internal interface between the host layer of libkda.so
// (kda_host.cpp: argument validation, the launch plan, the C ABI entry
// points) and its kernel layer (kda_decode.hip: the gfx950 kernels and their
// launches).  Plain C++17 without HIP types, so that the host layer builds
// with any C++ compiler (and host-only, with sanitizers, in the tests).
#ifndef KDA_LAUNCH_H
#define KDA_LAUNCH_H

#include <stdint.h>

#include "kda.h"

#define KDA_INTERNAL __attribute__((visibility("hidden")))

namespace kda_internal {

constexpr int KD = 128;   // key head size the kernels take
constexpr int VD = 128;   // value head size the kernels take

// Kernel families: the lane layouts of kda_decode.hip (KDA_LAYOUT_* values).
enum Kernel : int32_t {
    KERNEL_WIDE = KDA_LAYOUT_WIDE,         // kda_decode_kernel: 32-column waves
    KERNEL_QUARTER = KDA_LAYOUT_QUARTER,   // kda_decode_q_kernel: 16-column waves, 32 key rows per lane
    KERNEL_SPLIT = KDA_LAYOUT_SPLIT,       // kda_decode_split_kernel: 16 key rows per lane, two row halves
};

// Bodies of the 32-column kernel.
enum Body : int32_t { BODY_LOOP = 0, BODY_PEELED = 1, BODY_STAGED = 2 };

// One launch: which kernel, how many waves, which body and load order.
struct Plan {
    int32_t kernel = KERNEL_WIDE;
    int32_t waves = 4;       // WIDE: 1, 2 or 4 waves of 32 columns; QUARTER: 2, 4 or 8 waves of 16 columns;
                             // SPLIT: 4 (two column waves x two row halves)
    int32_t body = BODY_PEELED;   // WIDE only
    bool early = false;      // QUARTER, SPLIT: the first token's inputs before the state tile
    bool head_xcd = false;   // SPLIT: a head's value tiles on one XCD (KDA_PLACEMENT_HEAD_XCD)

    // value columns one workgroup holds
    int32_t columns() const
    {
        switch (kernel) {
        case KERNEL_WIDE: return 32 * waves;
        case KERNEL_QUARTER: return 16 * waves;
        default: return 32;   // KERNEL_SPLIT
        }
    }
};

// A validated decode call and its plan.
struct DecodeCall {
    const kda_decode_args *args = nullptr;
    int32_t T = 0;                        // step call: tokens per request; packed call: 0
    const int32_t *cu_seqlens = nullptr;  // packed call: [N + 1]
    int64_t tokens = 0;                   // token rows of the per-token tensors
    bool bf16_state = false, validate = false;
    uint32_t qk_magic = 0, qk_magic_hi = 0;   // q/k head of value head hv: hv / (HV / H) as a multiply
    Plan plan;
    void *stream = nullptr;
};

// The current device is a gfx950 (checked once per device, with the kernel
// attributes set there); KDA_ERR_DEVICE otherwise.
KDA_INTERNAL kda_status device_ready();

// Enqueue the call's kernels (the metadata check first with validation).
KDA_INTERNAL kda_status launch_decode(const DecodeCall &call);

// Enqueue the standalone gated RMSNorm over `rows` rows of V values.
KDA_INTERNAL kda_status launch_gated_rmsnorm(const void *x, const void *gate, const void *weight, void *y,
                                             int64_t rows, int32_t V, float eps, void *stream);

}  // namespace kda_internal

#endif  // KDA_LAUNCH_H

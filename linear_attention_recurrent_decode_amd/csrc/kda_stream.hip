// kda_stream.hip -- the tile-stream reference (include/kda_stream.h): the
// state bytes of a decode call moved in place with no arithmetic, timed by
// the benchmark beside the decode.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "kda_stream.h"

namespace {

constexpr int STREAM_THREADS = 512;
constexpr int TILE_ELEMS = 128 * 128;
constexpr int MAX_REQUESTS = 65535;   // grid y

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One (request, value head) tile per workgroup: PIECES 16-byte pieces per
// lane (8 for an fp32 tile of 64 KiB, 4 for bf16), lane t taking pieces
// t, t + 512, ...: each instruction of the workgroup covers 8 KiB of
// contiguous rows.  All loads return before the first store (the barrier).
template <int PIECES>
__global__ __launch_bounds__(STREAM_THREADS) void kda_stream_tiles_kernel(u32x4 *state, const int32_t *slot_idx,
                                                                          int64_t num_slots,
                                                                          int64_t slot_stride_bytes)
{
    const int64_t slot = slot_idx[blockIdx.y];
    if ((slot < 0) | (slot >= num_slots))
        return;
    constexpr int64_t TILE_BYTES = (int64_t)PIECES * STREAM_THREADS * 16;
    u32x4 *t = reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(state) + slot * slot_stride_bytes +
                                         (int64_t)blockIdx.x * TILE_BYTES) +
               threadIdx.x;
    u32x4 r[PIECES];
#pragma unroll
    for (int j = 0; j < PIECES; ++j)
        r[j] = __builtin_nontemporal_load(t + j * STREAM_THREADS);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PIECES; ++j)
        __builtin_nontemporal_store(r[j], t + j * STREAM_THREADS);
}

}  // namespace

extern "C" kda_status kda_stream_tiles(void *state, int32_t elem_bytes, int64_t num_slots, int64_t slot_stride,
                                       const int32_t *slot_idx, int32_t N, int32_t HV, void *stream)
{
    if (!state || !slot_idx)
        return KDA_ERR_NULL;
    if ((elem_bytes != 2 && elem_bytes != 4) || N < 0 || N > MAX_REQUESTS || HV < 1 || HV > 65535 ||
        num_slots < 0 || slot_stride < (int64_t)HV * TILE_ELEMS)
        return KDA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(state) & 15) || ((slot_stride * elem_bytes) & 15) ||
        (reinterpret_cast<uintptr_t>(slot_idx) & 3))
        return KDA_ERR_ALIGN;
    if (N == 0)
        return KDA_OK;
    u32x4 *st = static_cast<u32x4 *>(state);
    int64_t stride_bytes = slot_stride * elem_bytes;
    void *args[] = {&st, &slot_idx, &num_slots, &stride_bytes};
    const void *fn = elem_bytes == 4 ? reinterpret_cast<const void *>(&kda_stream_tiles_kernel<8>)
                                     : reinterpret_cast<const void *>(&kda_stream_tiles_kernel<4>);
    return hipLaunchKernel(fn, dim3((uint32_t)HV, (uint32_t)N), dim3(STREAM_THREADS), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? KDA_OK
               : KDA_ERR_LAUNCH;
}

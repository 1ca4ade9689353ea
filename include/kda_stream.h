/*
 * kda_stream.h -- the tile-stream reference of the benchmark (libkda_stream.so).
 *
 * Not part of the decode path.  It moves exactly the state bytes a decode
 * call moves -- every live (request, value head) tile of the pool read once
 * and written back once, in place -- and computes nothing, so that the
 * benchmark can time it beside the decode over the same tiles, with the same
 * cold rotation and timing protocol: the time of the call's state traffic
 * alone at its launch shape on this GPU, a yardstick for the decode's time
 * (in one access pattern: the decode's own lane layouts can move the same
 * tiles faster).  The pages read their kernels against memory-bound timing
 * the same way: vLLM PR 57585, "Microbenchmark and earlier serving limits",
 * times calls with cold L2 in graph replay; FlashInfer PR 4562, description,
 * reports state bandwidth beside the kernel time.
 *
 * One workgroup of 512 lanes per tile: 16-byte non-temporal loads of the
 * whole tile (K = V = 128 rows of 128 elements, contiguous), a barrier, then
 * the same bytes stored back; the best of the in-place access patterns
 * measured on MI355X (waiting for all of a workgroup's loads before its first
 * store, whole 512-byte rows per workgroup).
 */
#ifndef KDA_STREAM_H
#define KDA_STREAM_H

#include <stdint.h>

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * state       device pool, (slot, hv, i, j) at slot*slot_stride + (hv*128 + i)*128 + j
 *             elements of elem_bytes (4: fp32, 2: bf16); 16-byte aligned, slot_stride
 *             >= HV*128*128 and slot_stride*elem_bytes a multiple of 16
 * slot_idx    device int32 [N]; a slot outside [0, num_slots) (-1: padding) is skipped
 * N, HV       requests (0 .. 65535) and value heads (1 .. 65535)
 * stream      hipStream_t (NULL: the default stream)
 * Returns KDA_OK after enqueueing one kernel (nothing for N = 0), or the
 * kda_status of the first argument check that fails (nothing enqueued), or
 * KDA_ERR_LAUNCH.  The pool's contents are unchanged.
 */
kda_status kda_stream_tiles(void *state, int32_t elem_bytes, int64_t num_slots, int64_t slot_stride,
                            const int32_t *slot_idx, int32_t N, int32_t HV, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_STREAM_H */

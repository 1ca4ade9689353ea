/*
 * kda.h -- C ABI of the MI355X (gfx950) recurrent KDA decode library (libkda.so).
 *
 * Recurrent KDA (Kimi Delta Attention) decode advances, for every live request
 * and value head, a K x V fp32 state S by one token at a time:
 *
 *   S <- diag(exp g_t) S                 per-key-channel decay
 *   v' = beta_t (v_t - S^T k_t)          delta-rule correction (decayed S)
 *   S <- S + k_t v'^T                    rank-1 update
 *   o_t = scale S^T q_t                  readout (updated S)
 *   y_t = gated_rmsnorm(o_t, z_t, w)     optional epilogue, else y_t = o_t
 *
 * Sources.  vLLM PR 57585 (recurrent KDA launch tuning on SM90), "Purpose and
 * source" and "Retained baseline trace attribution": the operation is a fused
 * recurrent KDA forward over N requests x HV value heads, launched 34 times
 * per decode graph, with bf16 inputs and fp32 state at K = V = 128
 * ("Microbenchmark and earlier serving limits").  FlashInfer PR 4562 (H12
 * packed decode across the SM100 family), inline review of the binding: q, k
 * and v arrive as row-strided views of one fused projection, gate and beta
 * per token, an indexed state pool with per-request slot indices, a
 * caller-owned output, the readout scale 1/sqrt(128) and per-token row
 * strides; its description adds caller-stream execution, row-strided beta,
 * padding rows that are skipped and graph replay.  b12x PR 249 (direct
 * single-token KDA decode), walkthrough: the decode kernel is followed by a
 * normalisation kernel that gates the decoded output; its review asks that
 * the written buffers (output, state) be checked against every input for
 * overlap before launch; its purpose section keeps the one-token case an
 * internal route of the general call.  The pages never print the recurrence
 * itself; the one above is the gated delta rule of Kimi Delta Attention.
 *
 * Conventions for every entry point.
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing, never synchronises and never copies to or
 *     from the host.  Each call enqueues one kernel on `stream` (two with
 *     KDA_FLAG_VALIDATE on a call of more than 64 requests, and one more per
 *     further 65535 requests of a call with more; a hipStream_t, NULL = the
 *     default stream) and returns; it can be captured into a HIP graph.
 *   - Arguments are validated on the host in O(1) before anything is
 *     launched.  On any error status nothing was launched and no buffer was
 *     touched, except KDA_ERR_LAUNCH (the runtime refused a launch): for a
 *     call of more than 65535 requests the request ranges before the
 *     refused launch may have been enqueued.
 *   - Strides are counted in elements of the tensor's own type.
 *   - bf16 tensors hold raw bf16 bit patterns (uint16_t storage).
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,         /* a required pointer is NULL                          */
    KDA_ERR_SHAPE = 2,        /* a size is out of range, or K, V are not 128         */
    KDA_ERR_ALIGN = 3,        /* a pointer or stride breaks the alignment rules      */
    KDA_ERR_ALIAS = 4,        /* out or state overlaps another buffer of the call    */
    KDA_ERR_UNSUPPORTED = 5,  /* unknown flag bits, or a mixed gate input form        */
    KDA_ERR_DEVICE = 6,       /* the current device is not gfx950, or a HIP query failed */
    KDA_ERR_LAUNCH = 7        /* the kernel launch failed                            */
} kda_status;

/* flags: bit 0 selects a bf16 state pool (`state` then points to bf16 bit
 * patterns; default fp32).  The state is widened exactly to fp32 on load, the
 * call's tokens are recurred in fp32, and the state is rounded to nearest even
 * once, when it is written back. */
#define KDA_FLAG_STATE_BF16 (1u << 0)

/* flags: bit 1 validates the device metadata before the decode, all or
 * nothing, and writes `device_status`: KDA_DEVICE_OK, or the lowest-numbered
 * KDA_DEVICE_ERR_* found.  The decode proceeds only if the metadata is valid;
 * otherwise no state, output or other buffer is touched.  A call of at most
 * 64 requests is checked by the decode kernel's own waves (no extra launch);
 * a larger call runs a one-workgroup check kernel first on the call's stream
 * (one extra launch; duplicates found through a hash table, O(N / 1024) per
 * 4096 requests).  Without this flag the metadata is trusted (slots outside
 * the pool are skipped). */
#define KDA_FLAG_VALIDATE (1u << 1)
#define KDA_DEVICE_OK 0
#define KDA_DEVICE_ERR_SLOT_RANGE 1   /* a slot index outside [0, num_slots) other than -1 */
#define KDA_DEVICE_ERR_SLOT_DUP 2     /* two live requests share one slot */
#define KDA_DEVICE_ERR_CU_SEQLENS 3   /* cu_seqlens negative, decreasing, or past total_tokens */

/* flags: bits 8..9 force the value-tile width of one workgroup
 * (1 = 32 columns, 2 = 64, 3 = 128; 0 = the library's choice) of 32-column
 * waves; the library's choice may instead use one of the 16-column-wave
 * layouts (kda_decode_plan with KDA_PLAN_LAYOUT names it).  Results are
 * bit-identical for every width and lane layout; the knob exists for tests
 * and tuning. */
#define KDA_FLAG_VTILE_SHIFT 8u
#define KDA_FLAG_VTILE_MASK (3u << KDA_FLAG_VTILE_SHIFT)
#define KDA_FLAG_VTILE(code) (((uint32_t)(code) & 3u) << KDA_FLAG_VTILE_SHIFT)

/* flags: bits 12..15 force the kernel (lane layout and workgroup) instead
 * of the library's choice, and bits 16..17 its load order; for tests and
 * for measuring one choice against another.  Kernel codes:
 *   KDA_KERNEL_WIDE        32-column waves (the width from KDA_FLAG_VTILE,
 *                          else the library's)
 *   KDA_KERNEL_QUARTER2/4/8  16-column waves, 2, 4 or 8 per workgroup
 *   KDA_KERNEL_SPLIT       split-key 16-column waves (step calls only)
 * Order codes (16-column and split-key waves): KDA_ORDER_TILE_FIRST (the
 * state tile's loads first) or KDA_ORDER_INPUTS_FIRST (the first token's
 * inputs first); 0 = the library's.  A combination no kernel provides (the
 * norm epilogue outside KDA_KERNEL_WIDE at 128 columns and
 * KDA_KERNEL_QUARTER8, a packed call on KDA_KERNEL_SPLIT, two 16-column
 * waves outside one-token fp32 calls with the fused gate, inputs first with
 * a bf16 pool or one token, an order for the 32-column kernel) is
 * KDA_ERR_UNSUPPORTED.  Every kernel, width and order gives bitwise the same
 * results. */
#define KDA_FLAG_KERNEL_SHIFT 12u
#define KDA_FLAG_KERNEL_MASK (15u << KDA_FLAG_KERNEL_SHIFT)
#define KDA_FLAG_KERNEL(code) (((uint32_t)(code) & 15u) << KDA_FLAG_KERNEL_SHIFT)
#define KDA_KERNEL_WIDE 1
#define KDA_KERNEL_QUARTER2 2
#define KDA_KERNEL_QUARTER4 3
#define KDA_KERNEL_QUARTER8 4
#define KDA_KERNEL_SPLIT 5
#define KDA_FLAG_ORDER_SHIFT 16u
#define KDA_FLAG_ORDER_MASK (3u << KDA_FLAG_ORDER_SHIFT)
#define KDA_FLAG_ORDER(code) (((uint32_t)(code) & 3u) << KDA_FLAG_ORDER_SHIFT)
#define KDA_ORDER_TILE_FIRST 1
#define KDA_ORDER_INPUTS_FIRST 2

/* flags: bits 18..19 force the placement of a call's workgroups over the
 * chip's 8 XCDs (each with its own L2), for measuring one placement against
 * the other.  0 = the library's: consecutive workgroups hold one head's
 * value tiles, so the hardware's round-robin hand-out spreads a head over
 * several XCDs.  KDA_PLACEMENT_HEAD_XCD: the value tiles of a head run on one
 * XCD, which then fetches the head's token inputs once instead of once per
 * tile (split-key waves with two or more tokens per request and an fp32 pool
 * only; elsewhere KDA_ERR_UNSUPPORTED).  Results are bitwise the same. */
#define KDA_FLAG_PLACEMENT_SHIFT 18u
#define KDA_FLAG_PLACEMENT_MASK (3u << KDA_FLAG_PLACEMENT_SHIFT)
#define KDA_FLAG_PLACEMENT(code) (((uint32_t)(code) & 3u) << KDA_FLAG_PLACEMENT_SHIFT)
#define KDA_PLACEMENT_HEAD_XCD 1

/*
 * One decode call.  Token t of the call is row t of every per-token tensor.
 *
 *   N          requests in the call (N = 0: nothing to do, returns KDA_OK)
 *   H          q/k heads;  HV value heads (at most 65535), a multiple of H; value head hv
 *              reads q/k head hv / (HV / H)
 *   K, V       key and value head size; the GPU kernels take K = V = 128
 *   scale      readout scale (1/sqrt(K) in the serving models)
 *   q, k       bf16, element (t, h, i) at t*q_stride + h*K + i.
 *              16-byte aligned; q_stride, k_stride multiples of 8, >= H*K
 *   v          bf16, element (t, hv, j) at t*v_stride + hv*V + j.
 *              8-byte aligned; v_stride a multiple of 4, >= HV*V
 *   g          fp32 log-decay (already activated, <= 0 in practice, -inf
 *              allowed: it clears that key row), (t, hv, i) at
 *              t*g_stride + hv*K + i.  16-byte aligned; g_stride a multiple
 *              of 4, >= HV*K
 *   beta       fp32, (t, hv) at t*beta_stride + hv; beta_stride >= HV
 *   state      fp32 pool (bf16 with KDA_FLAG_STATE_BF16), (slot, hv, i, j) at
 *              slot*slot_stride + (hv*K + i)*V + j (V contiguous), num_slots
 *              slots.  Read and written IN PLACE.  16-byte aligned (8 for
 *              bf16); slot_stride a multiple of 4, >= HV*K*V
 *   slot_idx   int32 [N]: the pool slot of each request.  A value outside
 *              [0, num_slots) (-1 marks a padding row) skips the request:
 *              no state is read or written and its output rows are left
 *              untouched.  Two live requests must not share a slot in one
 *              call (their updates would race).
 *   out        bf16 result, (t, hv, j) at t*out_stride + hv*V + j, written
 *              for live requests only.  8-byte aligned; out_stride a
 *              multiple of 4, >= HV*V
 *   gate       NULL: out = o (no epilogue).  Otherwise bf16 z, (t, hv, j) at
 *              t*gate_stride + hv*V + j (8-byte aligned, gate_stride a
 *              multiple of 4, >= HV*V), and
 *   norm_weight bf16 [V] (8-byte aligned), norm_eps > 0 or 0:
 *              out = o / sqrt(mean_j o^2 + eps) * w * silu(z).
 *
 *   raw_gate   NULL: g and beta are given activated (above).  Otherwise the
 *              kernel activates them from raw projections itself (FlashInfer
 *              PR 4562, inline review of the binding: bf16 raw_gate and
 *              raw_beta, fp32 A_log and dt_bias; the pages do not print the
 *              activation, the one used is the gate of Kimi Delta Attention):
 *                g_t[hv][i] = -exp(A_log[hv]) * softplus(raw_gate_t[hv][i] + dt_bias[hv][i])
 *                beta_t[hv] = sigmoid(raw_beta_t[hv])
 *              in fp32.  g and beta must then be NULL, and
 *              raw_gate   bf16, (t, hv, i) at t*raw_gate_stride + hv*K + i;
 *                         16-byte aligned, raw_gate_stride a multiple of 8, >= HV*K
 *              raw_beta   bf16, (t, hv) at t*raw_beta_stride + hv; raw_beta_stride >= HV
 *              A_log      fp32 [HV], 4-byte aligned
 *              dt_bias    fp32 [HV][K], 16-byte aligned
 *              are all required.  raw_beta, A_log or dt_bias without
 *              raw_gate, or g/beta with it, is KDA_ERR_UNSUPPORTED.
 *
 *   device_status  with KDA_FLAG_VALIDATE, a device int32 the call writes
 *              (4-byte aligned, overlapping no other buffer); else ignored.
 *   inter_state NULL, or the state of each live request's value head right
 *              after each of its tokens: (t, hv, i, j) at
 *              t*inter_stride + (hv*K + i)*V + j, the pool's element type and
 *              alignment, inter_stride a multiple of 4, >= HV*K*V.  For
 *              speculative decoding: the pool still ends with the state after
 *              the last token; a caller that accepts a >= 1 of a request's
 *              tokens restores row bos+a-1.  Rows of skipped requests are not
 *              written.
 *
 * Aliasing: out, state, inter_state and device_status may not overlap each
 * other or any input (q, k, v, g, beta, slot_idx, cu_seqlens, gate,
 * norm_weight, raw_gate, raw_beta, A_log, dt_bias); inputs may
 * overlap each other (q, k, v are often views of one projection).  Ranges are
 * the bounding byte ranges of each strided tensor.
 */
typedef struct kda_decode_args {
    int32_t N, H, HV, K, V;
    float scale;
    const void *q;      int64_t q_stride;
    const void *k;      int64_t k_stride;
    const void *v;      int64_t v_stride;
    const float *g;     int64_t g_stride;
    const float *beta;  int64_t beta_stride;
    void *state;        int64_t num_slots;   int64_t slot_stride;
    const int32_t *slot_idx;
    void *out;          int64_t out_stride;
    const void *gate;   int64_t gate_stride;
    const void *norm_weight;
    float norm_eps;
    int32_t *device_status;   /* KDA_FLAG_VALIDATE only: caller-owned device int32 */
    void *inter_state;  int64_t inter_stride;   /* NULL, or per-token states (below) */
    const void *raw_gate;  int64_t raw_gate_stride;   /* NULL, or the fused gate activation */
    const void *raw_beta;  int64_t raw_beta_stride;
    const float *A_log;
    const float *dt_bias;
} kda_decode_args;

/*
 * Every request decodes exactly T >= 1 tokens, request-major: request n owns
 * token rows n*T .. n*T+T-1.  The tokens of one request are recurred in
 * order within the call with the state held on chip; the state is written
 * back once, after the last token.  One-token decode (T = 1) is the common
 * serving case and takes the same entry point.  Equivalent to
 * kda_decode_packed with cu_seqlens[n] = n*T.
 *
 * Source: vLLM PR 57585, "Microbenchmark and earlier serving limits": the
 * decode call over N requests of T = 1 or 4 tokens, 8 or 16 heads,
 * K = V = 128, bf16 inputs and fp32 state; b12x PR 249, "Purpose": ordinary
 * decode, where every live request brings exactly one token, is the hot
 * case, and its maintainer's review keeps it an internal route of the one
 * public call rather than a second entry point.
 */
kda_status kda_decode_step(const kda_decode_args *args, int32_t T, uint32_t flags, void *stream);

/*
 * Packed variable-length decode: request n owns token rows
 * cu_seqlens[n] .. cu_seqlens[n+1]-1 (cu_seqlens: device int32 [N+1],
 * non-decreasing, cu_seqlens[N] <= total_tokens; a request with no tokens
 * leaves its slot untouched).  total_tokens is the number of token rows the
 * per-token tensors hold; it bounds the overlap checks only.  The device
 * metadata (slot_idx, cu_seqlens) is trusted as the serving scheduler wrote
 * it; slots outside the pool are skipped, never dereferenced.
 *
 * Source: FlashInfer PR 4562, description: packed decode that keeps
 * caller-stream execution, row-strided beta, an indexed (noncompact)
 * recurrent state, inactive graph-padding rows, a caller-owned output and
 * graph replay; b12x PR 249, "Purpose": packed, padded, speculative and
 * multi-token requests take the general route, which validates the device
 * metadata (KDA_FLAG_VALIDATE here).
 */
kda_status kda_decode_packed(const kda_decode_args *args, const int32_t *cu_seqlens,
                             int64_t total_tokens, uint32_t flags, void *stream);

/*
 * Standalone gated RMSNorm over rows of V values (b12x PR 249, walkthrough:
 * the normalisation kernel that gates the decoded output):
 *   y[r][j] = x[r][j] / sqrt(mean_j x[r][j]^2 + eps) * w[j] * silu(z[r][j])
 * x, gate, y: bf16 [rows][V] contiguous; weight bf16 [V]; V even, 2 <= V <= 8192;
 * all four 4-byte aligned; eps >= 0.  y may equal x exactly (in place); any
 * other overlap of y with x, gate or weight is KDA_ERR_ALIAS.
 */
kda_status kda_gated_rmsnorm(const void *x, const void *gate, const void *weight, void *y,
                             int64_t rows, int32_t V, float eps, void *stream);

/* options of kda_decode_plan (bit set; 0 = fp32 pool, step call, no norm) */
#define KDA_PLAN_NORM 1u         /* the gated RMSNorm epilogue */
#define KDA_PLAN_STATE_BF16 2u   /* a bf16 state pool (KDA_FLAG_STATE_BF16) */
#define KDA_PLAN_PACKED 4u       /* a packed call (kda_decode_packed) */
#define KDA_PLAN_LAYOUT 8u       /* report the lane layout (KDA_LAYOUT_*) instead */
#define KDA_PLAN_RAW_GATE 16u    /* the fused gate activation (raw_gate set) */

/* lane layouts of the same arithmetic (the results are bitwise the same) */
#define KDA_LAYOUT_WIDE 0      /* 32-column waves: a lane holds 4 columns x 16 key rows */
#define KDA_LAYOUT_QUARTER 1   /* 16-column waves: a lane holds 1 column x 32 key rows */
#define KDA_LAYOUT_SPLIT 2     /* 16-column waves with the key rows split over two waves:
                                  a lane holds 1 column x 16 key rows */

/* The columns per workgroup (32, 64 or 128) the library picks for a call of
 * `units` = N*HV (request, value head) pairs with T tokens per request (any
 * T >= 1 for a packed call) and the given KDA_PLAN_* options, or with
 * KDA_PLAN_LAYOUT the lane layout it picks; without a forced KDA_FLAG_VTILE
 * width (which always selects KDA_LAYOUT_WIDE).  Host-only, no device
 * access.  The launch choice keyed on N*HV and T is the role of vLLM PR
 * 57585's stage predicate (description: two pipeline stages for grids of at
 * most 32 N*HV pairs) and of FlashInfer PR 4562's qualified batch selector
 * (description); the thresholds here are this chip's measurements. */
int32_t kda_decode_plan(int64_t units, int32_t T, uint32_t options);

/* Static description of a status code.  Source: b12x PR 249, inline review
 * of the overlap checks: a call whose written buffers overlap its inputs is
 * rejected with an error before any launch; FlashInfer PR 4562,
 * description: inputs outside the supported bands are routed fail-closed.
 * Every such refusal is a kda_status here; this returns its text. */
const char *kda_status_string(kda_status status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */

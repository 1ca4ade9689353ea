/*
 * The C ABI used from plain C: no Python, no torch.  Allocates device memory
 * with the HIP runtime, fills the inputs with a small deterministic generator
 * of its own (no step of the decode), runs kda_decode_step and
 * kda_decode_packed through kda.h with an fp32 and a bf16 state pool, and
 * compares outputs and states with the CPU oracle (test infrastructure,
 * linked only here).
 *
 * Exit status 0 and a last line "c abi ok" on success; 1 with a message on
 * the first mismatch; 2 when the HIP runtime or the library reports an error.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

/* the oracle's entry point (oracle/kda_oracle.c) */
int kda_oracle_decode(int64_t N, int64_t H, int64_t HV, int64_t K, int64_t V, const int32_t *cu_seqlens,
                      const uint16_t *q, int64_t q_stride, const uint16_t *k, int64_t k_stride,
                      const uint16_t *v, int64_t v_stride, const float *g, int64_t g_stride,
                      const float *beta, int64_t beta_stride, double *state, int64_t num_slots,
                      int64_t slot_stride, const int32_t *slot_idx, double scale, const uint16_t *gate,
                      int64_t gate_stride, const uint16_t *norm_weight, double eps, double *out,
                      int64_t out_stride, double *inter_state, int64_t inter_stride, const uint16_t *raw_gate,
                      int64_t raw_gate_stride, const uint16_t *raw_beta, int64_t raw_beta_stride,
                      const float *A_log, const float *dt_bias);

#define CHECK_HIP(x)                                                                 \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

enum { K = 128, V = 128 };
static const float SCALE = 0.08838834764831845f;   /* 1/sqrt(128), as the library receives it */

/* xorshift64* : uniform in [-1, 1) */
static uint64_t rng_state = 0x243F6A8885A308D3ull;
static double uniform_pm1(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    const uint64_t r = rng_state * 0x2545F4914F6CDD1Dull;
    return (double)(r >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float bf16_to_float(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static void *device_copy(const void *host, size_t bytes)
{
    void *d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes ? bytes : 1));
    if (bytes)
        CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* One call of N requests x T tokens (packed: per-request lengths in lens),
 * H q/k heads, HV value heads, an fp32 or bf16 state pool, checked against
 * the oracle (which starts from the pool's values and keeps fp64 state; a
 * bf16 pool is compared within half a bf16 ulp plus the recurrence's own
 * rounding). */
static int run_case(const char *name, int N, int H, int HV, int T, const int *lens, int num_slots, int bf16_pool)
{
    int32_t *cu = malloc(sizeof(int32_t) * (size_t)(N + 1));
    cu[0] = 0;
    for (int n = 0; n < N; ++n)
        cu[n + 1] = cu[n] + (lens ? lens[n] : T);
    const int tokens = cu[N];
    const size_t nq = (size_t)tokens * H * K, nv = (size_t)tokens * HV * V, ng = (size_t)tokens * HV * K;
    const size_t slot_elems = (size_t)HV * K * V, pool_elems = (size_t)num_slots * slot_elems;

    uint16_t *q = malloc(nq * 2), *k = malloc(nq * 2), *v = malloc(nv * 2);
    float *g = malloc(ng * 4), *beta = malloc((size_t)tokens * HV * 4), *pool = malloc(pool_elems * 4);
    int32_t *slot = malloc(sizeof(int32_t) * (size_t)N);
    for (size_t i = 0; i < nq; ++i) {
        q[i] = to_bf16((float)(0.09 * uniform_pm1()));
        k[i] = to_bf16((float)(0.09 * uniform_pm1()));
    }
    for (size_t i = 0; i < nv; ++i)
        v[i] = to_bf16((float)uniform_pm1());
    for (size_t i = 0; i < ng; ++i)
        g[i] = (float)(-0.7 + 0.6 * uniform_pm1());
    for (int i = 0; i < tokens * HV; ++i)
        beta[i] = (float)(0.5 + 0.4 * uniform_pm1());
    for (size_t i = 0; i < pool_elems; ++i)
        pool[i] = (float)(0.05 * uniform_pm1());
    uint16_t *pool16 = malloc(pool_elems * 2);
    if (bf16_pool)
        for (size_t i = 0; i < pool_elems; ++i) {
            pool16[i] = to_bf16(pool[i]);
            pool[i] = bf16_to_float(pool16[i]);      /* the oracle starts from the stored values */
        }
    for (int n = 0; n < N; ++n)     /* distinct slots (7 is odd and coprime to the pool sizes); every third request a padding row */
        slot[n] = (n % 3 == 2) ? -1 : (int32_t)((n * 7 + 1) % num_slots);

    uint16_t *dq = device_copy(q, nq * 2), *dk = device_copy(k, nq * 2), *dv = device_copy(v, nv * 2);
    float *dg = device_copy(g, ng * 4), *dbeta = device_copy(beta, (size_t)tokens * HV * 4);
    void *dpool = bf16_pool ? device_copy(pool16, pool_elems * 2) : device_copy(pool, pool_elems * 4);
    int32_t *dslot = device_copy(slot, sizeof(int32_t) * (size_t)N), *dcu = device_copy(cu, sizeof(int32_t) * (size_t)(N + 1));
    uint16_t *dout = NULL;
    const size_t out_bytes = nv > 0 ? nv * 2 : 1;
    CHECK_HIP(hipMalloc((void **)&dout, out_bytes));
    CHECK_HIP(hipMemset(dout, 0, out_bytes));

    kda_decode_args a;
    memset(&a, 0, sizeof a);
    a.N = N; a.H = H; a.HV = HV; a.K = K; a.V = V;
    a.scale = SCALE;
    a.q = dq; a.q_stride = H * K;
    a.k = dk; a.k_stride = H * K;
    a.v = dv; a.v_stride = HV * V;
    a.g = dg; a.g_stride = HV * K;
    a.beta = dbeta; a.beta_stride = HV;
    a.state = dpool; a.num_slots = num_slots; a.slot_stride = (int64_t)slot_elems;
    a.slot_idx = dslot;
    a.out = dout; a.out_stride = HV * V;
    const uint32_t flags = bf16_pool ? KDA_FLAG_STATE_BF16 : 0;
    kda_status st = lens ? kda_decode_packed(&a, dcu, tokens, flags, NULL) : kda_decode_step(&a, T, flags, NULL);
    if (st != KDA_OK) {
        fprintf(stderr, "%s: library status %d (%s)\n", name, (int)st, kda_status_string(st));
        return 2;
    }
    CHECK_HIP(hipDeviceSynchronize());

    uint16_t *out = malloc(nv * 2);
    float *gpool = malloc(pool_elems * 4);
    CHECK_HIP(hipMemcpy(out, dout, nv * 2, hipMemcpyDeviceToHost));
    if (bf16_pool) {
        CHECK_HIP(hipMemcpy(pool16, dpool, pool_elems * 2, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < pool_elems; ++i)
            gpool[i] = bf16_to_float(pool16[i]);
    } else {
        CHECK_HIP(hipMemcpy(gpool, dpool, pool_elems * 4, hipMemcpyDeviceToHost));
    }

    double *ref_pool = malloc(pool_elems * 8), *ref_out = malloc(nv * 8);
    for (size_t i = 0; i < pool_elems; ++i)
        ref_pool[i] = pool[i];
    for (size_t i = 0; i < nv; ++i)
        ref_out[i] = NAN;
    if (kda_oracle_decode(N, H, HV, K, V, cu, q, H * K, k, H * K, v, HV * V, g, HV * K, beta, HV, ref_pool,
                          num_slots, (int64_t)slot_elems, slot, (double)SCALE, NULL, 0, NULL, 0.0, ref_out,
                          HV * V, NULL, 0, NULL, 0, NULL, 0, NULL, NULL) != 0) {
        fprintf(stderr, "%s: oracle rejected the case\n", name);
        return 1;
    }
    double max_out = 0.0, max_state = 0.0;
    for (size_t i = 0; i < nv; ++i) {
        const double got = bf16_to_float(out[i]);
        if (isnan(ref_out[i])) {            /* padding rows stay untouched (zero) */
            if (out[i] != 0) {
                fprintf(stderr, "%s: padding output %zu written\n", name, i);
                return 1;
            }
            continue;
        }
        const double err = fabs(got - ref_out[i]);
        if (err > 2e-3 + ldexp(fabs(ref_out[i]), -8)) {
            fprintf(stderr, "%s: output %zu: %g vs %g\n", name, i, got, ref_out[i]);
            return 1;
        }
        if (err > max_out)
            max_out = err;
    }
    for (size_t i = 0; i < pool_elems; ++i) {
        const double err = fabs((double)gpool[i] - ref_pool[i]);
        if (err > (bf16_pool ? ldexp(fabs(ref_pool[i]), -8) : 1e-4 * fabs(ref_pool[i])) + 1e-6) {
            fprintf(stderr, "%s: state %zu: %g vs %g\n", name, i, (double)gpool[i], ref_pool[i]);
            return 1;
        }
        if (err > max_state)
            max_state = err;
    }
    printf("%s: %d requests, %d tokens: out max|d| %.3e, state max|d| %.3e\n", name, N, tokens, max_out, max_state);

    hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dg); hipFree(dbeta); hipFree(dpool); hipFree(dslot);
    hipFree(dcu); hipFree(dout);
    free(q); free(k); free(v); free(g); free(beta); free(pool); free(pool16); free(slot); free(cu); free(out);
    free(gpool);
    free(ref_pool); free(ref_out);
    return 0;
}

int main(void)
{
    int device_count = 0;
    if (hipGetDeviceCount(&device_count) != hipSuccess || device_count < 1) {
        fprintf(stderr, "no HIP device\n");
        return 2;
    }
    /* rejected before anything is launched: K = 64 */
    kda_decode_args bad;
    memset(&bad, 0, sizeof bad);
    bad.N = 1; bad.H = bad.HV = 1; bad.K = 64; bad.V = 128;
    if (kda_decode_step(&bad, 1, 0, NULL) != KDA_ERR_SHAPE) {
        fprintf(stderr, "K = 64 was not rejected\n");
        return 1;
    }
    /* the plan for a packed bf16 call: 64-column workgroups; a small step
     * call: the split-key layout */
    if (kda_decode_plan(4096, 1, KDA_PLAN_STATE_BF16 | KDA_PLAN_PACKED) != 64 || kda_decode_plan(256, 1, 0) != 64 ||
        kda_decode_plan(36, 3, KDA_PLAN_LAYOUT) != KDA_LAYOUT_SPLIT ||
        kda_decode_plan(9, 2, KDA_PLAN_STATE_BF16 | KDA_PLAN_LAYOUT) != KDA_LAYOUT_SPLIT) {
        fprintf(stderr, "unexpected launch plan\n");
        return 1;
    }
    static const int lens[7] = {1, 4, 2, 3, 1, 2, 4};
    int rc = run_case("step N=9 H=2 HV=4 T=3", 9, 2, 4, 3, NULL, 16, 0);
    if (rc == 0)
        rc = run_case("step N=40 H=8 HV=8 T=1", 40, 8, 8, 1, NULL, 64, 0);
    if (rc == 0)
        rc = run_case("packed N=7 H=1 HV=3", 7, 1, 3, 0, lens, 12, 0);
    if (rc == 0)
        rc = run_case("bf16 pool, step N=40 H=8 HV=8 T=2", 40, 8, 8, 2, NULL, 64, 1);
    if (rc == 0)
        rc = run_case("bf16 pool, packed N=7 H=1 HV=3", 7, 1, 3, 0, lens, 12, 1);
    if (rc == 0)
        rc = run_case("bf16 pool, step N=3 H=1 HV=3 T=2", 3, 1, 3, 2, NULL, 8, 1);
    if (rc == 0)
        printf("c abi ok\n");
    return rc;
}

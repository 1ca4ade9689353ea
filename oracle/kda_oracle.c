/*
 * CPU oracle for recurrent KDA (Kimi Delta Attention) decode.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only code that may load this library.
 * The GPU library never calls it and shares no code with it: no header,
 * helper, table or constant.
 *
 * What it computes.  The pages name the operation "recurrent KDA" decode
 * (vLLM PR 57585, "Purpose and source" and "Retained baseline trace
 * attribution": a fused recurrent KDA forward that each decode graph launches
 * 34 times, over N requests x HV value heads) but never print the
 * recurrence.  The recurrence used here is the per-key-channel gated delta
 * rule of Kimi Delta Attention, applied to one token after another for each
 * (request, value head) with a K x V fp state S:
 *
 *   1. decay        S[i][j] <- exp(g_t[i]) * S[i][j]
 *   2. correction   u[j] = sum_i S[i][j] k_t[i];   v'[j] = beta_t (v_t[j] - u[j])
 *   3. update       S[i][j] <- S[i][j] + k_t[i] v'[j]
 *   4. readout      o_t[j] = scale * sum_i S[i][j] q_t[i]
 *   5. (optional)   gated RMSNorm of o_t over j, then stored
 *
 * Step 2 uses the decayed state, step 4 the updated state.  The readout scale
 * the pages pass is 1/sqrt(128) (FlashInfer PR 4562, inline review of the
 * binding's launch arguments).  Step 5 follows the b12x PR 249 walkthrough,
 * where a normalisation kernel gates the decoded output with z before it is
 * written to the caller's buffer: y[j] = o[j] / sqrt(mean_j o^2 + eps) *
 * w[j] * silu(z[j]), silu(x) = x / (1 + exp(-x)).
 *
 * Gate activation (optional step 0).  The log-decay g_t and beta_t arrive
 * either already activated (fp32) or as raw projections: FlashInfer PR 4562
 * (inline review of the binding's launch arguments) hands its kernel a bf16
 * raw_gate and raw_beta with fp32 A_log and dt_bias, and b12x PR 249 (its
 * review of the aliasing checks) lists raw_g and raw_beta among the decode's
 * inputs.  Neither page prints the activation.  The reading taken here is
 * the gate of Kimi Delta Attention:
 *
 *   g_t[i]  = -exp(A_log[hv]) * softplus(raw_gate_t[hv][i] + dt_bias[hv][i])
 *   beta_t  = sigmoid(raw_beta_t[hv])
 *   softplus(x) = log(1 + exp(x)),  sigmoid(x) = 1 / (1 + exp(-x))
 *
 * A_log is one value per value head, dt_bias one per (value head, key
 * channel).  With A_log = 0 and dt_bias = 0 it reduces to g = -softplus(x)
 * and beta = sigmoid(x) of the raw values.
 *
 * Slots.  Request n reads and writes state slot slot_idx[n]; a slot outside
 * [0, num_slots) (the value -1 marks a padding row) means the request is
 * skipped: its state is neither read nor written and none of its output
 * tokens are written (FlashInfer PR 4562, description: indexed state and
 * padding rows).
 *
 * Arithmetic.  Everything is double precision, in the order written above,
 * one scalar at a time, sums taken in ascending index order.  bf16 inputs are
 * widened exactly.  Build without -ffast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double (exact: a bf16 is the top half of an fp32) */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double silu(double x)
{
    return x / (1.0 + exp(-x));
}

/* softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log(1 + e^-|x|) so
 * that no exponential overflows; +inf maps to +inf and -inf to 0. */
static double softplus(double x)
{
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* the logistic function; -inf maps to 0 and +inf to 1 */
static double sigmoid(double r)
{
    return 1.0 / (1.0 + exp(-r));
}

/* Step 0 for value head hv of token t: the log-decay of every key channel
 * and beta from the raw projections (reading at the top of this file).
 * raw_gate (t, hv, i) at t*raw_gate_stride + hv*K + i; raw_beta (t, hv) at
 * t*raw_beta_stride + hv; A_log [HV]; dt_bias (hv, i) at hv*K + i. */
static void activate_gates(int64_t t, int64_t hv, int64_t K,
                           const uint16_t *raw_gate, int64_t raw_gate_stride,
                           const uint16_t *raw_beta, int64_t raw_beta_stride,
                           const float *A_log, const float *dt_bias,
                           double *g_out, double *beta_out)
{
    const double A = exp((double)A_log[hv]);
    const uint16_t *rg = raw_gate + t * raw_gate_stride + hv * K;
    for (int64_t i = 0; i < K; ++i)
        g_out[i] = -A * softplus(bf16_value(rg[i]) + (double)dt_bias[hv * K + i]);
    *beta_out = sigmoid(bf16_value(raw_beta[t * raw_beta_stride + hv]));
}

/* Gated RMSNorm of one row of V values (b12x PR 249, walkthrough: the
 * normalisation kernel that gates the decoded output).  mean over the row,
 * eps inside the square root, then per-column weight and silu(gate). */
static void gated_rmsnorm_row(const double *o, const uint16_t *z, const uint16_t *w,
                              int64_t V, double eps, double *y)
{
    double sum_sq = 0.0;
    for (int64_t j = 0; j < V; ++j)
        sum_sq += o[j] * o[j];
    double r = 1.0 / sqrt(sum_sq / (double)V + eps);
    for (int64_t j = 0; j < V; ++j)
        y[j] = o[j] * r * bf16_value(w[j]) * silu(bf16_value(z[j]));
}

/*
 * Decode every request over its token range [cu_seqlens[n], cu_seqlens[n+1]).
 *
 *   q, k   bf16 bits, element (t, h, i) at  t*q_stride + h*K + i
 *   v      bf16 bits, element (t, hv, j) at t*v_stride + hv*V + j
 *   g      fp32 log-decay, (t, hv, i) at    t*g_stride + hv*K + i
 *   beta   fp32, (t, hv) at                 t*beta_stride + hv
 *   state  double pool, (slot, hv, i, j) at slot*slot_stride + (hv*K + i)*V + j,
 *          updated in place
 *   gate   bf16 bits (t, hv, j) at t*gate_stride + hv*V + j, or NULL (no norm)
 *   norm_weight bf16 bits [V] (used with gate)
 *   out    double, (t, hv, j) at t*out_stride + hv*V + j; written for live
 *          requests only
 *   inter_state  NULL, or double (t, hv, i, j) at t*inter_stride + (hv*K + i)*V + j:
 *          the state of each live request's value head right after token t
 *          (what a speculative decoder restores when it accepts tokens up to t)
 *   raw_gate  NULL: g and beta are used as given.  Otherwise step 0 computes
 *          the log-decay and beta from raw_gate, raw_beta (bf16 bits), A_log
 *          and dt_bias (layouts at activate_gates) and g, beta are ignored.
 *
 * Value head hv reads q/k head hv / (HV / H).
 * Returns 0, or a negative number for arguments it cannot interpret.
 */
int kda_oracle_decode(int64_t N, int64_t H, int64_t HV, int64_t K, int64_t V,
                      const int32_t *cu_seqlens,
                      const uint16_t *q, int64_t q_stride,
                      const uint16_t *k, int64_t k_stride,
                      const uint16_t *v, int64_t v_stride,
                      const float *g, int64_t g_stride,
                      const float *beta, int64_t beta_stride,
                      double *state, int64_t num_slots, int64_t slot_stride,
                      const int32_t *slot_idx, double scale,
                      const uint16_t *gate, int64_t gate_stride,
                      const uint16_t *norm_weight, double eps,
                      double *out, int64_t out_stride,
                      double *inter_state, int64_t inter_stride,
                      const uint16_t *raw_gate, int64_t raw_gate_stride,
                      const uint16_t *raw_beta, int64_t raw_beta_stride,
                      const float *A_log, const float *dt_bias)
{
    if (N < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0)
        return -1;
    if (slot_stride < HV * K * V || (inter_state && inter_stride < HV * K * V))
        return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -2;

    if (raw_gate && (!raw_beta || !A_log || !dt_bias))
        return -1;

    double *vp = malloc(sizeof(double) * (size_t)V);   /* v' */
    double *o = malloc(sizeof(double) * (size_t)V);
    double *y = malloc(sizeof(double) * (size_t)V);
    double *gd = malloc(sizeof(double) * (size_t)K);   /* log-decay of the token */
    if (!vp || !o || !y || !gd) {
        free(vp); free(o); free(y); free(gd);
        return -3;
    }
    const int64_t heads_per_qk = HV / H;

    for (int64_t n = 0; n < N; ++n) {
        const int64_t slot = slot_idx[n];
        if (slot < 0 || slot >= num_slots)
            continue;                               /* padding row: skipped */
        for (int64_t hv = 0; hv < HV; ++hv) {
            const int64_t h = hv / heads_per_qk;
            double *S = state + slot * slot_stride + hv * K * V;
            for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
                const uint16_t *qt = q + t * q_stride + h * K;
                const uint16_t *kt = k + t * k_stride + h * K;
                const uint16_t *vt = v + t * v_stride + hv * V;
                double bt;

                /* 0. log-decay and beta: given, or activated from raw projections */
                if (raw_gate) {
                    activate_gates(t, hv, K, raw_gate, raw_gate_stride, raw_beta, raw_beta_stride,
                                   A_log, dt_bias, gd, &bt);
                } else {
                    const float *gt = g + t * g_stride + hv * K;
                    for (int64_t i = 0; i < K; ++i)
                        gd[i] = (double)gt[i];
                    bt = (double)beta[t * beta_stride + hv];
                }

                /* 1. decay: row i of S scaled by exp(g_t[i]) */
                for (int64_t i = 0; i < K; ++i) {
                    const double a = exp(gd[i]);
                    for (int64_t j = 0; j < V; ++j)
                        S[i * V + j] = a * S[i * V + j];
                }
                /* 2. delta correction against the decayed state */
                for (int64_t j = 0; j < V; ++j) {
                    double u = 0.0;
                    for (int64_t i = 0; i < K; ++i)
                        u += S[i * V + j] * bf16_value(kt[i]);
                    vp[j] = bt * (bf16_value(vt[j]) - u);
                }
                /* 3. rank-1 update S += k v'^T */
                for (int64_t i = 0; i < K; ++i) {
                    const double ki = bf16_value(kt[i]);
                    for (int64_t j = 0; j < V; ++j)
                        S[i * V + j] = S[i * V + j] + ki * vp[j];
                }
                /* 4. readout from the updated state */
                for (int64_t j = 0; j < V; ++j) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < K; ++i)
                        acc += S[i * V + j] * bf16_value(qt[i]);
                    o[j] = scale * acc;
                }
                /* 5. optional gated RMSNorm, then the output row */
                double *dst = out + t * out_stride + hv * V;
                if (gate) {
                    gated_rmsnorm_row(o, gate + t * gate_stride + hv * V, norm_weight, V, eps, y);
                    memcpy(dst, y, sizeof(double) * (size_t)V);
                } else {
                    memcpy(dst, o, sizeof(double) * (size_t)V);
                }
                if (inter_state)
                    memcpy(inter_state + t * inter_stride + hv * K * V, S, sizeof(double) * (size_t)(K * V));
            }
        }
    }
    free(vp); free(o); free(y); free(gd);
    return 0;
}

/*
 * Step 0 alone over a batch of token rows: g (double [tokens][HV][K]) and
 * beta (double [tokens][HV]) from the raw projections, with the layouts of
 * activate_gates.
 */
int kda_oracle_gate_activation(int64_t tokens, int64_t HV, int64_t K,
                               const uint16_t *raw_gate, int64_t raw_gate_stride,
                               const uint16_t *raw_beta, int64_t raw_beta_stride,
                               const float *A_log, const float *dt_bias,
                               double *g, double *beta)
{
    if (tokens < 0 || HV < 1 || K < 1 || raw_gate_stride < HV * K || raw_beta_stride < HV)
        return -1;
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t hv = 0; hv < HV; ++hv)
            activate_gates(t, hv, K, raw_gate, raw_gate_stride, raw_beta, raw_beta_stride, A_log, dt_bias,
                           g + (t * HV + hv) * K, beta + t * HV + hv);
    return 0;
}

/*
 * Standalone gated RMSNorm over rows of V bf16 values (the same row
 * operation as step 5, applied to a bf16 input x instead of the fp o).
 *   x, gate: bf16 bits [rows][V] contiguous; norm_weight bf16 bits [V];
 *   y: double [rows][V].
 */
int kda_oracle_gated_rmsnorm(int64_t rows, int64_t V, const uint16_t *x,
                             const uint16_t *gate, const uint16_t *norm_weight,
                             double eps, double *y)
{
    if (rows < 0 || V < 1)
        return -1;
    double *row = malloc(sizeof(double) * (size_t)V);
    if (!row)
        return -3;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < V; ++j)
            row[j] = bf16_value(x[r * V + j]);
        gated_rmsnorm_row(row, gate + r * V, norm_weight, V, eps, y + r * V);
    }
    free(row);
    return 0;
}

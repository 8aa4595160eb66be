/*
 * CPU oracle for the DiLoCo outer-step merge.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP library.
 *
 * Every function is a plain loop over elements that applies the merge's
 * definition one IEEE-754 binary32 operation at a time, in the order written.
 * The source pages fix the precision: the merger keeps "a running fp32 sum"
 * (DiffuRefill-1B model card, "How it is trained", Merging bullet) and the
 * fragments are fp32 (GradientMail post, "Getting updates through the
 * bucket").  So each value is rounded to binary32 after every operation, with
 * round-to-nearest-even, no fused multiply-add (build with -ffp-contract=off),
 * IEEE division, denormals kept and NaN propagated.  On x86-64 the C float
 * type is evaluated in SSE registers (FLT_EVAL_METHOD 0), so a float
 * expression is rounded at each operator.
 *
 * Loops are split across threads with OpenMP where the build enables it;
 * every element is independent, so the split does not change any result.
 *
 * Pins (checked by the CPU test suite against mathematics, not against this
 * file): exact rational results on dyadic inputs, closed forms of the EMA and
 * of the Nesterov recursion, the reduction of momentum 0 / learning rate 1 to
 * the token-weighted mean, library means and weighted averages in fp64 within
 * derived bounds, the identity on identical checkpoints, and hand-derived
 * arrival-order examples.
 */
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* bfloat16 is the upper half of an IEEE binary32 word, so widening puts its
 * 16 bits in the high half of a 32-bit word with zeros below; exact. */
static float oracle_bf16_value(uint16_t bits)
{
    uint32_t word = ((uint32_t)bits) << 16;
    float value;
    memcpy(&value, &word, sizeof value);
    return value;
}

static float oracle_ckpt_value(const void *ckpt, int dtype, int64_t j)
{
    if (dtype == ORACLE_BF16)
        return oracle_bf16_value(((const uint16_t *)ckpt)[j]);
    return ((const float *)ckpt)[j];
}

/*
 * Plain replacement averaging, folding step (DiffuRefill-1B model card, "How
 * it is trained", Merging bullet: each checkpoint is added to an fp32 running
 * sum in the order it comes in, and the round's result is its average;
 * technical report, "Training system", Table 2, row "Outer step": the next
 * global is that average of the workers).
 *
 * One arriving checkpoint c of n elements (fp32 or bf16 widened to fp32) is
 * added to the running sum: sum[j] = c[j] for the first arrival of the round,
 * sum[j] = sum[j] + c[j] for every later one.  Callers fold in arrival order.
 */
void oracle_fold_mean(float *sum, const void *ckpt, int dtype, int64_t n, int first)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float c = oracle_ckpt_value(ckpt, dtype, j);
        if (first)
            sum[j] = c;
        else
            sum[j] = sum[j] + c;
    }
}

/*
 * Plain replacement averaging, closing step: global = sum / N, N the number of
 * checkpoints folded (same passages as above).  If ema is not NULL the EMA of
 * globals is advanced as well (technical report, Table 2, Side averages; model
 * card, EMA bullet: an exponentially weighted average over the sequence of
 * globals, beta 0.9):
 *     ema[j] = beta * ema[j] + (1 - beta) * global[j]
 * with 1 - beta formed once in binary32.  out may be the same array as sum.
 */
void oracle_finalize_mean(float *out, const float *sum, int64_t n, int count,
                          float *ema, float beta)
{
    float N = (float)count;
    float one_minus_beta = 1.0f - beta;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float g = sum[j] / N;
        out[j] = g;
        if (ema)
            ema[j] = beta * ema[j] + one_minus_beta * g;
    }
}

/*
 * Fragment merge, folding step (GradientMail post, "Getting updates through
 * the bucket": each participant's delta is weighted by its token count and
 * the weighted deltas are averaged).
 *
 * For one participant's fragment snapshot c (n elements) taken against the
 * fragment's current global theta, with t tokens:
 *     d = theta[j] - c[j]        (the delta, pointing from the new weights
 *                                 back to the global: an outer gradient)
 *     p = fp32(t) * d
 *     acc[j] = p                  first arrival
 *     acc[j] = acc[j] + p         later arrivals, in arrival order
 * The int64 token count is rounded to binary32 once (nearest-even).
 */
void oracle_fold_delta(float *acc, const float *theta, const void *ckpt, int dtype,
                       int64_t n, int64_t tokens, int first)
{
    float w = (float)tokens;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float d = theta[j] - oracle_ckpt_value(ckpt, dtype, j);
        float p = w * d;
        if (first)
            acc[j] = p;
        else
            acc[j] = acc[j] + p;
    }
}

/*
 * Fragment merge, closing step (GradientMail post, "Getting updates through
 * the bucket": the averaged, token-weighted delta drives an outer
 * Nesterov step, learning rate 0.7, momentum 0.9).
 *
 * With W = fp32(sum of the participants' tokens):
 *     dbar  = acc[j] / W                  token-weighted mean delta
 *     m'    = mu * m[j] + dbar            momentum buffer
 *     u     = dbar + mu * m'              Nesterov look-ahead step
 *     theta'= theta[j] - lr * u
 * and, if ema is not NULL, ema[j] = beta * ema[j] + (1 - beta) * theta'.
 * With mu = 0 and lr = 1 this is theta - dbar, the checkpoints averaged with
 * token weights: plain parameter averaging (GradientMail post, "What might
 * explain the loss difference", second follow-up run).
 */
void oracle_outer_nesterov(float *theta, float *m, const float *acc, int64_t n,
                           int64_t total_tokens, float lr, float mu,
                           float *ema, float beta)
{
    float W = (float)total_tokens;
    float one_minus_beta = 1.0f - beta;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float dbar = acc[j] / W;
        float m_new = mu * m[j] + dbar;
        float u = dbar + mu * m_new;
        float theta_new = theta[j] - lr * u;
        m[j] = m_new;
        theta[j] = theta_new;
        if (ema)
            ema[j] = beta * ema[j] + one_minus_beta * theta_new;
    }
}

/*
 * EMA of globals on its own (technical report, Table 2, Side averages; model
 * card, EMA bullet): ema[j] = beta * ema[j] + (1 - beta) * g[j].
 */
void oracle_ema(float *ema, const float *g, int64_t n, float beta)
{
    float one_minus_beta = 1.0f - beta;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        ema[j] = beta * ema[j] + one_minus_beta * g[j];
}

/*
 * Keep-local-drift adoption on a worker (DiffuRefill-1B technical report,
 * section "What we measured", "Distributed optimisation": instead of
 * replacing its weights by the new global g, a worker keeps the progress it
 * made since its push; model card, "What the run taught").  With theta the
 * worker's current weights and pushed the checkpoint it pushed:
 *     theta[j] = theta[j] + (g[j] - pushed[j])
 * the difference formed first, then added (two roundings).  pushed is fp32
 * or bf16 (widened exactly).
 */
void oracle_adopt_keep_drift(float *theta, const float *g, const void *pushed, int dtype,
                             int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float shift = g[j] - oracle_ckpt_value(pushed, dtype, j);
        theta[j] = theta[j] + shift;
    }
}

/* Number of threads an OpenMP loop here would use (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

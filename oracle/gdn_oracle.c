/*
 * gdn_oracle.c -- plain float64 CPU oracle for one Gated DeltaNet layer's prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this file's library.  The product path (the HIP library under
 * hybrid_linear_attention_prefill_amd/) never includes, links or calls anything here, and
 * this file includes nothing from it.
 *
 * What it computes, in the order the method defines it, one token at a time, in float64:
 *
 *  1. A causal depthwise convolution of width W over the q|k|v channels whose state is the
 *     last W-1 conv *inputs* (the three most recent conv inputs are kept per linear-attention layer:
 *     PR "qwen3_5: run prompts that share prefixes once per prefix", section Purpose; the
 *     convolution state compared bit for bit on replay: "The shadow reader", section
 *     "Exact on a grid").  Tap W-1 multiplies the current token; no bias; SiLU optional.
 *  2. L2 normalisation of each q and k head vector: x / sqrt(sum x^2 + eps).
 *  3. The gated delta rule per value head h (key head h / (Hv/Hk)):
 *         S <- exp(g_t) * S
 *         e <- v_t - S^T k_t
 *         S <- S + beta_t * k_t e^T
 *         o_t <- scale * S^T q_t
 *     i.e. S_t = a_t (I - b_t k k^T) S_{t-1} + b_t k v^T with the output read after the
 *     update.  The pages name this recurrent state (a float32 "running sum" that cannot be
 *     cut back to an arbitrary position: "Long context and sessions", section Checkpoints)
 *     but print no equation for it; this is the standard gated delta rule, state laid out
 *     [d_k][d_v].
 *
 * Parity pins for every function here live in tests/test_oracle_*.py (closed forms,
 * brute force by explicit matrix products, numpy.convolve, invariants).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_k_heads, n_v_heads, d_k, d_v;
    int32_t conv_width; /* 0 = inputs already post-conv; else the kernel width (4) */
    int32_t conv_silu;  /* 1 = apply x*sigmoid(x) after the convolution */
    double scale, l2_eps;
} oracle_desc;

/* Step 1: causal depthwise conv with carried window.
 * x [T][C], w [C][W], window [W-1][C] (oldest row first) -> y [T][C], window_out [W-1][C].
 * xt = window ++ x; y[t][c] = sum_j w[c][j] * xt[t+j][c]; window_out = last W-1 rows of xt. */
void oracle_causal_conv(int64_t T, int32_t C, int32_t W, const double *x, const double *w,
                        const double *window, int32_t silu, double *y, double *window_out)
{
    const int32_t H = W - 1;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int32_t j = 0; j < W; ++j) {
                int64_t r = t + j;                   /* row in xt */
                double xv = (r < H) ? window[r * C + c] : x[(r - H) * C + c];
                acc += w[c * W + j] * xv;
            }
            if (silu) acc = acc / (1.0 + exp(-acc));
            y[t * C + c] = acc;
        }
    }
    if (window_out) {
        for (int32_t i = 0; i < H; ++i) {
            int64_t r = T + i;                       /* row in xt, xt has T+H rows */
            for (int32_t c = 0; c < C; ++c)
                window_out[i * C + c] = (r < H) ? window[r * C + c] : x[(r - H) * C + c];
        }
    }
}

/* Step 2: row-wise L2 normalisation, out = in / sqrt(sum in^2 + eps).  in/out may alias. */
void oracle_l2norm(int64_t n, int32_t d, const double *in, int64_t in_stride, double eps,
                   double *out, int64_t out_stride)
{
    for (int64_t r = 0; r < n; ++r) {
        double ss = 0.0;
        for (int32_t i = 0; i < d; ++i) ss += in[r * in_stride + i] * in[r * in_stride + i];
        double inv = 1.0 / sqrt(ss + eps);
        for (int32_t i = 0; i < d; ++i) out[r * out_stride + i] = in[r * in_stride + i] * inv;
    }
}

/* Step 3: the gated delta rule for one value head, token by token.
 * q,k rows of length dk at stride qk_stride; v rows of length dv at stride v_stride;
 * g, beta at stride gb_stride.  S [dk][dv] is updated in place; o rows at o_stride. */
void oracle_gdr_head(int64_t T, int32_t dk, int32_t dv, const double *q, const double *k,
                     int64_t qk_stride, const double *v, int64_t v_stride, const double *g,
                     const double *beta, int64_t gb_stride, double scale, double *S, double *o,
                     int64_t o_stride)
{
    double *e = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int64_t t = 0; t < T; ++t) {
        const double *qt = q + t * qk_stride, *kt = k + t * qk_stride, *vt = v + t * v_stride;
        const double a = exp(g[t * gb_stride]), b = beta[t * gb_stride];
        for (int32_t i = 0; i < dk * dv; ++i) S[i] *= a;
        for (int32_t j = 0; j < dv; ++j) {
            double s = 0.0;
            for (int32_t i = 0; i < dk; ++i) s += S[i * dv + j] * kt[i];
            e[j] = vt[j] - s;
        }
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dv; ++j) S[i * dv + j] += b * kt[i] * e[j];
        if (o) {
            double *ot = o + t * o_stride;
            for (int32_t j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int32_t i = 0; i < dk; ++i) s += S[i * dv + j] * qt[i];
                ot[j] = scale * s;
            }
        }
    }
    free(e);
}

typedef struct {
    const oracle_desc *d;
    int64_t T;
    const double *qn, *kn, *y;   /* normalised q, k [T][Hk*dk]; conv output y [T][C] */
    const double *g, *beta;      /* [T][Hv] */
    double *S;                   /* [Hv][dk][dv] */
    double *o;                   /* [T][Hv][dv] */
    const int32_t *heads;
    int32_t n_heads, next;
    pthread_mutex_t mu;
} layer_job;

static void *layer_worker(void *arg)
{
    layer_job *J = (layer_job *)arg;
    const oracle_desc *d = J->d;
    const int32_t C = 2 * d->n_k_heads * d->d_k + d->n_v_heads * d->d_v;
    const int32_t group = d->n_v_heads / d->n_k_heads;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int32_t i = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (i >= J->n_heads) break;
        const int32_t h = J->heads[i], kh = h / group;
        const double *v = J->y + 2 * d->n_k_heads * d->d_k + (int64_t)h * d->d_v;
        oracle_gdr_head(J->T, d->d_k, d->d_v, J->qn + (int64_t)kh * d->d_k,
                        J->kn + (int64_t)kh * d->d_k, (int64_t)d->n_k_heads * d->d_k, v, C,
                        J->g + h, J->beta + h, d->n_v_heads, d->scale,
                        J->S + (int64_t)h * d->d_k * d->d_v, J->o ? J->o + (int64_t)h * d->d_v : NULL,
                        (int64_t)d->n_v_heads * d->d_v);
    }
    return NULL;
}

/* One layer: conv (if conv_width > 0) -> L2 norm of q, k -> gated delta rule per value head.
 * x [T][C] with C = 2*Hk*dk + Hv*dv (q | k | v, each head's dims contiguous);
 * conv_w [C][W]; window_in / window_out [W-1][C]; g, beta [T][Hv];
 * S [Hv][dk][dv] holds S0 on entry and the final state on exit (only for the heads listed);
 * o [T][Hv][dv] (only the listed heads' columns are written; may be NULL).
 * heads: the value heads to run (NULL = all).  Returns 0, or -1 on bad arguments. */
int32_t oracle_gdn_layer(const oracle_desc *d, int64_t T, const double *x, const double *conv_w,
                         const double *window_in, const double *g, const double *beta, double *S,
                         double *o, double *window_out, const int32_t *heads, int32_t n_heads,
                         int32_t n_threads)
{
    if (!d || T < 0 || d->n_k_heads <= 0 || d->n_v_heads <= 0 || d->d_k <= 0 || d->d_v <= 0 ||
        d->n_v_heads % d->n_k_heads != 0 || d->conv_width < 0)
        return -1;
    const int32_t Hk = d->n_k_heads, dk = d->d_k;
    const int32_t C = 2 * Hk * dk + d->n_v_heads * d->d_v;
    double *y = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * C);
    double *qn = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * Hk * dk);
    double *kn = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * Hk * dk);
    if (!y || !qn || !kn) { free(y); free(qn); free(kn); return -2; }
    if (d->conv_width > 0) {
        oracle_causal_conv(T, C, d->conv_width, x, conv_w, window_in, d->conv_silu, y, window_out);
    } else {
        memcpy(y, x, sizeof(double) * (size_t)T * C);
    }
    for (int32_t h = 0; h < Hk; ++h) {
        oracle_l2norm(T, dk, y + (int64_t)h * dk, C, d->l2_eps, qn + (int64_t)h * dk, (int64_t)Hk * dk);
        oracle_l2norm(T, dk, y + (int64_t)(Hk + h) * dk, C, d->l2_eps, kn + (int64_t)h * dk,
                      (int64_t)Hk * dk);
    }
    int32_t *all = NULL;
    if (!heads) {
        all = (int32_t *)malloc(sizeof(int32_t) * (size_t)d->n_v_heads);
        for (int32_t h = 0; h < d->n_v_heads; ++h) all[h] = h;
        heads = all;
        n_heads = d->n_v_heads;
    }
    layer_job J = {d, T, qn, kn, y, g, beta, S, o, heads, n_heads, 0, PTHREAD_MUTEX_INITIALIZER};
    if (n_threads < 1) n_threads = 1;
    if (n_threads > n_heads) n_threads = n_heads > 0 ? n_heads : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    for (int32_t i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, layer_worker, &J);
    for (int32_t i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(all);
    free(y);
    free(qn);
    free(kn);
    return 0;
}

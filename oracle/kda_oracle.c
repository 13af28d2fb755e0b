/*
 * kda_oracle.c -- plain double-precision CPU evaluation of one Kimi Delta
 * Attention (KDA) decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the GPU library is
 * compared against.  It is called from the test suite, from the package's
 * smoke check and from the CPU-baseline leg of the benchmark, and from
 * nothing else.  It shares no code, header or constant with the HIP library.
 *
 * Every loop below is the definition written out, in the order and notation
 * of the sources it cites; nothing is blocked, fused or reordered.  All
 * arithmetic is IEEE double.  Inputs are BF16/FP32 values widened exactly to
 * double by the caller.
 *
 * Sources (web pages, cited by title and section):
 *  [DD]  "GLM-5.3 deep dive" (gangliao.me, 2026):
 *        8.2.2 (delta rule), 8.2.3 (KDA update, Eq. 1, the order of
 *        operations in fla's reference recurrence, and the forget gate as
 *        fla computes it), 8.2.4 (the full layer: short convolution with
 *        SiLU, split into heads, write strength, forget gate, L2
 *        normalisation, gated RMSNorm on the output; implementation notes:
 *        FusedRMSNormGated(128, eps 1e-5, sigmoid)), 8.2.6 (decoding: fade,
 *        predict, correct, read; epsilon 1e-6, q scale).
 *  [P1]  "At the 262k cap the DSA indexer costs 12x the sparse MLA it selects
 *        for", sections "Geometry" and "Bytes per stream" (depthwise conv,
 *        kernel 4, 3 cached taps, 3 tensors).
 *
 * Readings taken where the pages leave a step open (each is listed with its
 * reason in the design notes of the repository):
 *  - conv: cross-correlation with causal left padding, no bias; tap 3
 *    multiplies the current token, tap 0 the oldest cached token; the cached
 *    taps are raw pre-conv inputs;
 *  - L2 norm: x * 1/sqrt(sum x^2 + eps);
 *  - the q scale is an argument (1/sqrt(D) in fla's decode, 1 in Eq. 1);
 *  - gated RMSNorm: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(g), per head
 *    over its D outputs, from the unrounded o.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int kda_oracle_version(void) { return 2; }

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Short causal convolution (kernel 4) followed by SiLU, for one stream of C
 * independent channels.  [DD] 8.2.4 step 2; [P1] "Geometry".
 *
 *   y[c]  = w[c][0]*cs[0][c] + w[c][1]*cs[1][c] + w[c][2]*cs[2][c] + w[c][3]*x[c]
 *   z[c]  = SiLU(y[c]) = y[c] / (1 + exp(-y[c]))
 *   cs'   = (cs[1], cs[2], x)        (the three most recent raw inputs)
 *
 * Layouts: x[C], w[C][4], cs_in/cs_out[3][C] (tap 0 oldest), z[C].
 * cs_out may equal cs_in.
 */
void kda_oracle_conv_silu(int C, const double *x, const double *w,
                          const double *cs_in, double *cs_out, double *z)
{
    for (int c = 0; c < C; ++c) {
        double t0 = cs_in[0 * (size_t)C + c];
        double t1 = cs_in[1 * (size_t)C + c];
        double t2 = cs_in[2 * (size_t)C + c];
        double xc = x[c];
        double y = w[4 * (size_t)c + 0] * t0 + w[4 * (size_t)c + 1] * t1 +
                   w[4 * (size_t)c + 2] * t2 + w[4 * (size_t)c + 3] * xc;
        z[c] = y / (1.0 + exp(-y));
        cs_out[0 * (size_t)C + c] = t1;
        cs_out[1 * (size_t)C + c] = t2;
        cs_out[2 * (size_t)C + c] = xc;
    }
}

/*
 * L2 normalisation with epsilon, times a scale.  [DD] 8.2.4 step 6 and
 * 8.2.6 implementation notes (epsilon 1e-6; q is then scaled).
 *
 *   out = scale * x / sqrt(sum_i x_i^2 + eps)
 */
void kda_oracle_l2norm(int n, const double *x, double eps, double scale,
                       double *out)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; ++i)
        out[i] = scale * x[i] * r;
}

/*
 * One gated delta-rule step for one head.  [DD] 8.2.3 Eq. 1,
 *
 *   S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,   o = S_t^T q,
 *
 * evaluated in the decode order of [DD] 8.2.6 (fade, predict, correct, read),
 * which 8.2.3 states is the same update as Eq. 1.
 *
 * S is [dk][dv], row i = key channel (the one alpha fades), column j = value
 * channel.  q and k are used as given (already normalised and scaled).
 * S is updated in place; o[dv] is written.
 */
void kda_oracle_delta_step(int dk, int dv, double *S, const double *q,
                           const double *k, const double *v,
                           const double *alpha, double beta, double *o)
{
    /* 1. fade: row i of S times alpha_i */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] *= alpha[i];

    /* 2. predict: vhat = S^T k with the faded state;
     * 3. correct: S += k (beta (v - vhat))^T */
    double *d = (double *)malloc(sizeof(double) * (size_t)(dv > 0 ? dv : 1));
    for (int j = 0; j < dv; ++j) {
        double vhat = 0.0;
        for (int i = 0; i < dk; ++i)
            vhat += S[(size_t)i * dv + j] * k[i];
        d[j] = beta * (v[j] - vhat);
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] += k[i] * d[j];
    free(d);

    /* 4. read: o = S^T q with the new state */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i)
            acc += S[(size_t)i * dv + j] * q[i];
        o[j] = acc;
    }
}

/*
 * One full KDA decode step over M streams and H heads of width D.
 * [DD] 8.2.4 steps 2, 3 and 6, with 8.2.6's per-token order.
 *
 *   x      [M][3][H*D]     pre-conv q|k|v of this token
 *   w      [3*H*D][4]      depthwise conv weights (q, k, v channels in order)
 *   cs_in  [M][3][3*H*D]   conv state, tap 0 oldest; cs_out same (may alias)
 *   S      [M][H][D][D]    recurrent state, updated in place
 *   alpha  [M][H][D]       per key-channel decay
 *   beta   [M][H]          write strength
 *   o      [M][H][D]       output
 *
 * For each stream: conv + SiLU over all 3*H*D channels; split into heads;
 * k^ = l2norm(k), q^ = scale * l2norm(q); then the delta step per head.
 * Streams and heads are independent; OpenMP runs them in parallel.
 */
int kda_oracle_decode_step(int M, int H, int D, double *S, const double *x,
                           const double *w, const double *cs_in,
                           double *cs_out, const double *alpha,
                           const double *beta, double scale, double eps,
                           double *o)
{
    if (M < 0 || H < 1 || D < 1)
        return 1;
    const size_t HD = (size_t)H * D;
    const size_t C = 3 * HD;
    double *z = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * C);
    if (!z)
        return 2;

    int m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m)
        kda_oracle_conv_silu((int)C, x + (size_t)m * C, w,
                             cs_in + (size_t)m * 3 * C,
                             cs_out + (size_t)m * 3 * C, z + (size_t)m * C);

    long unit;
    const long units = (long)M * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (unit = 0; unit < units; ++unit) {
        int mm = (int)(unit / H), h = (int)(unit % H);
        const double *zq = z + (size_t)mm * C + 0 * HD + (size_t)h * D;
        const double *zk = z + (size_t)mm * C + 1 * HD + (size_t)h * D;
        const double *zv = z + (size_t)mm * C + 2 * HD + (size_t)h * D;
        double *qh = (double *)malloc(sizeof(double) * (size_t)D);
        double *kh = (double *)malloc(sizeof(double) * (size_t)D);
        kda_oracle_l2norm(D, zq, eps, scale, qh);
        kda_oracle_l2norm(D, zk, eps, 1.0, kh);
        size_t u = (size_t)mm * H + h;
        kda_oracle_delta_step(D, D, S + u * (size_t)D * D, qh, kh, zv,
                              alpha + u * (size_t)D, beta[u], o + u * (size_t)D);
        free(qh);
        free(kh);
    }
    free(z);
    return 0;
}

/*
 * The recurrent part alone, from post-conv (post-SiLU) q|k|v:
 *   qkv [M][3][H*D]; the rest as kda_oracle_decode_step.
 * [DD] 8.2.4 step 6 with 8.2.6's order.
 */
int kda_oracle_recurrent_step(int M, int H, int D, double *S,
                              const double *qkv, const double *alpha,
                              const double *beta, double scale, double eps,
                              double *o)
{
    if (M < 0 || H < 1 || D < 1)
        return 1;
    const size_t HD = (size_t)H * D;
    long unit;
    const long units = (long)M * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (unit = 0; unit < units; ++unit) {
        int mm = (int)(unit / H), h = (int)(unit % H);
        const double *zq = qkv + (size_t)mm * 3 * HD + 0 * HD + (size_t)h * D;
        const double *zk = qkv + (size_t)mm * 3 * HD + 1 * HD + (size_t)h * D;
        const double *zv = qkv + (size_t)mm * 3 * HD + 2 * HD + (size_t)h * D;
        double *qh = (double *)malloc(sizeof(double) * (size_t)D);
        double *kh = (double *)malloc(sizeof(double) * (size_t)D);
        kda_oracle_l2norm(D, zq, eps, scale, qh);
        kda_oracle_l2norm(D, zk, eps, 1.0, kh);
        size_t u = (size_t)mm * H + h;
        kda_oracle_delta_step(D, D, S + u * (size_t)D * D, qh, kh, zv,
                              alpha + u * (size_t)D, beta[u], o + u * (size_t)D);
        free(qh);
        free(kh);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gate, write strength and output norm around the recurrence.               */

static double sigmoid_d(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + exp(x)), written so that exp never overflows:
 * for x > 0, log(1 + e^x) = x + log(1 + e^-x). */
static double softplus_d(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/*
 * Forget gate of one head, [DD] 8.2.3 "The gate in GLM-5.3-Flash, as fla
 * computes it", for the D channels c of head h:
 *
 *   kind 0 (with a lower bound lb < 0, GLM-5.3-Flash: lb = -5):
 *       g_c = lb * sigmoid(exp(A_h) * (f_c + b_c))
 *   kind 1 (fla's default, no floor):
 *       g_c = -exp(A_h) * softplus(f_c + b_c)
 *   alpha_c = exp(g_c)
 *
 * f is the raw gate projection, A_h the head's A_log, b the head's dt_bias.
 */
void kda_oracle_gate(int D, const double *f, double A_log, const double *dt_bias,
                     int kind, double lower_bound, double *alpha)
{
    const double eA = exp(A_log);
    for (int c = 0; c < D; ++c) {
        const double xin = f[c] + dt_bias[c];
        const double g = kind == 0 ? lower_bound * sigmoid_d(eA * xin)
                                   : -eA * softplus_d(xin);
        alpha[c] = exp(g);
    }
}

/* Write strength, [DD] 8.2.4 step 4: beta = sigmoid(logit), one per head. */
void kda_oracle_beta(int n, const double *logit, double *beta)
{
    for (int i = 0; i < n; ++i)
        beta[i] = sigmoid_d(logit[i]);
}

/*
 * Gated RMSNorm of one head's outputs, [DD] 8.2.4 step 7 and implementation
 * notes (FusedRMSNormGated over head_dim 128, eps 1e-5, sigmoid gate):
 *
 *   y_j = o_j / sqrt((1/D) sum_i o_i^2 + eps) * w_j * sigmoid(g_j)
 */
void kda_oracle_gated_rmsnorm(int D, const double *o, const double *g,
                              const double *w, double eps, double *y)
{
    double ss = 0.0;
    for (int i = 0; i < D; ++i)
        ss += o[i] * o[i];
    const double r = 1.0 / sqrt(ss / D + eps);
    for (int j = 0; j < D; ++j)
        y[j] = o[j] * r * w[j] * sigmoid_d(g[j]);
}

/*
 * The decode step with its gate inputs in raw form ([DD] 8.2.4 steps 4 and
 * 5): alpha from the forget gate of every (stream, head), beta from its
 * logit, then kda_oracle_decode_step.
 *
 *   f       [M][H*D]  raw forget-gate projection
 *   A_log   [H]       per head
 *   dt_bias [H*D]     per head and channel
 *   blogit  [M][H]    write-strength logits
 */
int kda_oracle_decode_step_gated(int M, int H, int D, double *S, const double *x,
                                 const double *w, const double *cs_in,
                                 double *cs_out, const double *f,
                                 const double *A_log, const double *dt_bias,
                                 const double *blogit, int kind,
                                 double lower_bound, double scale, double eps,
                                 double *o)
{
    if (M < 0 || H < 1 || D < 1)
        return 1;
    const size_t units = (size_t)M * H;
    double *alpha = (double *)malloc(sizeof(double) * (units > 0 ? units : 1) * (size_t)D);
    double *beta = (double *)malloc(sizeof(double) * (units > 0 ? units : 1));
    if (!alpha || !beta) {
        free(alpha);
        free(beta);
        return 2;
    }
    for (size_t u = 0; u < units; ++u) {
        const size_t h = u % (size_t)H;
        kda_oracle_gate(D, f + u * (size_t)D, A_log[h], dt_bias + h * (size_t)D, kind,
                        lower_bound, alpha + u * (size_t)D);
    }
    kda_oracle_beta((int)units, blogit, beta);
    int rc = kda_oracle_decode_step(M, H, D, S, x, w, cs_in, cs_out, alpha, beta, scale, eps, o);
    free(alpha);
    free(beta);
    return rc;
}

/*
 * The layer's recurrent core for one token: the gated decode step above,
 * then the gated RMSNorm of every head's outputs ([DD] 8.2.4 steps 2-7 up
 * to the final projection).
 *
 *   og      [M][H*D]  output-gate projection
 *   norm_w  [D]       RMSNorm weight, shared by the heads
 *   y       [M][H][D] output
 */
int kda_oracle_layer_step(int M, int H, int D, double *S, const double *x,
                          const double *w, const double *cs_in, double *cs_out,
                          const double *f, const double *A_log,
                          const double *dt_bias, const double *blogit, int kind,
                          double lower_bound, double scale, double eps,
                          const double *og, const double *norm_w, double norm_eps,
                          double *y)
{
    const size_t units = (size_t)(M > 0 ? M : 0) * (size_t)(H > 0 ? H : 0);
    double *o = (double *)malloc(sizeof(double) * (units > 0 ? units : 1) * (size_t)(D > 0 ? D : 1));
    if (!o)
        return 2;
    int rc = kda_oracle_decode_step_gated(M, H, D, S, x, w, cs_in, cs_out, f, A_log, dt_bias,
                                          blogit, kind, lower_bound, scale, eps, o);
    if (rc == 0)
        for (size_t u = 0; u < units; ++u)
            kda_oracle_gated_rmsnorm(D, o + u * (size_t)D, og + u * (size_t)D, norm_w, norm_eps,
                                     y + u * (size_t)D);
    free(o);
    return rc;
}

/*
 * T consecutive tokens of M streams in one call, [DD] 8.2.6 (fla's decode
 * mode loops over the tokens of an input of at most 64 tokens): token t of
 * every stream goes through kda_oracle_decode_step with the state and conv
 * state left by token t - 1.
 *
 *   x      [M][T][3][H*D]   alpha [M][T][H][D]   beta [M][T][H]
 *   o      [M][T][H][D]     S, w, cs_in, cs_out as kda_oracle_decode_step
 */
int kda_oracle_decode_multi(int T, int M, int H, int D, double *S, const double *x,
                            const double *w, const double *cs_in, double *cs_out,
                            const double *alpha, const double *beta, double scale,
                            double eps, double *o)
{
    if (T < 0 || M < 0 || H < 1 || D < 1)
        return 1;
    const size_t HD = (size_t)H * D, C = 3 * HD;
    if (cs_out != cs_in)
        memcpy(cs_out, cs_in, sizeof(double) * (size_t)M * 3 * C);
    double *xt = (double *)malloc(sizeof(double) * C);
    double *at = (double *)malloc(sizeof(double) * HD);
    double *bt = (double *)malloc(sizeof(double) * (size_t)H);
    double *ot = (double *)malloc(sizeof(double) * HD);
    if (!xt || !at || !bt || !ot) {
        free(xt); free(at); free(bt); free(ot);
        return 2;
    }
    int rc = 0;
    for (int m = 0; m < M && rc == 0; ++m) {
        double *Sm = S + (size_t)m * H * D * D;
        double *cm = cs_out + (size_t)m * 3 * C;
        for (int t = 0; t < T && rc == 0; ++t) {
            const size_t mt = (size_t)m * T + t;
            memcpy(xt, x + mt * C, sizeof(double) * C);
            memcpy(at, alpha + mt * HD, sizeof(double) * HD);
            memcpy(bt, beta + mt * H, sizeof(double) * (size_t)H);
            rc = kda_oracle_decode_step(1, H, D, Sm, xt, w, cm, cm, at, bt, scale, eps, ot);
            memcpy(o + mt * HD, ot, sizeof(double) * HD);
        }
    }
    free(xt); free(at); free(bt); free(ot);
    return rc;
}

/*
 * T consecutive tokens of M streams with raw gate inputs: token t of every
 * stream goes through kda_oracle_decode_step_gated with the state and conv
 * state left by token t - 1 ([DD] 8.2.4 steps 2-6 over a sequence; 8.2.5
 * computes the same recurrence chunk by chunk).
 *
 *   x [M][T][3][H*D]   f [M][T][H*D]   blogit [M][T][H]   o [M][T][H][D]
 *   A_log [H], dt_bias [H*D]; the rest as kda_oracle_decode_step_gated.
 */
int kda_oracle_sequence_gated(int T, int M, int H, int D, double *S, const double *x,
                              const double *w, const double *cs_in, double *cs_out,
                              const double *f, const double *A_log, const double *dt_bias,
                              const double *blogit, int kind, double lower_bound, double scale,
                              double eps, double *o)
{
    if (T < 0 || M < 0 || H < 1 || D < 1)
        return 1;
    const size_t HD = (size_t)H * D, C = 3 * HD;
    if (cs_out != cs_in)
        memcpy(cs_out, cs_in, sizeof(double) * (size_t)M * 3 * C);
    int rc = 0;
    for (int m = 0; m < M && rc == 0; ++m) {
        double *Sm = S + (size_t)m * H * D * D;
        double *cm = cs_out + (size_t)m * 3 * C;
        for (int t = 0; t < T && rc == 0; ++t) {
            const size_t mt = (size_t)m * T + t;
            rc = kda_oracle_decode_step_gated(1, H, D, Sm, x + mt * C, w, cm, cm, f + mt * HD, A_log,
                                              dt_bias, blogit + mt * H, kind, lower_bound, scale,
                                              eps, o + mt * HD);
        }
    }
    return rc;
}

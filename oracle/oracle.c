/*
 * fp64 CPU oracle for the selective-SSM scan and the scalar-A (SSD) form.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The HIP product path never
 * links, calls or includes anything from this directory, and this file shares
 * no code, header or table with it.
 *
 * What it computes is the plain definition: a per-timestep linear recurrence
 * run in double precision, one channel at a time, exactly in the order the
 * pages write it. No chunking, no blocking, no reassociation.
 *
 * Pages cited (titles as published; sections named as on the page):
 *   [Mamba-2 page]  "Mamba-2：把状态空间模型和 Attention 统一到一个数学框架里"
 *                   aiplusplus.yigather.com/tech/05-27a2ce5d
 *   [SSM page]      "状态空间模型与 Mamba：不用注意力读取长序列的方法"
 *                   ai-trend.me/zh/study/state-space-models/
 *   [Juejin page]   SSM/Mamba engineering article, juejin.cn/post/7634002571020402707
 *   [Reading page]  "论文解读：Mamba — 线性时间的序列建模革命"  agent.eake.cn
 *   [Hybrid page]   "基础知识：Mamba 与混合 SSM 架构"  charles2530.github.io
 *
 * Definition (per channel, state h in R^N, all arithmetic in double):
 *   v_t    = delta_raw_t + bias                    (bias placement: a reading)
 *   dt_t   = softplus(v_t) = log(1 + e^{v_t})      [Mamba-2 page, Core idea step 1;
 *                                                    Reading page section 3]
 *   Abar   = exp(dt_t * A[n])   (diagonal A)       [Mamba-2 page, step 1: A is
 *                                                    discretised through Delta]
 *   Bbar x = dt_t * B_t[n] * x_t                   (Euler form for B: a reading)
 *   h_t[n] = Abar * h_{t-1}[n] + Bbar x            [Mamba-2 page, Background, the
 *                                                    discrete recurrence; Reading
 *                                                    page section 2; Hybrid page section 2]
 *   y_t    = sum_n C_t[n] h_t[n] + Dskip * x_t     [Juejin page, "基本原理": output
 *                                                    equation with the D x term]
 *   out_t  = y_t * silu(z_t) = y_t * z_t / (1 + e^{-z_t})
 *                                                  [Reading page section 5, Hybrid
 *                                                    page section 3: the SSM output is
 *                                                    multiplied by the SiLU of the z branch]
 *   h_final = h_L (before the gate)                [Juejin page, streaming step(x, state)]
 * Each input channel carries its own N-dim state [SSM page, "工作原理"].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Stable two-branch softplus; log1p keeps full relative precision when the
 * step is small (dt down to 1e-4 and below). */
static double softplus_f64(double v)
{
    return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
}

static double silu_gate_f64(double z)
{
    return z / (1.0 + exp(-z));
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Selective scan, Mamba-1 form.
 *   x, delta, z : (batch, L, D)  row-major, D fastest (float32 storage values)
 *   Bm, Cm      : (batch, L, G, N)  G groups; channel d reads group d / (D / G)
 *                 (G = 1: one group shared by all D channels) [the pages' B_t,
 *                 C_t are functions of the token; grouping channels so that each
 *                 group has its own B, C is the multi-group variant]
 *   A           : (D, N)
 *   delta_bias, Dskip : (D)  (NULL -> 0)
 *   z           : NULL -> no gate
 *   h0          : (batch, D, N) double, NULL -> zero initial state (double so
 *                 that a state handed over from an earlier call is exact)
 *   delta_softplus : 1 -> dt = softplus(delta + bias); 0 -> dt = delta + bias
 *   chans/nchan : channel ids c = b*D + d to evaluate; chans == NULL -> all
 *                 B*D channels.
 * Outputs (double):
 *   chans == NULL:  y (batch, L, D), h_final (batch, D, N)
 *   chans != NULL:  y (nchan, L),    h_final (nchan, N)
 *   h_final may be NULL.
 * Returns 0, or -1 on a bad size.
 */
int oracle_selective_scan_f64(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t G,
                              const float *x, const float *delta, const float *z,
                              const float *Bm, const float *Cm, const float *A,
                              const float *delta_bias, const float *Dskip,
                              const double *h0, int delta_softplus,
                              const int64_t *chans, int64_t nchan,
                              double *y, double *h_final)
{
    if (batch < 0 || L < 0 || D <= 0 || N <= 0 || N > 4096 || G <= 0 || D % G) return -1;
    const int64_t total = chans ? nchan : batch * D;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < total; ++i) {
        const int64_t c = chans ? chans[i] : i;
        if (c < 0 || c >= batch * D) { bad = 1; continue; }
        const int64_t b = c / D, d = c % D;
        const int64_t g = d / (D / G);                  /* B, C group of this channel */
        double h[4096];
        for (int64_t n = 0; n < N; ++n)
            h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        const double bias = delta_bias ? (double)delta_bias[d] : 0.0;
        const double dsk = Dskip ? (double)Dskip[d] : 0.0;

        for (int64_t t = 0; t < L; ++t) {
            const int64_t e = (b * L + t) * D + d;      /* (b, t, d) */
            const int64_t r = ((b * L + t) * G + g) * N;  /* (b, t, g, :) */
            const double xv = (double)x[e];
            const double v = (double)delta[e] + bias;
            const double dt = delta_softplus ? softplus_f64(v) : v;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dt * (double)A[d * N + n]);
                const double bx = dt * (double)Bm[r + n] * xv;
                h[n] = abar * h[n] + bx;
                acc += (double)Cm[r + n] * h[n];
            }
            double out = acc + dsk * xv;
            if (z) out *= silu_gate_f64((double)z[e]);
            if (chans) y[i * L + t] = out;
            else y[e] = out;
        }
        if (h_final) {
            double *hf = chans ? h_final + i * N : h_final + (b * D + d) * N;
            for (int64_t n = 0; n < N; ++n) hf[n] = h[n];
        }
    }
    return bad ? -1 : 0;
}

/*
 * Scalar-A form (Mamba-2 / SSD): heads of P channels share one step size and
 * one scalar decay A_h; every channel still runs its own N-dim recurrence.
 * [Mamba-2 page, key point 3: selectivity restricted so the mixing matrix stays
 * semiseparable; read here as one scalar A per head.]
 *   x, z   : (batch, L, H, P)     z NULL -> no gate
 *   dt     : (batch, L, H) raw    dt_bias (H) NULL -> 0
 *   A      : (H)                  Dskip (H) NULL -> 0
 *   Bm, Cm : (batch, L, G, N)     head h reads group h / (H / G)
 *   h0     : (batch, H, P, N) double, NULL -> zero
 *   chans  : ids c = (b*H + h)*P + p; NULL -> all
 * Outputs: chans == NULL: y (batch, L, H, P), h_final (batch, H, P, N);
 *          otherwise y (nchan, L), h_final (nchan, N).
 * This is the same recurrence as above with the step shared across a head; it
 * is written out separately in the SSD layout rather than by broadcasting.
 */
int oracle_ssd_f64(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                   const float *x, const float *dt_raw, const float *dt_bias,
                   const float *A, const float *Bm, const float *Cm,
                   const float *Dskip, const float *z, const double *h0,
                   int dt_softplus, const int64_t *chans, int64_t nchan,
                   double *y, double *h_final)
{
    if (batch < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || N > 4096 || G <= 0 || H % G) return -1;
    const int64_t total = chans ? nchan : batch * H * P;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < total; ++i) {
        const int64_t c = chans ? chans[i] : i;
        if (c < 0 || c >= batch * H * P) { bad = 1; continue; }
        const int64_t b = c / (H * P), hh = (c / P) % H, p = c % P;
        const int64_t g = hh / (H / G);
        double h[4096];
        for (int64_t n = 0; n < N; ++n)
            h[n] = h0 ? h0[c * N + n] : 0.0;
        const double bias = dt_bias ? (double)dt_bias[hh] : 0.0;
        const double dsk = Dskip ? (double)Dskip[hh] : 0.0;
        const double a = (double)A[hh];

        for (int64_t t = 0; t < L; ++t) {
            const int64_t e = ((b * L + t) * H + hh) * P + p;   /* (b, t, h, p) */
            const int64_t r = ((b * L + t) * G + g) * N;
            const double xv = (double)x[e];
            const double v = (double)dt_raw[(b * L + t) * H + hh] + bias;
            const double dtv = dt_softplus ? softplus_f64(v) : v;
            const double abar = exp(dtv * a);
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                h[n] = abar * h[n] + dtv * (double)Bm[r + n] * xv;
                acc += (double)Cm[r + n] * h[n];
            }
            double out = acc + dsk * xv;
            if (z) out *= silu_gate_f64((double)z[e]);
            if (chans) y[i * L + t] = out;
            else y[e] = out;
        }
        if (h_final) {
            double *hf = h_final + (chans ? i : c) * N;
            for (int64_t n = 0; n < N; ++n) hf[n] = h[n];
        }
    }
    return bad ? -1 : 0;
}

/*
 * Causal depthwise convolution along time followed by SiLU, fp64.
 * [Reading page section 5 and Hybrid page section 3: the x branch passes a
 * short depthwise Conv1d and SiLU before the scan; Juejin page "基本使用":
 * kernel width d_conv = 4; Juejin page, streaming step(x, state): a call may
 * continue from the history an earlier call left.]
 *   x: (batch, L, D); w: (D, K); bias: (D) NULL -> 0; out (batch, L, D)
 *   x0: (batch, K-1, D) the K-1 inputs before t = 0, oldest first; NULL -> zeros
 *   With xx = [x0 ; x] along time (xx_s = x0[K-1+s] for -(K-1) <= s < 0):
 *   out[b,t,d] = silu( bias[d] + sum_{k=0}^{K-1} w[d,k] * xx[b, t-(K-1)+k, d] ).
 *   apply_silu = 0 leaves the convolution output ungated.
 *   final_state (batch, K-1, D), NULL -> not written: the last K-1 entries of xx,
 *   which is the x0 of a call that continues this sequence.
 */
static double conv_input(const float *x, const float *x0, int64_t b, int64_t s, int64_t L,
                         int64_t D, int64_t K, int64_t d)
{
    if (s >= 0) return (double)x[(b * L + s) * D + d];
    if (x0 && s >= -(K - 1)) return (double)x0[(b * (K - 1) + (K - 1) + s) * D + d];
    return 0.0;
}

int oracle_causal_conv1d_f64(int64_t batch, int64_t L, int64_t D, int64_t K,
                             const float *x, const float *w, const float *bias,
                             const float *x0, int apply_silu, double *out, double *final_state)
{
    if (batch < 0 || L < 0 || D <= 0 || K <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < batch * D; ++c) {
        const int64_t b = c / D, d = c % D;
        for (int64_t t = 0; t < L; ++t) {
            double acc = bias ? (double)bias[d] : 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t s = t - (K - 1) + k;
                acc += (double)w[d * K + k] * conv_input(x, x0, b, s, L, D, K, d);
            }
            out[(b * L + t) * D + d] = apply_silu ? silu_gate_f64(acc) : acc;
        }
        if (final_state) {
            for (int64_t j = 0; j < K - 1; ++j)
                final_state[(b * (K - 1) + j) * D + d] = conv_input(x, x0, b, L - (K - 1) + j, L, D, K, d);
        }
    }
    return 0;
}

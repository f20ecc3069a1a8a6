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
#include <stdlib.h>
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

static int oracle_num_threads_in_team(void)
{
#ifdef _OPENMP
    return omp_get_num_threads();
#else
    return 1;
#endif
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

/*
 * Gradients of the selective scan (the training pass: the pages note that
 * training runs the same scan, [Mamba-2 page, Core idea: Mamba-1's scan and
 * training throughput]). Reverse-mode differentiation of the recurrence above,
 * per channel, in fp64, with the loss L = sum dy * y + sum dh_final * h_final:
 *   dyc_t  = dy_t * silu(z_t)                      (dyc_t = dy_t without a gate)
 *   g_t    = C_t[n] dyc_t + abar_{t+1}[n] g_{t+1}[n]   (adjoint of h_t; the last step
 *            adds dh_final instead of the term from t+1)
 *   dC_t[n] += dyc_t h_t[n],  dB_t[n] += g_t[n] dt_t x_t      (summed over the
 *            channels of the group)
 *   dx_t   = dyc_t Dskip + dt_t sum_n g_t[n] B_t[n]
 *   ddt_t  = sum_n g_t[n] (B_t[n] x_t + A[n] abar_t[n] h_{t-1}[n])
 *   ddelta_t = ddt_t * sigmoid(v_t) (softplus) or ddt_t;  dbias += ddelta_t
 *   dA[n] += g_t[n] dt_t abar_t[n] h_{t-1}[n];  dDskip += dyc_t x_t
 *   dz_t   = dy_t (C_t.h_t + Dskip x_t) silu'(z_t),  silu' = s (1 + z (1 - s))
 *   dh0[n] = abar_0[n] g_0[n]
 * Inputs as oracle_selective_scan_f64 (h0 and dh_final double, NULL -> 0).
 * Outputs (double, all required except dz when z is NULL): dx, ddelta, dz
 * (batch, L, D); dB, dC (batch, L, G, N); dA (D, N); dDskip, dbias (D);
 * dh0 (batch, D, N). Returns 0, or -1 on a bad size.
 */
int oracle_selective_scan_bwd_f64(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t G,
                                  const float *x, const float *delta, const float *z,
                                  const float *Bm, const float *Cm, const float *A,
                                  const float *delta_bias, const float *Dskip,
                                  const double *h0, int delta_softplus,
                                  const float *dy, const double *dh_final,
                                  double *dx, double *ddelta, double *dz, double *dB, double *dC,
                                  double *dA, double *dDskip, double *dbias, double *dh0)
{
    if (batch < 0 || L < 0 || D <= 0 || N <= 0 || N > 4096 || G <= 0 || D % G) return -1;
    const int64_t nbc = batch * L * G * N;
    for (int64_t i = 0; i < nbc; ++i) { dB[i] = 0.0; dC[i] = 0.0; }
    for (int64_t i = 0; i < D * N; ++i) dA[i] = 0.0;
    for (int64_t i = 0; i < D; ++i) { dDskip[i] = 0.0; dbias[i] = 0.0; }

#pragma omp parallel
    {
        /* per-thread sums over channels, added in thread order at the end */
        double *pB = (double *)calloc((size_t)nbc, sizeof(double));
        double *pC = (double *)calloc((size_t)nbc, sizeof(double));
        double *hs = (double *)malloc((size_t)(L + 1) * (size_t)N * sizeof(double));
        double *dts = (double *)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
        double g[4096];

#pragma omp for schedule(static)
        for (int64_t d = 0; d < D; ++d) {
            const int64_t grp = d / (D / G);
            const double bias = delta_bias ? (double)delta_bias[d] : 0.0;
            const double dsk = Dskip ? (double)Dskip[d] : 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                /* forward: hs[t+1] = h_t, hs[0] = h_{-1} = h0 */
                for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t e = (b * L + t) * D + d;
                    const int64_t r = ((b * L + t) * G + grp) * N;
                    const double v = (double)delta[e] + bias;
                    const double dt = delta_softplus ? softplus_f64(v) : v;
                    dts[t] = dt;
                    for (int64_t n = 0; n < N; ++n) {
                        const double abar = exp(dt * (double)A[d * N + n]);
                        hs[(t + 1) * N + n] = abar * hs[t * N + n] + dt * (double)Bm[r + n] * (double)x[e];
                    }
                }
                /* reverse */
                for (int64_t n = 0; n < N; ++n) g[n] = dh_final ? dh_final[(b * D + d) * N + n] : 0.0;
                for (int64_t t = L - 1; t >= 0; --t) {
                    const int64_t e = (b * L + t) * D + d;
                    const int64_t r = ((b * L + t) * G + grp) * N;
                    const double xv = (double)x[e], dt = dts[t];
                    const double v = (double)delta[e] + bias;
                    double yc = dsk * xv;
                    for (int64_t n = 0; n < N; ++n) yc += (double)Cm[r + n] * hs[(t + 1) * N + n];
                    double gate = 1.0, dyc = (double)dy[e];
                    if (z) {
                        const double zv = (double)z[e], s = 1.0 / (1.0 + exp(-zv));
                        gate = zv * s;
                        dz[e] = (double)dy[e] * yc * s * (1.0 + zv * (1.0 - s));
                        dyc = (double)dy[e] * gate;
                    }
                    double gB = 0.0, ddt = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        const double abar = exp(dt * (double)A[d * N + n]);
                        const double gn = (double)Cm[r + n] * dyc + g[n];   /* g_t; g[n] held the term from t+1 */
                        const double hprev = hs[t * N + n];
                        pC[r + n] += dyc * hs[(t + 1) * N + n];
                        pB[r + n] += gn * dt * xv;
                        gB += gn * (double)Bm[r + n];
                        ddt += gn * ((double)Bm[r + n] * xv + (double)A[d * N + n] * abar * hprev);
                        dA[d * N + n] += gn * dt * abar * hprev;   /* channel d is this thread's */
                        g[n] = abar * gn;                                  /* term for t-1 */
                    }
                    dx[e] = dyc * dsk + dt * gB;
                    const double dd = delta_softplus ? ddt / (1.0 + exp(-v)) : ddt;
                    ddelta[e] = dd;
                    dbias[d] += dd;
                    dDskip[d] += dyc * xv;
                }
                for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = g[n];
            }
        }
#pragma omp for ordered schedule(static, 1)
        for (int th = 0; th < oracle_num_threads_in_team(); ++th) {
#pragma omp ordered
            for (int64_t i = 0; i < nbc; ++i) { dB[i] += pB[i]; dC[i] += pC[i]; }
        }
        free(pB); free(pC); free(hs); free(dts);
    }
    return 0;
}

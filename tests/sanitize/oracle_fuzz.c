/*
 * Address/undefined-behaviour sanitizer run of the fp64 oracle (CPU only).
 * Every buffer is allocated at exactly the size the oracle's contract gives it,
 * so a read or write past any of them is reported; sizes include the empty and
 * one-step cases, several groups, channel subsets and absent optional inputs.
 * Exit status 0 when every call returned its documented status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_selective_scan_f64(int64_t, int64_t, int64_t, int64_t, int64_t, const float *,
                              const float *, const float *, const float *, const float *,
                              const float *, const float *, const float *, const double *, int,
                              const int64_t *, int64_t, double *, double *);
int oracle_ssd_f64(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const float *,
                   const float *, const float *, const float *, const float *, const float *,
                   const float *, const float *, const double *, int, const int64_t *, int64_t,
                   double *, double *);
int oracle_causal_conv1d_f64(int64_t, int64_t, int64_t, int64_t, const float *, const float *,
                             const float *, const float *, int, double *, double *);
int oracle_selective_scan_bwd_f64(int64_t, int64_t, int64_t, int64_t, int64_t, const float *,
                                  const float *, const float *, const float *, const float *,
                                  const float *, const float *, const float *, const double *,
                                  int, const float *, const double *, double *, double *,
                                  double *, double *, double *, double *, double *, double *,
                                  double *);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33);
}
static float *fbuf(int64_t n) {
    float *p = malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) p[i] = ((float)(rnd() % 2001) - 1000.0f) / 1000.0f;
    return p;
}
static double *dbuf(int64_t n) {
    double *p = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = ((double)(rnd() % 2001) - 1000.0) / 1000.0;
    return p;
}
static int coin(void) { return rnd() & 1; }

static int fails = 0;
#define EXPECT(cond, what) do { if (!(cond)) { fprintf(stderr, "FAIL: %s\n", what); ++fails; } } while (0)

static void scan_case(int64_t B, int64_t L, int64_t D, int64_t N, int64_t G) {
    float *x = fbuf(B * L * D), *dl = fbuf(B * L * D), *z = fbuf(B * L * D);
    float *Bm = fbuf(B * L * G * N), *Cm = fbuf(B * L * G * N), *A = fbuf(D * N);
    for (int64_t i = 0; i < D * N; ++i) A[i] = -1.0f - (float)(i % N);
    float *bias = fbuf(D), *dsk = fbuf(D);
    double *h0 = dbuf(B * D * N);
    const int opt = (int)(rnd() % 16);
    const float *zp = (opt & 1) ? z : NULL, *bp = (opt & 2) ? bias : NULL, *dp = (opt & 4) ? dsk : NULL;
    const double *hp = (opt & 8) ? h0 : NULL;
    double *y = dbuf(B * L * D), *hf = dbuf(B * D * N);
    EXPECT(oracle_selective_scan_f64(B, L, D, N, G, x, dl, zp, Bm, Cm, A, bp, dp, hp, coin(), NULL, 0,
                                     y, coin() ? hf : NULL) == 0, "scan");
    /* a channel subset, in arbitrary order */
    int64_t nch = B * D > 0 ? 1 + (int64_t)(rnd() % (uint32_t)(B * D)) : 0;
    int64_t *ch = malloc((size_t)(nch > 0 ? nch : 1) * sizeof(int64_t));
    for (int64_t i = 0; i < nch; ++i) ch[i] = (int64_t)(rnd() % (uint32_t)(B * D));
    double *ys = dbuf(nch * L), *hs = dbuf(nch * N);
    if (nch) EXPECT(oracle_selective_scan_f64(B, L, D, N, G, x, dl, zp, Bm, Cm, A, bp, dp, hp, 1, ch, nch,
                                              ys, hs) == 0, "scan channels");
    /* gradients (all outputs required except dz without z) */
    float *dy = fbuf(B * L * D);
    double *dhf = dbuf(B * D * N);
    double *dx = dbuf(B * L * D), *ddl = dbuf(B * L * D), *dz = dbuf(B * L * D);
    double *dB = dbuf(B * L * G * N), *dC = dbuf(B * L * G * N), *dA = dbuf(D * N);
    double *dD = dbuf(D), *db = dbuf(D), *dh0 = dbuf(B * D * N);
    EXPECT(oracle_selective_scan_bwd_f64(B, L, D, N, G, x, dl, zp, Bm, Cm, A, bp, dp, hp, coin(), dy,
                                         coin() ? dhf : NULL, dx, ddl, zp ? dz : NULL, dB, dC, dA, dD,
                                         db, dh0) == 0, "scan bwd");
    free(x); free(dl); free(z); free(Bm); free(Cm); free(A); free(bias); free(dsk); free(h0);
    free(y); free(hf); free(ch); free(ys); free(hs); free(dy); free(dhf); free(dx); free(ddl);
    free(dz); free(dB); free(dC); free(dA); free(dD); free(db); free(dh0);
}

static void ssd_case(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G) {
    float *x = fbuf(B * L * H * P), *dt = fbuf(B * L * H), *z = fbuf(B * L * H * P);
    float *Bm = fbuf(B * L * G * N), *Cm = fbuf(B * L * G * N), *A = fbuf(H);
    for (int64_t h = 0; h < H; ++h) A[h] = -1.0f - (float)h;
    float *bias = fbuf(H), *dsk = fbuf(H);
    double *h0 = dbuf(B * H * P * N);
    const int opt = (int)(rnd() % 16);
    double *y = dbuf(B * L * H * P), *hf = dbuf(B * H * P * N);
    EXPECT(oracle_ssd_f64(B, L, H, P, N, G, x, dt, (opt & 2) ? bias : NULL, A, Bm, Cm,
                          (opt & 4) ? dsk : NULL, (opt & 1) ? z : NULL, (opt & 8) ? h0 : NULL, coin(),
                          NULL, 0, y, coin() ? hf : NULL) == 0, "ssd");
    int64_t total = B * H * P;
    int64_t nch = total > 0 ? 1 + (int64_t)(rnd() % (uint32_t)total) : 0;
    int64_t *ch = malloc((size_t)(nch > 0 ? nch : 1) * sizeof(int64_t));
    for (int64_t i = 0; i < nch; ++i) ch[i] = (int64_t)(rnd() % (uint32_t)total);
    double *ys = dbuf(nch * L), *hs = dbuf(nch * N);
    if (nch) EXPECT(oracle_ssd_f64(B, L, H, P, N, G, x, dt, bias, A, Bm, Cm, dsk, z, h0, 1, ch, nch, ys,
                                   hs) == 0, "ssd channels");
    free(x); free(dt); free(z); free(Bm); free(Cm); free(A); free(bias); free(dsk); free(h0);
    free(y); free(hf); free(ch); free(ys); free(hs);
}

static void conv_case(int64_t B, int64_t L, int64_t D, int64_t K) {
    float *x = fbuf(B * L * D), *w = fbuf(D * K), *bias = fbuf(D), *x0 = fbuf(B * (K - 1) * D);
    double *out = dbuf(B * L * D), *fs = dbuf(B * (K - 1) * D);
    EXPECT(oracle_causal_conv1d_f64(B, L, D, K, x, w, coin() ? bias : NULL, coin() ? x0 : NULL, coin(),
                                    out, coin() ? fs : NULL) == 0, "conv");
    free(x); free(w); free(bias); free(x0); free(out); free(fs);
}

int main(void) {
    /* fixed edge cases */
    scan_case(1, 0, 1, 1, 1);
    scan_case(0, 5, 4, 2, 1);
    scan_case(1, 1, 1, 1, 1);
    scan_case(2, 3, 6, 4, 3);
    ssd_case(1, 0, 2, 3, 2, 1);
    ssd_case(2, 1, 4, 2, 3, 2);
    conv_case(1, 0, 3, 4);
    conv_case(2, 1, 3, 4);
    conv_case(1, 2, 5, 4);
    /* rejected sizes */
    EXPECT(oracle_selective_scan_f64(1, 1, 4, 2, 3, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                     NULL, 1, NULL, 0, NULL, NULL) == -1, "scan: G must divide D");
    EXPECT(oracle_selective_scan_f64(1, 1, 4, 5000, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                     NULL, 1, NULL, 0, NULL, NULL) == -1, "scan: N too large");
    EXPECT(oracle_ssd_f64(1, 1, 3, 2, 2, 2, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1,
                          NULL, 0, NULL, NULL) == -1, "ssd: G must divide H");
    EXPECT(oracle_causal_conv1d_f64(1, 1, 0, 4, NULL, NULL, NULL, NULL, 1, NULL, NULL) == -1, "conv: D");
    /* random small shapes */
    for (int it = 0; it < 300; ++it) {
        const int64_t G = 1 + rnd() % 3;
        scan_case(rnd() % 3, rnd() % 20, G * (1 + rnd() % 5), 1 + rnd() % 6, G);
        const int64_t Gs = 1 + rnd() % 2;
        ssd_case(rnd() % 3, rnd() % 12, Gs * (1 + rnd() % 3), 1 + rnd() % 4, 1 + rnd() % 5, Gs);
        conv_case(rnd() % 3, rnd() % 9, 1 + rnd() % 7, 1 + rnd() % 4);
    }
    if (fails) { fprintf(stderr, "%d failures\n", fails); return 1; }
    printf("oracle sanitizer run: ok\n");
    return 0;
}

/*
 * oracle_drive.c -- test driver that runs every entry point of the C oracle
 * (oracle/mssm_oracle.c) on small seeded inputs, including the edge cases:
 * zero lengths, an empty batch, one state, optional pointers left NULL, more
 * threads than channels.  Built by tests/test_oracle_sanitized.py with
 * AddressSanitizer + UndefinedBehaviorSanitizer (and separately with
 * ThreadSanitizer) on the host; any finding aborts the run.
 *
 * It also checks two identities the oracle must satisfy whatever the build:
 * the scan equals L single decode steps, and the SSD on heads equals the S6
 * scan with the head's scalar A broadcast over the states.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_s6_scan(const double *u, const double *delta, const double *A, const double *Bm, const double *Cm,
                   const double *Dskip, const double *z, const double *h0, double *y, double *hT, long batch,
                   long d_inner, long seqlen, long d_state, int nthreads);
int oracle_s6_scan_zoh(const double *u, const double *delta, const double *A, const double *Bm, const double *Cm,
                       const double *Dskip, const double *z, const double *h0, double *y, double *hT, long batch,
                       long d_inner, long seqlen, long d_state, int nthreads);
int oracle_state_update(double *state, const double *u, const double *delta, const double *A, const double *Bm,
                        const double *Cm, const double *Dskip, const double *z, double *y, long batch,
                        long d_inner, long d_state, int nthreads);
int oracle_ssd(const double *x, const double *dt, const double *A, const double *Bm, const double *Cm,
               const double *Dskip, const double *z, const double *h0, double *y, double *hT, long batch,
               long seqlen, long nheads, long headdim, long d_state, long ngroups, int nthreads);
int oracle_s6_scan_bwd(const double *u, const double *delta, const double *A, const double *Bm, const double *Cm,
                       const double *Dskip, const double *z, const double *h0, const double *dout,
                       const double *dhT, double *du, double *ddelta, double *dA, double *dB, double *dC,
                       double *dD, double *dz, double *dh0, long batch, long d_inner, long seqlen, long d_state,
                       int nthreads);

static unsigned long long rng = 0x9E3779B97F4A7C15ull;
static double unif(void) {             /* xorshift64*, in [0, 1) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}
/* exactly n doubles on the heap (so a read past the end is caught); n may be 0 */
static double *arr(long n, double lo, double hi) {
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (long i = 0; i < n; ++i) p[i] = lo + (hi - lo) * unif();
    return p;
}

static int fails = 0;
#define CHECK(c, ...)                        \
    do {                                     \
        if (!(c)) {                          \
            fprintf(stderr, __VA_ARGS__);    \
            fputc('\n', stderr);             \
            ++fails;                         \
        }                                    \
    } while (0)

static void s6_case(long b, long d, long L, long N, int opt, int threads) {
    double *u = arr(b * d * L, -1, 1), *dl = arr(b * d * L, 1e-3, 0.2), *A = arr(d * N, -3, 0);
    double *Bm = arr(b * N * L, -1, 1), *Cm = arr(b * N * L, -1, 1), *D = arr(d, -1, 1), *z = arr(b * d * L, -2, 2);
    double *h0 = arr(b * d * N, -1, 1), *y = arr(b * d * L, 0, 0), *hT = arr(b * d * N, 0, 0);
    const int gz = opt & 1, gd = opt & 2, gh = opt & 4, gf = opt & 8;
    int rc = oracle_s6_scan(u, dl, A, Bm, Cm, gd ? D : NULL, gz ? z : NULL, gh ? h0 : NULL, y, gf ? hT : NULL, b, d,
                            L, N, threads);
    CHECK(rc == 0, "s6 rc %d", rc);
    rc = oracle_s6_scan_zoh(u, dl, A, Bm, Cm, gd ? D : NULL, gz ? z : NULL, gh ? h0 : NULL, y, gf ? hT : NULL, b,
                            d, L, N, threads);
    CHECK(rc == 0, "zoh rc %d", rc);

    /* scan == L decode steps ([B, D] / [B, N] slices of the [.., L] layouts) */
    if (L > 0 && b > 0 && d > 0) {
        double *ys = arr(b * d * L, 0, 0), *st = arr(b * d * N, 0, 0);
        double *ut = arr(b * d, 0, 0), *dt = arr(b * d, 0, 0), *zt = arr(b * d, 0, 0), *yt = arr(b * d, 0, 0);
        double *bt = arr(b * N, 0, 0), *ct = arr(b * N, 0, 0), *hs = arr(b * d * N, 0, 0);
        oracle_s6_scan(u, dl, A, Bm, Cm, D, z, h0, ys, hs, b, d, L, N, threads);
        memcpy(st, h0, (size_t)(b * d * N) * sizeof(double));
        double err = 0.0;
        for (long t = 0; t < L; ++t) {
            for (long i = 0; i < b * d; ++i) {
                ut[i] = u[i * L + t];
                dt[i] = dl[i * L + t];
                zt[i] = z[i * L + t];
            }
            for (long i = 0; i < b * N; ++i) {
                bt[i] = Bm[i * L + t];
                ct[i] = Cm[i * L + t];
            }
            CHECK(oracle_state_update(st, ut, dt, A, bt, ct, D, zt, yt, b, d, N, threads) == 0, "decode rc");
            for (long i = 0; i < b * d; ++i) err = fmax(err, fabs(yt[i] - ys[i * L + t]));
        }
        for (long i = 0; i < b * d * N; ++i) err = fmax(err, fabs(st[i] - hs[i]));
        CHECK(err <= 1e-12, "scan != decode steps: %g", err);
        free(ys); free(st); free(ut); free(dt); free(zt); free(yt); free(bt); free(ct); free(hs);
    }

    double *dout = arr(b * d * L, -1, 1), *dhT = arr(b * d * N, -1, 1);
    double *du = arr(b * d * L, 0, 0), *ddl = arr(b * d * L, 0, 0), *dA = arr(d * N, 0, 0), *dB = arr(b * N * L, 0, 0);
    double *dC = arr(b * N * L, 0, 0), *dD = arr(d, 0, 0), *dz = arr(b * d * L, 0, 0), *dh0 = arr(b * d * N, 0, 0);
    rc = oracle_s6_scan_bwd(u, dl, A, Bm, Cm, gd ? D : NULL, gz ? z : NULL, gh ? h0 : NULL, dout, gf ? dhT : NULL,
                            du, ddl, dA, dB, dC, dD, gz ? dz : NULL, gh ? dh0 : NULL, b, d, L, N, threads);
    CHECK(rc == 0, "bwd rc %d", rc);
    free(u); free(dl); free(A); free(Bm); free(Cm); free(D); free(z); free(h0); free(y); free(hT);
    free(dout); free(dhT); free(du); free(ddl); free(dA); free(dB); free(dC); free(dD); free(dz); free(dh0);
}

static void ssd_case(long b, long L, long H, long P, long N, long G, int opt, int threads) {
    double *x = arr(b * L * H * P, -1, 1), *dt = arr(b * L * H, 1e-3, 0.2), *A = arr(H, -3, 0);
    double *Bm = arr(b * L * G * N, -1, 1), *Cm = arr(b * L * G * N, -1, 1), *D = arr(H, -1, 1);
    double *z = arr(b * L * H * P, -2, 2), *h0 = arr(b * H * P * N, -1, 1);
    double *y = arr(b * L * H * P, 0, 0), *hT = arr(b * H * P * N, 0, 0);
    const int gz = opt & 1, gd = opt & 2, gh = opt & 4, gf = opt & 8;
    int rc = oracle_ssd(x, dt, A, Bm, Cm, gd ? D : NULL, gz ? z : NULL, gh ? h0 : NULL, y, gf ? hT : NULL, b, L, H,
                        P, N, G, threads);
    CHECK(rc == 0, "ssd rc %d", rc);

    /* SSD on heads == S6 with A_h broadcast over the states, per (b, h) */
    if (b > 0 && L > 0 && gf) {
        for (long bb = 0; bb < b; ++bb)
            for (long h = 0; h < H; ++h) {
                const long g = h / (H / G);
                double *u1 = arr(P * L, 0, 0), *d1 = arr(P * L, 0, 0), *A1 = arr(P * N, 0, 0);
                double *B1 = arr(N * L, 0, 0), *C1 = arr(N * L, 0, 0), *D1 = arr(P, 0, 0), *z1 = arr(P * L, 0, 0);
                double *h1 = arr(P * N, 0, 0), *y1 = arr(P * L, 0, 0), *t1 = arr(P * N, 0, 0);
                for (long p = 0; p < P; ++p) {
                    for (long t = 0; t < L; ++t) {
                        const long o = ((bb * L + t) * H + h) * P + p;
                        u1[p * L + t] = x[o];
                        d1[p * L + t] = dt[(bb * L + t) * H + h];
                        z1[p * L + t] = z[o];
                    }
                    for (long n = 0; n < N; ++n) {
                        A1[p * N + n] = A[h];
                        h1[p * N + n] = h0[((bb * H + h) * P + p) * N + n];
                    }
                    D1[p] = D[h];
                }
                for (long n = 0; n < N; ++n)
                    for (long t = 0; t < L; ++t) {
                        B1[n * L + t] = Bm[((bb * L + t) * G + g) * N + n];
                        C1[n * L + t] = Cm[((bb * L + t) * G + g) * N + n];
                    }
                oracle_s6_scan(u1, d1, A1, B1, C1, gd ? D1 : NULL, gz ? z1 : NULL, gh ? h1 : NULL, y1, t1, 1, P, L, N,
                               threads);
                double err = 0.0;
                for (long p = 0; p < P; ++p) {
                    for (long t = 0; t < L; ++t) err = fmax(err, fabs(y1[p * L + t] - y[((bb * L + t) * H + h) * P + p]));
                    for (long n = 0; n < N; ++n)
                        err = fmax(err, fabs(t1[p * N + n] - hT[((bb * H + h) * P + p) * N + n]));
                }
                CHECK(err <= 1e-12, "ssd != s6 on head %ld: %g", h, err);
                free(u1); free(d1); free(A1); free(B1); free(C1); free(D1); free(z1); free(h1); free(y1); free(t1);
            }
    }
    free(x); free(dt); free(A); free(Bm); free(Cm); free(D); free(z); free(h0); free(y); free(hT);
}

int main(void) {
    const long s6[][4] = {{1, 1, 1, 1}, {2, 3, 7, 3}, {1, 5, 0, 4}, {0, 4, 5, 2}, {3, 2, 9, 16}, {1, 7, 33, 1}};
    const int thr[] = {1, 3, 8, 64};
    for (int i = 0; i < (int)(sizeof(s6) / sizeof(s6[0])); ++i)
        for (int opt = 0; opt < 16; opt += 5)
            s6_case(s6[i][0], s6[i][1], s6[i][2], s6[i][3], opt | 8, thr[(i + opt) % 4]);
    s6_case(2, 3, 7, 3, 0, 2);
    const long sd[][6] = {{1, 5, 2, 3, 4, 1}, {2, 9, 4, 2, 3, 2}, {1, 0, 2, 2, 2, 1}, {0, 3, 2, 2, 2, 2}, {1, 17, 3, 1, 1, 3}};
    for (int i = 0; i < (int)(sizeof(sd) / sizeof(sd[0])); ++i)
        for (int opt = 0; opt < 16; opt += 5)
            ssd_case(sd[i][0], sd[i][1], sd[i][2], sd[i][3], sd[i][4], sd[i][5], opt | 8, thr[(i + opt) % 4]);
    ssd_case(2, 9, 4, 2, 3, 2, 0, 3);
    /* argument errors: no crash, an error code */
    CHECK(oracle_ssd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 1, 1, 1, 1) != 0,
          "ssd accepted NULL");
    CHECK(oracle_s6_scan_bwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                             NULL, NULL, NULL, 1, 1, 1, 1, 1) != 0,
          "bwd accepted NULL");
    if (fails) {
        fprintf(stderr, "%d failures\n", fails);
        return 1;
    }
    printf("oracle drive: ok\n");
    return 0;
}

/*
 * Float64 CPU oracle for the Mamba-2 selective state-space (SSD) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code with the HIP library.
 *
 * What it computes (the Mamba-2 selective state-space layer whose forward and
 * backward kernels the Zyphra/AMD post "Training Transformers and Hybrid
 * models on AMD Instinct MI300X Accelerators", section "Mamba-2", ports to
 * AMD GPUs).  The pages print no formula; this is the layer's defining
 * recurrence, evaluated token by token with no chunking:
 *
 *   for every batch b and head h, with group g = h / (nheads / ngroups):
 *     state S_{-1} = S0 (the initial state, zero when none is given;
 *                        dstate x headdim)
 *     a_t   = exp(dt_t * A_h)
 *     S_t   = a_t * S_{t-1} + dt_t * B_t x_t^T          (B_t: dstate, x_t: headdim)
 *     y_t   = S_t^T C_t + D_h * x_t
 *   final_state[b][h][p][n] = S_{L-1}[n][p]
 *
 * Backward: the exact reverse-mode gradient of the scalar
 *   sum_t <dy_t, y_t> + <dS_fin, final_state>
 * (dS_fin, the final-state cotangent, zero when none is given), derived by
 * hand from the recurrence:
 *
 *   Gt = dL/dS_t satisfies  G_{L-1} = C_{L-1} dy_{L-1}^T + dS_fin,
 *                           G_t     = C_t dy_t^T + a_{t+1} G_{t+1}
 *   dC_t  += S_t dy_t                      (summed over the heads of the group)
 *   dx_t   = dt_t G_t^T B_t + D_h dy_t
 *   dB_t  += dt_t G_t x_t                  (summed over the heads of the group)
 *   r_t    = a_t <G_t, S_{t-1}>            (Frobenius product)
 *   ddt_t  = B_t^T G_t x_t + A_h r_t
 *   dA_h  += dt_t r_t
 *   dD_h  += <dy_t, x_t>
 *   dS0    = a_0 G_0                       (gradient of the initial state)
 *
 * S_{t-1} is re-derived during the reverse sweep from float64 checkpoints
 * taken every ORACLE_SEG steps; re-running the same float64 operations in the
 * same order reproduces the forward states bit for bit.
 *
 * Layouts (row-major, float64): x, y, dx, dy [b][L][H][P]; dt, ddt [b][L][H];
 * B, C, dB, dC [b][L][G][N]; A, D, dA, dD [H]; final_state, initial state,
 * its gradient and the final-state cotangent [b][H][P][N] (element [p][n]
 * is S[n][p]).  Every state pointer may be NULL: a missing initial state or
 * cotangent is zero, a missing gradient output is not written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_SEG 256

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One time step of the recurrence for one (b, h): S <- a S + dt B x^T. */
static void step_state(double *S, int64_t N, int64_t P, double a, double dt,
                       const double *Bt, const double *xt) {
    for (int64_t n = 0; n < N; ++n) {
        const double bn = dt * Bt[n];
        double *row = S + n * P;
        for (int64_t p = 0; p < P; ++p) row[p] = a * row[p] + bn * xt[p];
    }
}

/* S[n][p] = src[p][n] (src in the [P][N] interface layout), or zero. */
static void load_state(double *S, const double *src, int64_t N, int64_t P) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t p = 0; p < P; ++p) S[n * P + p] = src ? src[p * N + n] : 0.0;
}

static void store_state(double *dst, const double *S, int64_t N, int64_t P) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t p = 0; p < P; ++p) dst[p * N + n] = S[n * P + p];
}

int oracle_ssd_fwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                   const double *x, const double *dt, const double *A,
                   const double *B, const double *C, const double *D,
                   const double *init_state, double *y, double *final_state, int nthreads) {
    if (batch <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
    set_threads(nthreads);
    const int64_t hpg = H / G;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < batch * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        double *S = (double *)calloc((size_t)(N * P), sizeof(double));
        if (!S) {
#pragma omp atomic write
            err = 2;
            continue;
        }
        load_state(S, init_state ? init_state + (b * H + h) * P * N : NULL, N, P);
        for (int64_t t = 0; t < L; ++t) {
            const double dtt = dt[(b * L + t) * H + h];
            const double a = exp(dtt * A[h]);
            const double *xt = x + ((b * L + t) * H + h) * P;
            const double *Bt = B + ((b * L + t) * G + g) * N;
            const double *Ct = C + ((b * L + t) * G + g) * N;
            step_state(S, N, P, a, dtt, Bt, xt);
            double *yt = y + ((b * L + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) yt[p] = D[h] * xt[p];
            for (int64_t n = 0; n < N; ++n) {
                const double cn = Ct[n];
                const double *row = S + n * P;
                for (int64_t p = 0; p < P; ++p) yt[p] += cn * row[p];
            }
        }
        if (final_state) store_state(final_state + (b * H + h) * P * N, S, N, P);
        free(S);
    }
    return err;
}

int oracle_ssd_bwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                   const double *x, const double *dt, const double *A,
                   const double *B, const double *C, const double *D, const double *dy,
                   const double *init_state, const double *dfinal_state,
                   double *dx, double *ddt, double *dA, double *dB, double *dC, double *dD,
                   double *dinit_state, int nthreads) {
    if (batch <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
    set_threads(nthreads);
    const int64_t hpg = H / G;
    const int64_t nseg = (L + ORACLE_SEG - 1) / ORACLE_SEG;
    const int64_t NP = N * P;
    /* Per-(b,h) contributions to dB/dC and dA/dD; summed over heads and batch
     * in a fixed order afterwards so the result does not depend on threading. */
    double *dBh = (double *)calloc((size_t)(batch * H * L * N), sizeof(double));
    double *dCh = (double *)calloc((size_t)(batch * H * L * N), sizeof(double));
    double *dAh = (double *)calloc((size_t)(batch * H), sizeof(double));
    double *dDh = (double *)calloc((size_t)(batch * H), sizeof(double));
    if (!dBh || !dCh || !dAh || !dDh) {
        free(dBh); free(dCh); free(dAh); free(dDh);
        return 2;
    }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < batch * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        /* ckpt[s] = state before segment s, i.e. S_{s*SEG - 1} (S0 for s = 0). */
        double *ckpt = (double *)calloc((size_t)(nseg * NP), sizeof(double));
        double *seg = (double *)malloc((size_t)(ORACLE_SEG * NP) * sizeof(double));
        double *Gs = (double *)calloc((size_t)NP, sizeof(double));
        double *tmp = (double *)malloc((size_t)N * sizeof(double));
        if (!ckpt || !seg || !Gs || !tmp) {
#pragma omp atomic write
            err = 2;
            free(ckpt); free(seg); free(Gs); free(tmp);
            continue;
        }
        /* Forward sweep: record checkpoints. */
        {
            double *S = seg; /* scratch state */
            load_state(S, init_state ? init_state + (b * H + h) * P * N : NULL, N, P);
            for (int64_t t = 0; t < L; ++t) {
                if (t % ORACLE_SEG == 0) memcpy(ckpt + (t / ORACLE_SEG) * NP, S, (size_t)NP * sizeof(double));
                const double dtt = dt[(b * L + t) * H + h];
                step_state(S, N, P, exp(dtt * A[h]), dtt,
                           B + ((b * L + t) * G + g) * N, x + ((b * L + t) * H + h) * P);
            }
        }
        double dA_acc = 0.0, dD_acc = 0.0;
        /* Reverse sweep.  Gs holds a_{t+1} G_{t+1} on entry to step t; on
         * entry to the last step that is the final-state cotangent. */
        load_state(Gs, dfinal_state ? dfinal_state + (b * H + h) * P * N : NULL, N, P);
        for (int64_t s = nseg - 1; s >= 0; --s) {
            const int64_t t0 = s * ORACLE_SEG;
            const int64_t t1 = (t0 + ORACLE_SEG < L) ? t0 + ORACLE_SEG : L;
            /* Recompute S_t for t in [t0, t1) into seg[t - t0]. */
            const double *prev = ckpt + s * NP;
            for (int64_t t = t0; t < t1; ++t) {
                double *S = seg + (t - t0) * NP;
                memcpy(S, prev, (size_t)NP * sizeof(double));
                const double dtt = dt[(b * L + t) * H + h];
                step_state(S, N, P, exp(dtt * A[h]), dtt,
                           B + ((b * L + t) * G + g) * N, x + ((b * L + t) * H + h) * P);
                prev = S;
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const double dtt = dt[(b * L + t) * H + h];
                const double a = exp(dtt * A[h]);
                const double *xt = x + ((b * L + t) * H + h) * P;
                const double *dyt = dy + ((b * L + t) * H + h) * P;
                const double *Bt = B + ((b * L + t) * G + g) * N;
                const double *Ct = C + ((b * L + t) * G + g) * N;
                const double *St = seg + (t - t0) * NP;
                const double *Sprev = (t > t0) ? seg + (t - t0 - 1) * NP : ckpt + s * NP;
                /* G_t = C_t dy_t^T + a_{t+1} G_{t+1} */
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p) Gs[n * P + p] += Ct[n] * dyt[p];
                /* dC_t (this head) = S_t dy_t */
                double *dCt = dCh + ((b * H + h) * L + t) * N;
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) acc += St[n * P + p] * dyt[p];
                    dCt[n] = acc;
                }
                /* dx_t = dt G_t^T B_t + D dy_t */
                double *dxt = dx + ((b * L + t) * H + h) * P;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) acc += Gs[n * P + p] * Bt[n];
                    dxt[p] = dtt * acc + D[h] * dyt[p];
                }
                /* tmp = G_t x_t;  dB_t (this head) = dt tmp;  B^T G x = <B_t, tmp> */
                double bgx = 0.0;
                double *dBt = dBh + ((b * H + h) * L + t) * N;
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) acc += Gs[n * P + p] * xt[p];
                    tmp[n] = acc;
                    dBt[n] = dtt * acc;
                    bgx += Bt[n] * acc;
                }
                /* r_t = a_t <G_t, S_{t-1}> */
                double gs = 0.0;
                for (int64_t i = 0; i < NP; ++i) gs += Gs[i] * Sprev[i];
                const double r = a * gs;
                ddt[(b * L + t) * H + h] = bgx + A[h] * r;
                dA_acc += dtt * r;
                double xy = 0.0;
                for (int64_t p = 0; p < P; ++p) xy += dyt[p] * xt[p];
                dD_acc += xy;
                /* carry a_t G_t to step t-1 */
                for (int64_t i = 0; i < NP; ++i) Gs[i] *= a;
            }
        }
        /* Gs now holds a_0 G_0 = dL/dS_{-1}. */
        if (dinit_state) store_state(dinit_state + (b * H + h) * P * N, Gs, N, P);
        dAh[b * H + h] = dA_acc;
        dDh[b * H + h] = dD_acc;
        free(ckpt); free(seg); free(Gs); free(tmp);
    }
    if (!err) {
        /* Fixed-order sums: dB/dC over the heads of each group, dA/dD over batch. */
#pragma omp parallel for schedule(static)
        for (int64_t bt = 0; bt < batch * L; ++bt) {
            const int64_t b = bt / L, t = bt % L;
            for (int64_t g = 0; g < G; ++g) {
                double *ob = dB + ((b * L + t) * G + g) * N;
                double *oc = dC + ((b * L + t) * G + g) * N;
                for (int64_t n = 0; n < N; ++n) { ob[n] = 0.0; oc[n] = 0.0; }
                for (int64_t hh = g * hpg; hh < (g + 1) * hpg; ++hh) {
                    const double *sb = dBh + ((b * H + hh) * L + t) * N;
                    const double *sc = dCh + ((b * H + hh) * L + t) * N;
                    for (int64_t n = 0; n < N; ++n) { ob[n] += sb[n]; oc[n] += sc[n]; }
                }
            }
        }
        for (int64_t h = 0; h < H; ++h) {
            double sa = 0.0, sd = 0.0;
            for (int64_t b = 0; b < batch; ++b) { sa += dAh[b * H + h]; sd += dDh[b * H + h]; }
            dA[h] = sa;
            dD[h] = sd;
        }
    }
    free(dBh); free(dCh); free(dAh); free(dDh);
    return err;
}

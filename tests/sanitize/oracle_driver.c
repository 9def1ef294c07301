/* Runs the float64 oracle (oracle/ssd_oracle.c, linked in) on small shapes
 * under AddressSanitizer and UndefinedBehaviorSanitizer: every path of the
 * forward and the backward (initial state and final-state cotangent absent or
 * given, reverse sweeps that cross the 256-step checkpoint boundary, one and
 * several OpenMP threads, bad sizes).  Exits non-zero on a non-finite output,
 * on an unexpected return code, or (through the sanitizers) on any memory or
 * undefined-behaviour error.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_ssd_fwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const double *x,
                   const double *dt, const double *A, const double *B, const double *C, const double *D,
                   const double *init_state, double *y, double *final_state, int nthreads);
int oracle_ssd_bwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const double *x,
                   const double *dt, const double *A, const double *B, const double *C, const double *D,
                   const double *dy, const double *init_state, const double *dfinal_state, double *dx, double *ddt,
                   double *dA, double *dB, double *dC, double *dD, double *dinit_state, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double unif(void) { /* xorshift64 in [0, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static double *arr(int64_t n, double lo, double hi) {
    double *a = (double *)malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * unif();
    return a;
}
static int finite_all(const double *a, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static int run(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int states, int nthreads) {
    const int64_t nx = b * L * H * P, nt = b * L * H, nb = b * L * G * N, ns = b * H * P * N;
    double *x = arr(nx, -1, 1), *dt = arr(nt, 0, 0.2), *A = arr(H, -4, -0.1), *B = arr(nb, -1, 1);
    double *C = arr(nb, -1, 1), *D = arr(H, -1, 1), *dy = arr(nx, -1, 1);
    double *s0 = states ? arr(ns, -1, 1) : NULL, *dfs = states ? arr(ns, -1, 1) : NULL;
    double *y = arr(nx, 0, 0), *fs = arr(ns, 0, 0), *dx = arr(nx, 0, 0), *ddt = arr(nt, 0, 0);
    double *dA = arr(H, 0, 0), *dB = arr(nb, 0, 0), *dC = arr(nb, 0, 0), *dD = arr(H, 0, 0), *ds0 = arr(ns, 0, 0);
    int bad = 0;
    if (oracle_ssd_fwd(b, L, H, P, N, G, x, dt, A, B, C, D, s0, y, fs, nthreads)) bad |= 1;
    if (oracle_ssd_bwd(b, L, H, P, N, G, x, dt, A, B, C, D, dy, s0, dfs, dx, ddt, dA, dB, dC, dD, ds0, nthreads))
        bad |= 2;
    if (!finite_all(y, nx) || !finite_all(fs, ns) || !finite_all(dx, nx) || !finite_all(ddt, nt) ||
        !finite_all(dA, H) || !finite_all(dB, nb) || !finite_all(dC, nb) || !finite_all(dD, H) ||
        !finite_all(ds0, ns))
        bad |= 4;
    /* optional outputs left out */
    if (oracle_ssd_fwd(b, L, H, P, N, G, x, dt, A, B, C, D, s0, y, NULL, nthreads)) bad |= 8;
    if (oracle_ssd_bwd(b, L, H, P, N, G, x, dt, A, B, C, D, dy, s0, dfs, dx, ddt, dA, dB, dC, dD, NULL, nthreads))
        bad |= 16;
    double *ptrs[] = {x, dt, A, B, C, D, dy, s0, dfs, y, fs, dx, ddt, dA, dB, dC, dD, ds0};
    for (unsigned i = 0; i < sizeof ptrs / sizeof ptrs[0]; ++i) free(ptrs[i]);
    if (bad) fprintf(stderr, "shape b=%lld L=%lld H=%lld P=%lld N=%lld G=%lld states=%d threads=%d: flags %d\n",
                     (long long)b, (long long)L, (long long)H, (long long)P, (long long)N, (long long)G, states,
                     nthreads, bad);
    return bad;
}

int main(void) {
    static const int64_t shapes[][6] = {
        {1, 1, 1, 1, 1, 1}, {2, 5, 4, 3, 2, 2}, {1, 257, 2, 4, 3, 1}, {2, 513, 2, 2, 2, 2}, {1, 64, 6, 2, 5, 3}};
    int bad = 0;
    for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int states = 0; states < 2; ++states)
            for (int th = 1; th <= 4; th += 3)
                bad |= run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], shapes[s][4], shapes[s][5],
                           states, th);
    /* invalid sizes are refused before any access */
    double one = 1.0;
    if (oracle_ssd_fwd(1, 0, 1, 1, 1, 1, &one, &one, &one, &one, &one, &one, NULL, &one, NULL, 1) != 1) bad |= 32;
    if (oracle_ssd_fwd(1, 1, 3, 1, 1, 2, &one, &one, &one, &one, &one, &one, NULL, &one, NULL, 1) != 1) bad |= 32;
    if (oracle_ssd_bwd(1, 1, 1, 1, -1, 1, &one, &one, &one, &one, &one, &one, &one, NULL, NULL, &one, &one, &one, &one,
                       &one, &one, NULL, 1) != 1)
        bad |= 32;
    printf("oracle sanitizer driver: %s\n", bad ? "FAILED" : "ok");
    return bad ? 1 : 0;
}

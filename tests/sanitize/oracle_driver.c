/* Runs the fp64 oracle's C routines on small shapes and edge cases (empty sequences, conv
 * width 1, one group per head, gated and ungated outputs, bf16-state emulation, the
 * selective scan with and without its optional inputs) under the address and
 * undefined-behaviour sanitizers, with a few closed-form checks. Exits nonzero on a failed
 * check; the sanitizers abort on any memory or undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_conv1d_seq(int64_t T, int64_t C, int32_t W, const double *u, const double *w, const double *bias,
                       double *state, double *out);
void oracle_ssm_seq(int64_t T, int32_t H, int32_t P, int32_t N, int32_t G, const double *xbc, const double *dt_raw,
                    const double *A_log, const double *dt_bias, const double *D, const double *z, double *h,
                    double *y, int32_t round_state_bf16);
void oracle_selective_scan_seq(int64_t T, int32_t Dc, int32_t N, int32_t G, const double *u, const double *delta_raw,
                               const double *A, const double *B, const double *C, const double *Dv, const double *z,
                               const double *delta_bias, int32_t delta_softplus, double *h, double *y);
double oracle_softplus(double v);
double oracle_silu(double v);
double oracle_round_bf16(double v);

static int fails = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            fails = 1;                                                  \
        }                                                               \
    } while (0)

static double *arr(size_t n, unsigned *seed) {
    double *a = malloc((n ? n : 1) * sizeof *a);
    for (size_t i = 0; i < n; ++i) a[i] = (double)rand_r(seed) / RAND_MAX - 0.5;
    return a;
}

int main(void) {
    unsigned seed = 7;
    /* conv: every width, lengths around the width, with and without bias */
    for (int W = 1; W <= 5; ++W)
        for (int T = 0; T <= 6; ++T)
            for (int b = 0; b < 2; ++b) {
                const int C = 3;
                double *u = arr((size_t)T * C, &seed), *w = arr((size_t)C * W, &seed), *bias = arr(C, &seed);
                double *st = arr((size_t)(W - 1) * C, &seed), *st0 = malloc(((W - 1) * C + 1) * sizeof *st0);
                double *out = malloc(((size_t)T * C + 1) * sizeof *out);
                for (int i = 0; i < (W - 1) * C; ++i) st0[i] = st[i];
                oracle_conv1d_seq(T, C, W, u, w, b ? bias : NULL, st, out);
                /* the new state is the last W-1 entries of [old state || u] */
                for (int j = 0; j < W - 1; ++j)
                    for (int c = 0; c < C; ++c) {
                        const int pos = T + j - (W - 1);
                        const double want = pos >= 0 ? u[pos * C + c] : st0[(W - 1 + pos) * C + c];
                        CHECK(st[j * C + c] == want);
                    }
                if (W == 1)
                    for (int t = 0; t < T; ++t)
                        for (int c = 0; c < C; ++c)
                            CHECK(fabs(out[t * C + c] - oracle_silu(w[c] * u[t * C + c] + (b ? bias[c] : 0.0))) <
                                  1e-15);
                free(u), free(w), free(bias), free(st), free(st0), free(out);
            }
    /* recurrence: several (H, P, N, G), T = 0..5, gated or not, bf16-state emulation */
    const int shapes[][4] = {{1, 1, 1, 1}, {2, 3, 4, 1}, {4, 2, 3, 4}, {4, 4, 4, 2}};
    for (int si = 0; si < 4; ++si)
        for (int T = 0; T <= 5; ++T)
            for (int gz = 0; gz < 2; ++gz)
                for (int rb = 0; rb < 2; ++rb) {
                    const int H = shapes[si][0], P = shapes[si][1], N = shapes[si][2], G = shapes[si][3];
                    const int cd = H * P + 2 * G * N;
                    double *x = arr((size_t)T * cd, &seed), *dtr = arr((size_t)T * H, &seed);
                    double *al = arr(H, &seed), *db = arr(H, &seed), *D = arr(H, &seed);
                    double *z = arr((size_t)T * H * P, &seed), *h = arr((size_t)H * P * N, &seed);
                    double *y = malloc(((size_t)T * H * P + 1) * sizeof *y);
                    oracle_ssm_seq(T, H, P, N, G, x, dtr, al, db, D, gz ? z : NULL, h, y, rb);
                    for (int i = 0; i < T * H * P; ++i) CHECK(isfinite(y[i]));
                    free(x), free(dtr), free(al), free(db), free(D), free(z), free(h), free(y);
                }
    /* one token from zero state: y = C.(dt x B) + D x in closed form */
    {
        const int H = 1, P = 1, N = 2, G = 1, cd = H * P + 2 * G * N;
        double x[5] = {0.7, 0.3, -0.2, 0.5, 0.25}, dtr = 0.1, al = 0.4, db = -0.3, D = 1.5, h[2] = {0, 0}, y;
        (void)cd;
        oracle_ssm_seq(1, H, P, N, G, x, &dtr, &al, &db, &D, NULL, h, &y, 0);
        const double dt = log1p(exp(-0.2)) + 0.0;  /* softplus(-0.2) */
        const double want = dt * 0.7 * (0.3 * 0.5 + -0.2 * 0.25) + 1.5 * 0.7;
        CHECK(fabs(dt - oracle_softplus(-0.2)) < 1e-15);
        CHECK(fabs(y - want) < 1e-14);
    }
    /* selective scan: optional inputs present or absent, groups, T = 0..4 */
    for (int T = 0; T <= 4; ++T)
        for (int opt = 0; opt < 4; ++opt) {
            const int Dc = 4, N = 3, G = (opt & 1) ? 2 : 1;
            double *u = arr((size_t)T * Dc, &seed), *dr = arr((size_t)T * Dc, &seed), *A = arr((size_t)Dc * N, &seed);
            double *B = arr((size_t)T * G * N, &seed), *C = arr((size_t)T * G * N, &seed);
            double *Dv = arr(Dc, &seed), *z = arr((size_t)T * Dc, &seed), *bias = arr(Dc, &seed);
            double *h = arr((size_t)Dc * N, &seed), *y = malloc(((size_t)T * Dc + 1) * sizeof *y);
            oracle_selective_scan_seq(T, Dc, N, G, u, dr, A, B, C, (opt & 2) ? Dv : NULL, (opt & 2) ? z : NULL,
                                      (opt & 1) ? bias : NULL, opt & 1, h, y);
            for (int i = 0; i < T * Dc; ++i) CHECK(isfinite(y[i]));
            free(u), free(dr), free(A), free(B), free(C), free(Dv), free(z), free(bias), free(h), free(y);
        }
    /* scalar helpers at their edges */
    CHECK(oracle_softplus(800.0) == 800.0);
    CHECK(oracle_softplus(-800.0) >= 0.0);
    CHECK(oracle_round_bf16(1.0 + ldexp(1.0, -9)) == 1.0);
    CHECK(oracle_round_bf16(ldexp(1.0, -140)) >= 0.0);
    CHECK(isinf(oracle_round_bf16(INFINITY)));
    if (!fails) printf("oracle driver: ok\n");
    return fails;
}

/*
 * Mamba-2 SSM core -- plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; it exists so tests, the smoke check and the CPU baseline
 * leg of the benchmark can compare the HIP kernels with an obviously correct
 * sequential definition. It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (one sequence at a time, tokens strictly in order):
 *
 *  1. Causal depthwise conv1d + SiLU over every x/B/C channel. The model
 *     record "Nemotron-H-8B-Base-8K" lists a "conv1d" tensor among the
 *     Mamba-2 mixer tensors; the trace page ("Hybrid Mamba-Transformer MoEs
 *     hide their stalls...") names conv1d as a Mamba-layer kernel. Reading
 *     taken where the pages are silent: a cross-correlation whose last tap
 *     multiplies the current token, left context = the W-1 cached raw inputs
 *     (oldest first) or zeros, optional bias, SiLU after the sum. The new
 *     conv state is the last W-1 entries of [cached inputs || tokens].
 *
 *  2. Selective recurrence with one scalar decay per head (the mixer tensors
 *     A_log, D and dt_bias of the same record; the recurrence of the Mamba
 *     paper cited on the trace page, in its Mamba-2 scalar-A form):
 *        dt  = softplus(dt_raw + dt_bias),  A = -exp(A_log),  a = exp(dt*A)
 *        h_t = a * h_{t-1} + (dt * x_t) (outer) B_t
 *        y_t = C_t . h_t + D * x_t            (optionally * SiLU(z_t))
 *     B and C are shared by the H/G heads of a group; the vllm.cpp issue
 *     ("NemotronH runs the PREFILL mamba kernels at decode", section "Confirm
 *     or refute") gives hpg = H/G. Reading: head h belongs to group h / hpg.
 *
 *  3. The selective scan of the Mamba paper (S6, the "selective_scan_fwd"
 *     kernel the trace page names for Mamba layers): a diagonal state per
 *     (channel d, state n) with its own decay A[d][n],
 *        delta = softplus(delta_raw + delta_bias)   (or delta_raw + bias)
 *        h_t[d][n] = exp(delta_t[d] * A[d][n]) * h_{t-1}[d][n]
 *                    + delta_t[d] * B_t[g][n] * u_t[d]
 *        y_t[d]    = sum_n C_t[g][n] * h_t[d][n] + D[d] * u_t[d]  (* SiLU(z))
 *     with B and C shared by the D/G channels of a group g = d / (D/G).
 *     Reading: the input matrix is discretised as delta * B (the form the
 *     paper's implementation uses), A as exp(delta * A).
 *
 * Everything is fp64, no fast-math; OpenMP runs only across heads or
 * channels, which are independent, never across time.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }
static double silu(double v) { return v / (1.0 + exp(-v)); }

/* Round a double to the nearest bfloat16 value (ties to even), returned as a
 * double. Used only by the optional "state stored as bf16" emulation. */
static double round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    double m = frexp(v, &e);          /* v = m * 2^e, 0.5 <= |m| < 1 */
    if (e < -125) {                   /* bf16 subnormal range: fixed quantum 2^-133 */
        return nearbyint(ldexp(v, 133)) * ldexp(1.0, -133);
    }
    return ldexp(nearbyint(ldexp(m, 8)), e - 8); /* 8 significant bits */
}

/*
 * Conv for one sequence.
 *   u      [T][C]      raw (pre-conv) inputs
 *   w      [C][W]      taps, tap W-1 multiplies the current token
 *   bias   [C] or NULL
 *   state  [W-1][C]    in: cached raw inputs (oldest first, zeros for a new
 *                      sequence); out: last W-1 entries of [state || u]
 *   out    [T][C]      SiLU(conv)
 */
void oracle_conv1d_seq(int64_t T, int64_t C, int32_t W, const double *u, const double *w,
                       const double *bias, double *state, double *out)
{
    const int64_t K = W - 1;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        for (int64_t t = 0; t < T; ++t) {
            double v = bias ? bias[c] : 0.0;
            for (int32_t k = 0; k < W; ++k) {
                int64_t src = t - K + k; /* index into u; negative -> cached state */
                double val = src >= 0 ? u[src * C + c] : state[(K + src) * C + c];
                v += w[c * W + k] * val;
            }
            out[t * C + c] = silu(v);
        }
        /* new state = last K entries of the concatenation [state || u] */
        double tail[16];
        for (int64_t j = 0; j < K; ++j) {
            int64_t pos = T + j; /* position in the concatenation, which has K + T entries */
            int64_t src = pos - K;
            tail[j] = src >= 0 ? u[src * C + c] : state[(K + src) * C + c];
        }
        for (int64_t j = 0; j < K; ++j) state[j * C + c] = tail[j];
    }
}

/*
 * Selective recurrence for one sequence.
 *   xbc     [T][Cdim]  post-conv channels, Cdim = H*P + 2*G*N, laid out as
 *                      x (head-major, h*P + p) || B (g*N + n) || C (g*N + n)
 *   dt_raw  [T][H]
 *   A_log, dt_bias, D [H]
 *   z       [T][H*P] or NULL (gate y by SiLU(z) when given)
 *   h       [H][P][N]  in: initial state, out: final state
 *   y       [T][H*P]
 *   round_state_bf16: if nonzero, the state is rounded to bf16 after every
 *                     token (emulates a bf16-stored state)
 */
void oracle_ssm_seq(int64_t T, int32_t H, int32_t P, int32_t N, int32_t G, const double *xbc,
                    const double *dt_raw, const double *A_log, const double *dt_bias,
                    const double *D, const double *z, double *h, double *y,
                    int32_t round_state_bf16)
{
    const int64_t Cdim = (int64_t)H * P + 2 * (int64_t)G * N;
    const int32_t hpg = H / G;
    const int64_t offB = (int64_t)H * P;
    const int64_t offC = offB + (int64_t)G * N;
#pragma omp parallel for schedule(static)
    for (int32_t hd = 0; hd < H; ++hd) {
        const int32_t g = hd / hpg;
        const double A = -exp(A_log[hd]);
        double *hs = h + (int64_t)hd * P * N;
        for (int64_t t = 0; t < T; ++t) {
            const double *row = xbc + t * Cdim;
            const double dt = softplus(dt_raw[t * H + hd] + dt_bias[hd]);
            const double a = exp(dt * A);
            for (int32_t p = 0; p < P; ++p) {
                const double xv = row[(int64_t)hd * P + p];
                const double dx = dt * xv;
                double acc = 0.0;
                for (int32_t n = 0; n < N; ++n) {
                    double s = a * hs[(int64_t)p * N + n] + dx * row[offB + (int64_t)g * N + n];
                    if (round_state_bf16) s = round_bf16(s);
                    hs[(int64_t)p * N + n] = s;
                    acc += row[offC + (int64_t)g * N + n] * s;
                }
                double yv = acc + D[hd] * xv;
                if (z) yv *= silu(z[t * (int64_t)H * P + (int64_t)hd * P + p]);
                y[t * (int64_t)H * P + (int64_t)hd * P + p] = yv;
            }
        }
    }
}

/* Scalar helpers exposed so tests can pin them against closed forms. */
/* One sequence of the selective scan (item 3). u, delta_raw [T][Dc]; A [Dc][N];
 * B, C [T][G][N]; Dv, delta_bias [Dc] or NULL; z [T][Dc] or NULL; h [Dc][N]
 * in/out; y [T][Dc]. */
void oracle_selective_scan_seq(int64_t T, int32_t Dc, int32_t N, int32_t G, const double *u,
                               const double *delta_raw, const double *A, const double *B,
                               const double *C, const double *Dv, const double *z,
                               const double *delta_bias, int32_t delta_softplus, double *h,
                               double *y) {
    const int32_t cpg = Dc / G;
#pragma omp parallel for schedule(static)
    for (int32_t d = 0; d < Dc; ++d) {
        const int32_t g = d / cpg;
        double *hd = h + (int64_t)d * N;
        for (int64_t t = 0; t < T; ++t) {
            double dl = delta_raw[t * Dc + d] + (delta_bias ? delta_bias[d] : 0.0);
            if (delta_softplus) dl = softplus(dl);
            const double ut = u[t * Dc + d];
            const double *Bt = B + (t * G + g) * N;
            const double *Ct = C + (t * G + g) * N;
            double acc = 0.0;
            for (int32_t n = 0; n < N; ++n) {
                hd[n] = exp(dl * A[(int64_t)d * N + n]) * hd[n] + dl * Bt[n] * ut;
                acc += Ct[n] * hd[n];
            }
            if (Dv) acc += Dv[d] * ut;
            if (z) acc *= silu(z[t * Dc + d]);
            y[t * Dc + d] = acc;
        }
    }
}

double oracle_softplus(double v) { return softplus(v); }
double oracle_silu(double v) { return silu(v); }
double oracle_round_bf16(double v) { return round_bf16(v); }

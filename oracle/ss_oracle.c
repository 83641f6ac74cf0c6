/*
 * ss_oracle.c -- plain, slow, double-precision CPU reference of the Mamba
 * selective scan with a softplus step size, and of its single-token
 * state-update step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark.  It shares no code, header, table or
 * constant with the HIP library and includes no HIP header.
 *
 * What it computes follows the pages:
 *   - mhpn.cn "PyTorch新手也能懂：手把手拆解Mamba-minimal中的selective_scan实现",
 *     section 2 (argument shapes), section 3 with 3.1/3.2 (discretisation:
 *     ZOH exp(delta*A) for A, forward Euler delta*B*u for B), section 4 (the
 *     sequential loop: zero initial state, update then read out with C),
 *     section 5 (the D skip), section 7 (A = -exp(A_log), softplus keeps
 *     delta positive);
 *   - jiafeimiao.top "代码连连看——mamba", the Mamba.step listing (dt bias
 *     added before the softplus, A = -exp(A_log), the in-place state update,
 *     readout with C, D skip, then the gate y * silu(z)).
 * Every loop is written in the order of that definition; there is no
 * blocking, fusion or reordering.  All arithmetic is in double; the caller
 * widens its fp32 / bf16 inputs exactly.
 *
 * The _ex forms add two options: an initial state h0 for the scan (instead
 * of zero) and the zero-order-hold input weight (exp(delta*A) - 1)/A * B in
 * place of forward Euler delta*B (mhpn.cn page, sections 3.2 and 6).
 *
 * ss_oracle_conv_update is the convolution step that Mamba.step runs before
 * the SSM step (jiafeimiao.top page, the "Conv step" branch written out in
 * torch): a rolling window of the last W inputs per channel, a depthwise dot
 * product with the channel's W weights, the bias, then silu.
 *
 * ss_oracle_scan_bwd_ex is the gradient of ss_oracle_scan_ex (Euler or
 * zero-order-hold input term) with respect to every input, for a given
 * gradient of y and of last_state; ss_oracle_scan_bwd is its Euler form.
 * The pages only name the autograd wrappers, so the formulas are derived
 * here by the chain rule and written out step by step below; they are pinned
 * to torch autograd and to finite differences of the forward.
 *
 * ss_oracle_cross_scan is VMamba's CrossScan / scan / CrossMerge
 * (githubissues.com VMamba issue 206: the cross operations only arrange the
 * sequence): each feature map is read as four sequences -- row-major,
 * column-major, and both of those backwards -- each scanned as its own
 * sequence, and the four outputs are added back at the positions they came
 * from.
 *
 * The scan and the step also build as a second library with OpenMP (the
 * baseline timed on all host cores): the only difference is the pragma
 * that hands the independent (batch, channel) recurrences to threads; each
 * recurrence runs exactly the same arithmetic in the same order, so both
 * builds give the same results bit for bit.  Without -fopenmp the pragmas
 * are ignored.
 *
 * Layouts (row-major, last index fastest):
 *   u, delta, z, y : (b, L, d_in)      B, C : (b, L, n)
 *   A_log          : (d_in, n)         D, delta_bias : (d_in)
 *   state, h0, last_state : (b, d_in, n)
 *   x, dt, z, y of the step : (b, d_in)     B, C of the step : (b, n)
 *   conv_state : (b, d_in, W)   conv weight : (d_in, W)   conv bias : (d_in)
 * Return value: 0 on success, -1 on a NULL required pointer, -2 on a
 * non-positive size.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the (batch, channel) loops may use: 1 unless built with OpenMP. */
int ss_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* softplus(x) = log(1 + e^x), evaluated without overflow or cancellation:
 * for x > 0 it is x + log(1 + e^-x).  (mhpn.cn page, section 7: softplus
 * keeps delta positive.) */
double ss_oracle_softplus(double x)
{
    if (x > 0.0)
        return x + log1p(exp(-x));
    return log1p(exp(x));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z)  (the gate act(z) of Mamba.step). */
double ss_oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* The step size of one (b, t, d) element: delta plus the optional bias,
 * then the optional softplus (jiafeimiao.top page, Mamba.step: the bias is
 * not added to dt earlier, it goes inside the softplus). */
static double step_size(double delta, const double *bias, int64_t d, int softplus)
{
    double v = delta + (bias ? bias[d] : 0.0);
    return softplus ? ss_oracle_softplus(v) : v;
}

/* Discretised input weight of one state: forward Euler delta*B (the
 * mamba-minimal loop, mhpn.cn page section 3.2), or with zoh != 0 the
 * zero-order hold (exp(delta*A) - 1) / A * B that the page contrasts it with
 * in section 6 (for a diagonal A the matrix form (delta A)^-1 (exp(delta A) - I)
 * delta B reduces to this per state).  A = 0 exactly (A_log below about
 * -745) takes the limit delta*B. */
static double input_weight(double dl, double A, double Bk, int zoh)
{
    if (!zoh)
        return dl * Bk;
    if (A == 0.0)
        return dl * Bk;
    return expm1(dl * A) / A * Bk;
}

int ss_oracle_scan_ex(const double *u, const double *delta, const double *A_log,
                      const double *B, const double *C, const double *D,
                      const double *z, const double *delta_bias, int delta_softplus,
                      const double *h0, int zoh,
                      double *y, double *last_state,
                      int64_t b, int64_t L, int64_t d_in, int64_t n)
{
    if (!u || !delta || !A_log || !B || !C || !D || !y)
        return -1;
    if (b <= 0 || L <= 0 || d_in <= 0 || n <= 0)
        return -2;

    #pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t bi = 0; bi < b; bi++) {
        for (int64_t d = 0; d < d_in; d++) {
            /* h starts at zero (section 4 of the mhpn.cn page), or at the
             * given initial state h0 (b, d_in, n). */
            double h[n];
            double A[n];
            for (int64_t k = 0; k < n; k++) {
                h[k] = h0 ? h0[(bi * d_in + d) * n + k] : 0.0;
                A[k] = -exp(A_log[d * n + k]);          /* A = -exp(A_log), elementwise */
            }
            for (int64_t t = 0; t < L; t++) {
                int64_t e = (bi * L + t) * d_in + d;    /* (b, t, d) element */
                int64_t r = (bi * L + t) * n;           /* row of B and C at (b, t) */
                double dl = step_size(delta[e], delta_bias, d, delta_softplus);
                /* state update: h = exp(delta*A) * h + (input weight) * u */
                for (int64_t k = 0; k < n; k++) {
                    double dA = exp(dl * A[k]);
                    double dBu = input_weight(dl, A[k], B[r + k], zoh) * u[e];
                    h[k] = dA * h[k] + dBu;
                }
                /* read out with C after the update, then the D skip */
                double yt = 0.0;
                for (int64_t k = 0; k < n; k++)
                    yt += C[r + k] * h[k];
                yt += D[d] * u[e];
                /* optional gate, applied after the skip */
                if (z)
                    yt *= ss_oracle_silu(z[e]);
                y[e] = yt;
            }
            if (last_state)
                for (int64_t k = 0; k < n; k++)
                    last_state[(bi * d_in + d) * n + k] = h[k];
        }
    }
    return 0;
}

int ss_oracle_scan(const double *u, const double *delta, const double *A_log,
                   const double *B, const double *C, const double *D,
                   const double *z, const double *delta_bias, int delta_softplus,
                   double *y, double *last_state,
                   int64_t b, int64_t L, int64_t d_in, int64_t n)
{
    return ss_oracle_scan_ex(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, NULL, 0,
                             y, last_state, b, L, d_in, n);
}

int ss_oracle_state_update_ex(double *state, const double *x, const double *dt,
                              const double *A_log, const double *B, const double *C,
                              const double *D, const double *z, const double *dt_bias,
                              int dt_softplus, int zoh, double *y,
                              int64_t b, int64_t d_in, int64_t n)
{
    if (!state || !x || !dt || !A_log || !B || !C || !D || !y)
        return -1;
    if (b <= 0 || d_in <= 0 || n <= 0)
        return -2;

    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bi = 0; bi < b; bi++) {
        for (int64_t d = 0; d < d_in; d++) {
            int64_t e = bi * d_in + d;
            double dl = step_size(dt[e], dt_bias, d, dt_softplus);
            double yt = 0.0;
            for (int64_t k = 0; k < n; k++) {
                double A = -exp(A_log[d * n + k]);
                double dA = exp(dl * A);
                double dB = input_weight(dl, A, B[bi * n + k], zoh);
                double *h = &state[e * n + k];
                *h = *h * dA + x[e] * dB;               /* in place */
                yt += C[bi * n + k] * *h;
            }
            yt += D[d] * x[e];
            if (z)
                yt *= ss_oracle_silu(z[e]);
            y[e] = yt;
        }
    }
    return 0;
}

int ss_oracle_state_update(double *state, const double *x, const double *dt,
                           const double *A_log, const double *B, const double *C,
                           const double *D, const double *z, const double *dt_bias,
                           int dt_softplus, double *y,
                           int64_t b, int64_t d_in, int64_t n)
{
    return ss_oracle_state_update_ex(state, x, dt, A_log, B, C, D, z, dt_bias, dt_softplus, 0,
                                     y, b, d_in, n);
}

/* One convolution step of Mamba.step (jiafeimiao.top page, "Conv step"):
 *   1. the window conv_state[b, d, 0..W-1] moves one place towards index 0
 *      (torch.roll by -1 along the last axis; the value at index 0 leaves),
 *   2. the new input x[b, d] is written at index W-1,
 *   3. out = sum_w conv_state[b, d, w] * weight[d, w], plus bias[d] when a
 *      bias is given,
 *   4. out = silu(out) when act != 0 (the block's activation).
 * conv_state is updated in place. */
int ss_oracle_conv_update(double *conv_state, const double *x, const double *weight,
                          const double *bias, int act, double *out,
                          int64_t b, int64_t d_in, int64_t W)
{
    if (!conv_state || !x || !weight || !out)
        return -1;
    if (b <= 0 || d_in <= 0 || W <= 0)
        return -2;

    for (int64_t bi = 0; bi < b; bi++) {
        for (int64_t d = 0; d < d_in; d++) {
            double *win = &conv_state[(bi * d_in + d) * W];
            for (int64_t w = 0; w + 1 < W; w++)          /* roll by -1 */
                win[w] = win[w + 1];
            win[W - 1] = x[bi * d_in + d];              /* newest input last */
            double acc = 0.0;
            for (int64_t w = 0; w < W; w++)
                acc += win[w] * weight[d * W + w];
            if (bias)
                acc += bias[d];
            out[bi * d_in + d] = act ? ss_oracle_silu(acc) : acc;
        }
    }
    return 0;
}

/* Map position (row-major index h*W + w of an H x W map) of step t of
 * traversal direction k: 0 row-major, 1 column-major (step t = w*H + h),
 * 2 and 3 the same two orders run backwards. */
static int64_t cross_position(int k, int64_t t, int64_t H, int64_t W)
{
    int64_t s = (k >= 2) ? H * W - 1 - t : t;
    if (k % 2 == 0)
        return s;
    int64_t w = s / H, h = s % H;
    return h * W + w;
}

/* CrossScan, the selective scan of each direction, CrossMerge.
 *   x           : (maps, H, W, d_in)   the feature map, channels last
 *   delta, B, C : (maps, 4, H*W, d_in) and (maps, 4, H*W, n): direction k's
 *                 values in its own step order
 *   A_log       : (4, d_in, n)   D, delta_bias : (4, d_in)   per direction
 *   y           : (maps, H, W, d_in)   sum over the four directions
 *   last_state  : (maps, 4, d_in, n) or NULL
 * Direction k of map m is the scan (ss_oracle_scan_ex, b = 1, zero initial
 * state, Euler input term) of u_k[t] = x[m, position_k(t)]. */
int ss_oracle_cross_scan(const double *x, const double *delta, const double *A_log,
                         const double *B, const double *C, const double *D,
                         const double *delta_bias, int delta_softplus,
                         double *y, double *last_state,
                         int64_t maps, int64_t H, int64_t W, int64_t d_in, int64_t n)
{
    if (!x || !delta || !A_log || !B || !C || !D || !y)
        return -1;
    if (maps <= 0 || H <= 0 || W <= 0 || d_in <= 0 || n <= 0)
        return -2;
    const int64_t L = H * W;
    double *uk = malloc(sizeof(double) * (size_t)(L * d_in));
    double *yk = malloc(sizeof(double) * (size_t)(L * d_in));
    if (!uk || !yk) {
        free(uk);
        free(yk);
        return -3;
    }
    for (int64_t i = 0; i < maps * L * d_in; i++)
        y[i] = 0.0;
    int rc = 0;
    for (int64_t m = 0; m < maps && rc == 0; m++) {
        for (int k = 0; k < 4 && rc == 0; k++) {
            /* CrossScan: direction k's sequence of map positions */
            for (int64_t t = 0; t < L; t++)
                for (int64_t d = 0; d < d_in; d++)
                    uk[t * d_in + d] = x[(m * L + cross_position(k, t, H, W)) * d_in + d];
            int64_t seq = m * 4 + k;
            rc = ss_oracle_scan_ex(uk, delta + seq * L * d_in, A_log + k * d_in * n,
                                   B + seq * L * n, C + seq * L * n, D + k * d_in, NULL,
                                   delta_bias ? delta_bias + k * d_in : NULL, delta_softplus,
                                   NULL, 0, yk, last_state ? last_state + seq * d_in * n : NULL,
                                   1, L, d_in, n);
            /* CrossMerge: add the outputs back where their inputs came from */
            for (int64_t t = 0; t < L; t++)
                for (int64_t d = 0; d < d_in; d++)
                    y[(m * L + cross_position(k, t, H, W)) * d_in + d] += yk[t * d_in + d];
        }
    }
    free(uk);
    free(yk);
    return rc;
}

/* Gradient of the scan (optional h0) for given dy (b, L, d_in) and dlast
 * (b, d_in, n, or NULL for zero).  Per (b, d) channel, with
 * a_tk = exp(Delta_t A_k), the input weight beta_tk (B-bar = beta B:
 * Euler beta = Delta, zero-order hold beta = (exp(Delta A) - 1)/A, mhpn.cn
 * page sections 3.2 and 6), h_tk = a_tk h_(t-1)k + beta_tk B_tk u_t, the
 * pre-gate output y'_t = sum_k C_tk h_tk + D u_t and y_t = y'_t silu(z_t):
 *   dz_t    = dy_t y'_t silu'(z_t),  dy'_t = dy_t silu(z_t)     (dy'_t = dy_t without z)
 *   g_tk    = dL/dh_tk = dy'_t C_tk + a_(t+1)k g_(t+1)k,  g_(L)k = dlast_k
 *   du_t    = dy'_t D + sum_k g_tk beta_tk B_tk
 *   dDelta_t= sum_k g_tk (A_k a_tk h_(t-1)k + dbeta/dDelta B_tk u_t)
 *             (dbeta/dDelta = 1 for Euler, a_tk for the hold)
 *   ddelta_t= dDelta_t softplus'(delta_t + bias) = dDelta_t sigmoid(delta_t + bias)  (dDelta_t without softplus)
 *   dB_tk  += sum_d g_tk beta_tk u_t,   dC_tk += sum_d dy'_t h_tk
 *   dA_log_dk += sum_(b,t) g_tk (Delta_t a_tk h_(t-1)k + dbeta/dA B_tk u_t) A_k   (dA/dA_log = A;
 *             dbeta/dA = 0 for Euler, (Delta a_tk - beta_tk)/A_k for the hold)
 *   dD_d   += sum_(b,t) dy'_t u_t,      dbias_d += sum_(b,t) ddelta_t
 *   dh0_k   = a_0k g_0k
 * Outputs are overwritten (the sums start from zero); dz, ddelta_bias and
 * dh0 may be NULL when z, the bias or h0 are absent. */
int ss_oracle_scan_bwd_ex(const double *u, const double *delta, const double *A_log,
                          const double *B, const double *C, const double *D,
                          const double *z, const double *delta_bias, int delta_softplus,
                          const double *h0, int zoh, const double *dy, const double *dlast,
                          double *du, double *ddelta, double *dA_log, double *dB, double *dC,
                          double *dD, double *dz, double *ddelta_bias, double *dh0,
                          int64_t b, int64_t L, int64_t d_in, int64_t n)
{
    if (!u || !delta || !A_log || !B || !C || !D || !dy || !du || !ddelta || !dA_log || !dB || !dC || !dD)
        return -1;
    if (b <= 0 || L <= 0 || d_in <= 0 || n <= 0)
        return -2;
    double *hs = malloc(sizeof(double) * (size_t)((L + 1) * n));   /* h_(t-1) for t = 0 .. L */
    double *g = malloc(sizeof(double) * (size_t)n);
    double *A = malloc(sizeof(double) * (size_t)n);
    if (!hs || !g || !A) {
        free(hs);
        free(g);
        free(A);
        return -3;
    }
    for (int64_t i = 0; i < b * L * n; i++)
        dB[i] = dC[i] = 0.0;
    for (int64_t i = 0; i < d_in * n; i++)
        dA_log[i] = 0.0;
    for (int64_t d = 0; d < d_in; d++) {
        dD[d] = 0.0;
        if (ddelta_bias)
            ddelta_bias[d] = 0.0;
    }
    for (int64_t bi = 0; bi < b; bi++) {
        for (int64_t d = 0; d < d_in; d++) {
            /* forward again, keeping every state: hs[(t+1) n + k] = h_tk */
            for (int64_t k = 0; k < n; k++) {
                A[k] = -exp(A_log[d * n + k]);
                hs[k] = h0 ? h0[(bi * d_in + d) * n + k] : 0.0;
            }
            for (int64_t t = 0; t < L; t++) {
                int64_t e = (bi * L + t) * d_in + d, r = (bi * L + t) * n;
                double dl = step_size(delta[e], delta_bias, d, delta_softplus);
                for (int64_t k = 0; k < n; k++)
                    hs[(t + 1) * n + k] = exp(dl * A[k]) * hs[t * n + k] + input_weight(dl, A[k], B[r + k], zoh) * u[e];
            }
            /* backward in time */
            for (int64_t k = 0; k < n; k++)
                g[k] = dlast ? dlast[(bi * d_in + d) * n + k] : 0.0;
            for (int64_t t = L - 1; t >= 0; t--) {
                int64_t e = (bi * L + t) * d_in + d, r = (bi * L + t) * n;
                double x = delta[e] + (delta_bias ? delta_bias[d] : 0.0);
                double dl = delta_softplus ? ss_oracle_softplus(x) : x;
                /* the gate: y = y' silu(z) */
                double dyp = dy[e];
                if (z) {
                    double yp = D[d] * u[e];
                    for (int64_t k = 0; k < n; k++)
                        yp += C[r + k] * hs[(t + 1) * n + k];
                    double sg = 1.0 / (1.0 + exp(-z[e]));                  /* sigmoid(z) */
                    dz[e] = dy[e] * yp * sg * (1.0 + z[e] * (1.0 - sg));    /* silu'(z) = s (1 + z (1 - s)) */
                    dyp = dy[e] * z[e] * sg;                                /* dy * silu(z) */
                }
                double dut = dyp * D[d];
                double ddl = 0.0;
                dD[d] += dyp * u[e];
                for (int64_t k = 0; k < n; k++) {
                    double a = exp(dl * A[k]);
                    double hprev = hs[t * n + k];
                    /* the input weight and its derivatives in Delta and in A */
                    double beta = zoh ? expm1(dl * A[k]) / A[k] : dl;
                    double dbeta_ddl = zoh ? a : 1.0;
                    double dbeta_dA = zoh ? (dl * a - beta) / A[k] : 0.0;
                    g[k] += dyp * C[r + k];                   /* dL/dh_tk */
                    dC[r + k] += dyp * hs[(t + 1) * n + k];
                    dB[r + k] += g[k] * beta * u[e];
                    dut += g[k] * beta * B[r + k];
                    ddl += g[k] * (A[k] * a * hprev + dbeta_ddl * B[r + k] * u[e]);
                    dA_log[d * n + k] += g[k] * (dl * a * hprev + dbeta_dA * B[r + k] * u[e]) * A[k];
                    g[k] *= a;                                /* on to h_(t-1) */
                }
                du[e] = dut;
                double dd = delta_softplus ? ddl / (1.0 + exp(-x)) : ddl;   /* softplus' = sigmoid */
                ddelta[e] = dd;
                if (ddelta_bias)
                    ddelta_bias[d] += dd;
            }
            if (dh0)
                for (int64_t k = 0; k < n; k++)
                    dh0[(bi * d_in + d) * n + k] = g[k];
        }
    }
    free(hs);
    free(g);
    free(A);
    return 0;
}

int ss_oracle_scan_bwd(const double *u, const double *delta, const double *A_log,
                       const double *B, const double *C, const double *D,
                       const double *z, const double *delta_bias, int delta_softplus,
                       const double *h0, const double *dy, const double *dlast,
                       double *du, double *ddelta, double *dA_log, double *dB, double *dC,
                       double *dD, double *dz, double *ddelta_bias, double *dh0,
                       int64_t b, int64_t L, int64_t d_in, int64_t n)
{
    return ss_oracle_scan_bwd_ex(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, h0, 0, dy, dlast,
                                 du, ddelta, dA_log, dB, dC, dD, dz, ddelta_bias, dh0, b, L, d_in, n);
}

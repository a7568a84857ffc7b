/*
 * oracle.c -- float64 CPU oracle for the Mamba selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline of the benchmark may load this library.  The GPU product path never
 * calls it and shares no code, header or constant with it.
 *
 * What it computes (plain definition, no blocking, no reordering):
 *
 *   The recurrence and readout are the sequential loop printed in the Hacker
 *   News comments of the page "PyTorch 한 파일에서의 Mamba 구현" (news.hada.io,
 *   mamba-minimal): per time step the state is decayed by deltaA, the input
 *   term deltaB_u is added, and the output is the contraction of the state
 *   with C over the state dimension, one (batch, channel) output per step.
 *   The pages name deltaA and deltaB_u but print no formula for them; the
 *   reading taken here is the one of the selective SSM (Mamba paper,
 *   Section 3 / Algorithm 2, named in the description section of the page
 *   "Mamba SSM 架构"): zero-order hold for A, Euler for B:
 *
 *       x_t      = delta[b,t,d] + dt_bias[d]           (dt_bias may be absent)
 *       Delta_t  = softplus(x_t) if the flag is set, else x_t
 *       a_{t,n}  = exp(Delta_t * A[d,n])
 *       h_{t,n}  = a_{t,n} * h_{t-1,n} + Delta_t * Bm[b,t,n] * u[b,t,d]
 *       s_t      = sum_n Cm[b,t,n] * h_{t,n} + Dskip[d] * u[b,t,d]
 *       y[b,t,d] = s_t * silu(z[b,t,d])                 (z may be absent)
 *
 *   with h_{-1} = h0 (zeros when absent) and h_final = h_{L-1}.
 *
 *   The backward is the analytic adjoint of that recurrence (reverse-time
 *   adjoint scan), evaluated from the full stored history of the forward
 *   in float64 -- no recomputation, no chunking.
 *
 * Layouts (row-major, contiguous):
 *   u, delta, z, y, dy, du, ddelta, dz : (B, L, D)
 *   Bm, Cm, dB, dC                     : (B, L, N)
 *   A, dA                              : (D, N)
 *   Dskip, dt_bias, dD, ddt_bias       : (D)
 *   h0, h_final, dh_final, dh0         : (B, D, N)
 * Every optional input may be NULL; every optional output may be NULL.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the parallel loops below use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* softplus(x) = log(1 + e^x), written in the overflow-free form
 * max(x, 0) + log1p(e^{-|x|}). */
static double sp(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* logistic sigmoid; also the derivative of softplus. */
static double sig(double x) { return 1.0 / (1.0 + exp(-x)); }

/* silu(z) = z * sigmoid(z), the gate applied to the output. */
static double silu(double z) { return z * sig(z); }

static double opt(const double* p, int64_t i) { return p ? p[i] : 0.0; }

/* Discretised step size Delta for one element. */
static double step_size(double delta, const double* dt_bias, int64_t d, int softplus_flag) {
    double x = delta + opt(dt_bias, d);
    return softplus_flag ? sp(x) : x;
}

void oracle_scan_fwd(int64_t B, int64_t L, int64_t D, int64_t N, int softplus_flag,
                     const double* u, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, const double* dt_bias, const double* h0,
                     double* y, double* h_final) {
    #pragma omp parallel for schedule(static)
    for (int64_t bd = 0; bd < B * D; ++bd) {
        const int64_t b = bd / D, d = bd % D;
        double* h = (double*)malloc((size_t)N * sizeof(double));
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t e = (b * L + t) * D + d;     /* element (b,t,d) */
            const int64_t r = (b * L + t) * N;         /* row (b,t,:) of Bm, Cm */
            const double dt = step_size(delta[e], dt_bias, d, softplus_flag);
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double a = exp(dt * A[d * N + n]);
                h[n] = a * h[n] + dt * Bm[r + n] * u[e];
                s += Cm[r + n] * h[n];
            }
            s += opt(Dskip, d) * u[e];
            y[e] = z ? s * silu(z[e]) : s;
        }
        if (h_final)
            for (int64_t n = 0; n < N; ++n) h_final[(b * D + d) * N + n] = h[n];
        free(h);
    }
}

/* One token of the recurrent (RNN) form: the same iteration as one time step
 * of the scan, with the carried state read and overwritten in place.  The
 * step function is the one the page "mamba.py: 一个简单高效的Mamba实现"
 * lists in its updates section (RNN form for inference). */
void oracle_step(int64_t B, int64_t D, int64_t N, int softplus_flag,
                 const double* u_t, const double* delta_t, const double* A,
                 const double* Bm_t, const double* Cm_t, const double* Dskip,
                 const double* z_t, const double* dt_bias,
                 double* state, double* y_t) {
    oracle_scan_fwd(B, 1, D, N, softplus_flag, u_t, delta_t, A, Bm_t, Cm_t, Dskip,
                    z_t, dt_bias, state, y_t, state);
}

/*
 * Analytic adjoint.  For one (b,d), with Delta_t, a_{t,n}, h_{t,n}, s_t as in
 * the forward and g_t = silu(z_t):
 *
 *   sbar_t      = dy_t * g_t                     (dy_t when there is no gate)
 *   zbar_t      = dy_t * s_t * silu'(z_t),  silu'(z) = sig(z) * (1 + z * (1 - sig(z)))
 *   lam_{L-1,n} = sbar_{L-1} Cm_{L-1,n} + dh_final_n
 *   lam_{t,n}   = sbar_t Cm_{t,n} + a_{t+1,n} lam_{t+1,n}     (reverse in time)
 *   du_t        = sbar_t Dskip + Delta_t sum_n lam_{t,n} Bm_{t,n}
 *   dDelta_t    = sum_n lam_{t,n} (A_n a_{t,n} h_{t-1,n} + Bm_{t,n} u_t)
 *   ddelta_t    = dDelta_t * sig(x_t) if softplus else dDelta_t
 *   dA[d,n]    += lam_{t,n} Delta_t a_{t,n} h_{t-1,n}        (sum over b, t)
 *   dB[b,t,n]  += lam_{t,n} Delta_t u_t                      (sum over d)
 *   dC[b,t,n]  += sbar_t h_{t,n}                             (sum over d)
 *   dD[d]      += sbar_t u_t                                 (sum over b, t)
 *   ddt_bias[d]+= ddelta_t                                   (sum over b, t)
 *   dh0_n       = a_{0,n} lam_{0,n}
 *
 * Parallel over the batch index only: every b owns its rows of dB and dC, and
 * the per-channel sums over b are formed afterwards in ascending b, so the
 * result does not depend on the thread count.
 */
void oracle_scan_bwd(int64_t B, int64_t L, int64_t D, int64_t N, int softplus_flag,
                     const double* u, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, const double* dt_bias, const double* h0,
                     const double* dy, const double* dh_final,
                     double* du, double* ddelta, double* dA, double* dB, double* dC,
                     double* dD, double* dz, double* ddt_bias, double* dh0) {
    /* per-batch partial sums of the per-channel gradients */
    double* pA = (double*)calloc((size_t)(B * D * N), sizeof(double));
    double* pD = (double*)calloc((size_t)(B * D), sizeof(double));
    double* pbias = (double*)calloc((size_t)(B * D), sizeof(double));

    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        double* H = (double*)malloc((size_t)((L + 1) * N) * sizeof(double)); /* H[(t+1)*N+n] = h_{t,n} */
        double* Aa = (double*)malloc((size_t)(L * N) * sizeof(double));      /* a_{t,n} */
        double* dts = (double*)malloc((size_t)L * sizeof(double));
        double* xs = (double*)malloc((size_t)L * sizeof(double));
        double* ss = (double*)malloc((size_t)L * sizeof(double));
        double* lam = (double*)malloc((size_t)N * sizeof(double));
        for (int64_t t = 0; t < L; ++t)
            for (int64_t n = 0; n < N; ++n) dB[(b * L + t) * N + n] = 0.0, dC[(b * L + t) * N + n] = 0.0;

        for (int64_t d = 0; d < D; ++d) {
            /* forward, keeping the whole history */
            for (int64_t n = 0; n < N; ++n) H[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t e = (b * L + t) * D + d, r = (b * L + t) * N;
                xs[t] = delta[e] + opt(dt_bias, d);
                dts[t] = softplus_flag ? sp(xs[t]) : xs[t];
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = exp(dts[t] * A[d * N + n]);
                    Aa[t * N + n] = a;
                    H[(t + 1) * N + n] = a * H[t * N + n] + dts[t] * Bm[r + n] * u[e];
                    s += Cm[r + n] * H[(t + 1) * N + n];
                }
                ss[t] = s + opt(Dskip, d) * u[e];
            }
            /* reverse adjoint */
            for (int64_t n = 0; n < N; ++n) lam[n] = dh_final ? dh_final[(b * D + d) * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t e = (b * L + t) * D + d, r = (b * L + t) * N;
                double sbar;
                if (z) {
                    const double zz = z[e], sg = sig(zz);
                    sbar = dy[e] * zz * sg;
                    if (dz) dz[e] = dy[e] * ss[t] * sg * (1.0 + zz * (1.0 - sg));
                } else {
                    sbar = dy[e];
                }
                if (t < L - 1)
                    for (int64_t n = 0; n < N; ++n) lam[n] *= Aa[(t + 1) * N + n];
                double lb = 0.0, dDelta = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    lam[n] += sbar * Cm[r + n];
                    const double hp = H[t * N + n];          /* h_{t-1,n} */
                    const double q = lam[n] * Aa[t * N + n] * hp;
                    lb += lam[n] * Bm[r + n];
                    dDelta += A[d * N + n] * q + lam[n] * Bm[r + n] * u[e];
                    pA[(b * D + d) * N + n] += q * dts[t];
                    dB[r + n] += lam[n] * dts[t] * u[e];
                    dC[r + n] += sbar * H[(t + 1) * N + n];
                }
                du[e] = sbar * opt(Dskip, d) + dts[t] * lb;
                const double dx = softplus_flag ? dDelta * sig(xs[t]) : dDelta;
                ddelta[e] = dx;
                pD[b * D + d] += sbar * u[e];
                pbias[b * D + d] += dx;
            }
            if (dh0)
                for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = Aa[n] * lam[n];
        }
        free(H); free(Aa); free(dts); free(xs); free(ss); free(lam);
    }
    for (int64_t d = 0; d < D; ++d) {
        double sD = 0.0, sbias = 0.0;
        for (int64_t b = 0; b < B; ++b) { sD += pD[b * D + d]; sbias += pbias[b * D + d]; }
        if (dD) dD[d] = sD;
        if (ddt_bias) ddt_bias[d] = sbias;
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t b = 0; b < B; ++b) s += pA[(b * D + d) * N + n];
            dA[d * N + n] = s;
        }
    }
    free(pA); free(pD); free(pbias);
}

/*
 * naju_oracle.c -- plain, slow, fp64 CPU oracle of the Naju native-discrete
 * selective scan and of the mixer-block pieces fused around it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path
 * (the HIP library and its Python binding) never calls it and shares no
 * code, header, table or helper with it.
 *
 * What it computes (sources: the Naju pages, cited by title and section):
 *
 *   Recurrence ("Core equations", reproduction README of arXiv 2607.21000):
 *       x_n = f_n (.) x_{n-1} + i_n (.) (h_n B_n^T),  f_n = sigma(a_n),
 *       i_n = sigma(b_n)
 *     with, per batch row and channel c, a state row x_n[c, 0..N-1];
 *     f, i, h are per (token, channel) and broadcast over the state index,
 *     B_n is one N-vector per (batch, token) shared by all channels.
 *   Readout (same section, second equation):
 *       ys_n[c] = (1/sqrt(N)) sum_s x_n[c,s] C_n[s] + D[c] h_n[c]
 *     using the post-update state x_n.
 *   Block front end ("Background and main changes" and the block flowchart
 *   of the same page): causal depthwise convolution followed by SiLU,
 *       pre_n[c] = sum_{k=0}^{K-1} w[c,k] u_{n-K+1+k}[c],   h = pre*sigma(pre)
 *     with u_m for m < 0 taken from conv_state (zeros if absent).
 *   Output modulation (same flowchart): y_n = ys_n * SiLU(z_n).
 *
 * The backward functions are reverse-mode differentiation of exactly these
 * definitions, written as a plain reverse time loop over a stored state
 * history.  Cross-channel reductions (dB, dC) are stored per channel and
 * summed afterwards in ascending channel order; cross-token reductions
 * (dD, dconv_w) are summed in ascending (batch, token) order.
 *
 * Layouts (row-major, all fp64):
 *   per (token, channel): [Bt][L][Di]     per token: [Bt][L][N]
 *   states x0, x_final:   [Bt][Di][N]     D: [Di]   conv_w: [Di][K]
 *   conv_state:           [Bt][K-1][Di]   (the K-1 inputs preceding u_0)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* sigma(v) = 1/(1+e^{-v}); the two branches keep exp() from overflowing
 * and give sigma(+inf)=1, sigma(-inf)=0 exactly; NaN propagates. */
static double sigm(double v)
{
    if (v >= 0.0) return 1.0 / (1.0 + exp(-v));
    double e = exp(v);
    return e / (1.0 + e);
}

/* d sigma / dv written as sigma(v) sigma(-v) (no 1 - sigma cancellation). */
static double dsigm(double v) { return sigm(v) * sigm(-v); }

static double silu(double v) { return v * sigm(v); }

/* d SiLU / dv = sigma(v) + v sigma(v) sigma(-v) */
static double dsilu(double v) { return sigm(v) + v * sigm(v) * sigm(-v); }

/* ------------------------------------------------------------------ */
/* Scan forward.                                                        */
/* ------------------------------------------------------------------ */
void naju_oracle_scan_fwd(int64_t Bt, int64_t L, int64_t Di, int64_t N,
                          const double *h, const double *a, const double *b,
                          const double *Bm, const double *Cm, const double *D,
                          const double *x0, /* may be NULL = zeros */
                          double *ys, double *x_final /* may be NULL */)
{
    const double scale = 1.0 / sqrt((double)N);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < Bt; ++bb) {
        for (int64_t c = 0; c < Di; ++c) {
            double *x = (double *)malloc(sizeof(double) * (size_t)N);
            for (int64_t s = 0; s < N; ++s)
                x[s] = x0 ? x0[(bb * Di + c) * N + s] : 0.0;
            for (int64_t n = 0; n < L; ++n) {
                const int64_t t = (bb * L + n) * Di + c;
                const double *Bn = Bm + (bb * L + n) * N;
                const double *Cn = Cm + (bb * L + n) * N;
                const double f = sigm(a[t]);
                const double i = sigm(b[t]);
                double acc = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    x[s] = f * x[s] + i * (h[t] * Bn[s]);
                    acc += x[s] * Cn[s];
                }
                ys[t] = scale * acc + D[c] * h[t];
            }
            if (x_final)
                for (int64_t s = 0; s < N; ++s) x_final[(bb * Di + c) * N + s] = x[s];
            free(x);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Scan backward.                                                       */
/*   g        = dLoss/dys            [Bt][L][Di]                        */
/*   dx_final = dLoss/dx_L           [Bt][Di][N] or NULL (= 0)          */
/* Adjoint of the state, lam_n = dLoss/dx_n (through all later uses):   */
/*   lam_{L-1} = dx_final + g_{L-1} C_{L-1}/sqrt(N)                     */
/*   lam_n     = f_{n+1} lam_{n+1} + g_n C_n/sqrt(N)                    */
/* and per token, with x_{n-1} the state before token n:               */
/*   dLoss/df_n = <lam_n, x_{n-1}>,   dLoss/dw_n = <lam_n, B_n>,        */
/*   w_n = i_n h_n,  dB_n += lam_n w_n,  dC_n += g_n x_n / sqrt(N).     */
/* ------------------------------------------------------------------ */
void naju_oracle_scan_bwd(int64_t Bt, int64_t L, int64_t Di, int64_t N,
                          const double *h, const double *a, const double *b,
                          const double *Bm, const double *Cm, const double *D,
                          const double *x0, /* may be NULL */
                          const double *g, const double *dx_final, /* may be NULL */
                          double *dh, double *da, double *db,
                          double *dB, double *dC, /* [Bt][L][N] */
                          double *dD,             /* [Di] */
                          double *dx0 /* may be NULL */)
{
    const double scale = 1.0 / sqrt((double)N);
    /* per-channel contributions of one batch row, reduced afterwards */
    double *cB = (double *)malloc(sizeof(double) * (size_t)(Di * L * N));
    double *cC = (double *)malloc(sizeof(double) * (size_t)(Di * L * N));
    for (int64_t c = 0; c < Di; ++c) dD[c] = 0.0;

    for (int64_t bb = 0; bb < Bt; ++bb) {
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < Di; ++c) {
            /* state history xs[n] = state before token n, n = 0..L */
            double *xs = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
            double *lam = (double *)malloc(sizeof(double) * (size_t)N);
            for (int64_t s = 0; s < N; ++s) xs[s] = x0 ? x0[(bb * Di + c) * N + s] : 0.0;
            for (int64_t n = 0; n < L; ++n) {
                const int64_t t = (bb * L + n) * Di + c;
                const double *Bn = Bm + (bb * L + n) * N;
                const double f = sigm(a[t]);
                const double i = sigm(b[t]);
                for (int64_t s = 0; s < N; ++s)
                    xs[(n + 1) * N + s] = f * xs[n * N + s] + i * (h[t] * Bn[s]);
            }
            for (int64_t s = 0; s < N; ++s)
                lam[s] = dx_final ? dx_final[(bb * Di + c) * N + s] : 0.0;
            double dDc = 0.0;
            for (int64_t n = L - 1; n >= 0; --n) {
                const int64_t t = (bb * L + n) * Di + c;
                const double *Bn = Bm + (bb * L + n) * N;
                const double *Cn = Cm + (bb * L + n) * N;
                const double i = sigm(b[t]);
                const double w = i * h[t];
                /* lam currently holds f_{n+1} lam_{n+1} (+ dx_final at n=L-1) */
                for (int64_t s = 0; s < N; ++s) lam[s] += g[t] * scale * Cn[s];
                double df = 0.0, dw = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    df += lam[s] * xs[n * N + s];
                    dw += lam[s] * Bn[s];
                    cB[(c * L + n) * N + s] = lam[s] * w;
                    cC[(c * L + n) * N + s] = g[t] * scale * xs[(n + 1) * N + s];
                }
                da[t] = df * dsigm(a[t]);
                db[t] = dw * h[t] * dsigm(b[t]);
                dh[t] = dw * i + D[c] * g[t];
                dDc += g[t] * h[t];
                const double f = sigm(a[t]);
                for (int64_t s = 0; s < N; ++s) lam[s] *= f;
            }
            /* lam now holds f_0 lam_0 = dLoss/dx0 */
            if (dx0)
                for (int64_t s = 0; s < N; ++s) dx0[(bb * Di + c) * N + s] = lam[s];
            dD[c] += dDc;
            free(xs);
            free(lam);
        }
        /* channel reductions in ascending channel order */
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < L; ++n) {
            for (int64_t s = 0; s < N; ++s) {
                double sb = 0.0, sc = 0.0;
                for (int64_t c = 0; c < Di; ++c) {
                    sb += cB[(c * L + n) * N + s];
                    sc += cC[(c * L + n) * N + s];
                }
                dB[(bb * L + n) * N + s] = sb;
                dC[(bb * L + n) * N + s] = sc;
            }
        }
    }
    free(cB);
    free(cC);
}

/* ------------------------------------------------------------------ */
/* Causal depthwise convolution + SiLU (block front end).               */
/*   pre_n[c] = sum_k w[c,k] u_{n-K+1+k}[c];  h = SiLU(pre)             */
/* ------------------------------------------------------------------ */
static double u_at(const double *u, const double *conv_state, int64_t bb, int64_t m,
                   int64_t L, int64_t Di, int64_t K, int64_t c)
{
    if (m >= 0) return u[(bb * L + m) * Di + c];
    /* m in [-(K-1), -1]  ->  conv_state row m + K - 1 */
    if (!conv_state || m < -(K - 1)) return 0.0;
    return conv_state[(bb * (K - 1) + (m + K - 1)) * Di + c];
}

void naju_oracle_conv_silu(int64_t Bt, int64_t L, int64_t Di, int64_t K,
                           const double *u, const double *w, const double *conv_state,
                           double *pre, double *h)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < Bt; ++bb)
        for (int64_t n = 0; n < L; ++n)
            for (int64_t c = 0; c < Di; ++c) {
                double p = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    p += w[c * K + k] * u_at(u, conv_state, bb, n - K + 1 + k, L, Di, K, c);
                pre[(bb * L + n) * Di + c] = p;
                h[(bb * L + n) * Di + c] = silu(p);
            }
}

/* ------------------------------------------------------------------ */
/* Block forward:  y = ScanReadout(SiLU(conv(u)), a, b, B, C, D) * SiLU(z) */
/* Also returns the final state and the conv state for a following call  */
/* (the last K-1 inputs of the concatenation [conv_state; u]).           */
/* ------------------------------------------------------------------ */
void naju_oracle_block_fwd(int64_t Bt, int64_t L, int64_t Di, int64_t N, int64_t K,
                           const double *u, const double *z, const double *w,
                           const double *conv_state, /* may be NULL */
                           const double *a, const double *b, const double *Bm,
                           const double *Cm, const double *D, const double *x0,
                           double *y, double *x_final, double *conv_state_out /* may be NULL */)
{
    const size_t nt = (size_t)(Bt * L * Di);
    double *pre = (double *)malloc(sizeof(double) * nt);
    double *h = (double *)malloc(sizeof(double) * nt);
    double *ys = (double *)malloc(sizeof(double) * nt);
    naju_oracle_conv_silu(Bt, L, Di, K, u, w, conv_state, pre, h);
    naju_oracle_scan_fwd(Bt, L, Di, N, h, a, b, Bm, Cm, D, x0, ys, x_final);
    for (size_t t = 0; t < nt; ++t) y[t] = ys[t] * silu(z[t]);
    if (conv_state_out)
        for (int64_t bb = 0; bb < Bt; ++bb)
            for (int64_t j = 0; j < K - 1; ++j)
                for (int64_t c = 0; c < Di; ++c)
                    conv_state_out[(bb * (K - 1) + j) * Di + c] =
                        u_at(u, conv_state, bb, L - (K - 1) + j, L, Di, K, c);
    free(pre);
    free(h);
    free(ys);
}

/* ------------------------------------------------------------------ */
/* Block backward (chain rule through modulation, scan, SiLU and conv). */
/*   gs = dy * SiLU(z),  dz = dy * ys * SiLU'(z)                        */
/*   dpre = dh * SiLU'(pre)                                             */
/*   du_m = sum_k w[c,k] dpre_{m+K-1-k}  (terms with index >= L vanish) */
/*   dw[c,k] = sum_{b,n} dpre_n u_{n-K+1+k}                             */
/*   dconv_state[j] = du at time index j-(K-1)                          */
/* ------------------------------------------------------------------ */
void naju_oracle_block_bwd(int64_t Bt, int64_t L, int64_t Di, int64_t N, int64_t K,
                           const double *u, const double *z, const double *w,
                           const double *conv_state, const double *a, const double *b,
                           const double *Bm, const double *Cm, const double *D,
                           const double *x0, const double *dy, const double *dx_final,
                           double *du, double *dz, double *dw, double *dconv_state,
                           double *da, double *db, double *dB, double *dC, double *dD,
                           double *dx0)
{
    const size_t nt = (size_t)(Bt * L * Di);
    double *pre = (double *)malloc(sizeof(double) * nt);
    double *h = (double *)malloc(sizeof(double) * nt);
    double *ys = (double *)malloc(sizeof(double) * nt);
    double *gs = (double *)malloc(sizeof(double) * nt);
    double *dh = (double *)malloc(sizeof(double) * nt);
    double *dpre = (double *)malloc(sizeof(double) * nt);
    naju_oracle_conv_silu(Bt, L, Di, K, u, w, conv_state, pre, h);
    naju_oracle_scan_fwd(Bt, L, Di, N, h, a, b, Bm, Cm, D, x0, ys, NULL);
    for (size_t t = 0; t < nt; ++t) {
        gs[t] = dy[t] * silu(z[t]);
        dz[t] = dy[t] * ys[t] * dsilu(z[t]);
    }
    naju_oracle_scan_bwd(Bt, L, Di, N, h, a, b, Bm, Cm, D, x0, gs, dx_final,
                         dh, da, db, dB, dC, dD, dx0);
    for (size_t t = 0; t < nt; ++t) dpre[t] = dh[t] * dsilu(pre[t]);

#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < Di; ++c) {
        for (int64_t k = 0; k < K; ++k) {
            double acc = 0.0;
            for (int64_t bb = 0; bb < Bt; ++bb)
                for (int64_t n = 0; n < L; ++n)
                    acc += dpre[(bb * L + n) * Di + c] *
                           u_at(u, conv_state, bb, n - K + 1 + k, L, Di, K, c);
            dw[c * K + k] = acc;
        }
        for (int64_t bb = 0; bb < Bt; ++bb) {
            /* input time index m in [-(K-1), L-1] */
            for (int64_t m = -(K - 1); m < L; ++m) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t n = m + K - 1 - k;
                    if (n >= 0 && n < L) acc += w[c * K + k] * dpre[(bb * L + n) * Di + c];
                }
                if (m >= 0)
                    du[(bb * L + m) * Di + c] = acc;
                else if (dconv_state)
                    dconv_state[(bb * (K - 1) + (m + K - 1)) * Di + c] = acc;
            }
        }
    }
    free(pre);
    free(h);
    free(ys);
    free(gs);
    free(dh);
    free(dpre);
}

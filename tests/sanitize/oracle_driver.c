/*
 * Runs every function of the fp64 oracle (oracle/naju_oracle.c) on small
 * seeded inputs -- several shapes, with and without each optional argument --
 * for a build under AddressSanitizer and UndefinedBehaviorSanitizer.  It checks
 * only that every output is finite; the values are checked elsewhere (the
 * oracle's pins).  Exit status 0 on success, 2 on a non-finite output.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void naju_oracle_scan_fwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *,
                          const double *, const double *, const double *, const double *,
                          const double *, double *, double *);
void naju_oracle_scan_bwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *,
                          const double *, const double *, const double *, const double *,
                          const double *, const double *, const double *, double *, double *,
                          double *, double *, double *, double *, double *);
void naju_oracle_conv_silu(int64_t, int64_t, int64_t, int64_t, const double *, const double *,
                           const double *, double *, double *);
void naju_oracle_block_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, const double *,
                           const double *, const double *, const double *, const double *,
                           const double *, const double *, const double *, const double *,
                           const double *, double *, double *, double *);
void naju_oracle_block_bwd(int64_t, int64_t, int64_t, int64_t, int64_t, const double *,
                           const double *, const double *, const double *, const double *,
                           const double *, const double *, const double *, const double *,
                           const double *, const double *, const double *, double *, double *,
                           double *, double *, double *, double *, double *, double *, double *,
                           double *);

static uint64_t rng = 0x9E3779B97F4A7C15ull;

/* uniform in [lo, hi) from a 64-bit linear congruential generator */
static double uni(double lo, double hi)
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}

/* exactly n doubles (malloc'd even for n == 0, so every pointer is valid) */
static double *arr(size_t n, double lo, double hi)
{
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = uni(lo, hi);
    return p;
}

static int finite_all(const char *what, const double *p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) {
            fprintf(stderr, "%s[%zu] is not finite\n", what, i);
            return 0;
        }
    return 1;
}

static int run(int64_t Bt, int64_t L, int64_t Di, int64_t N, int with_opt)
{
    const int64_t K = 4;
    const size_t nt = (size_t)(Bt * L * Di), nb = (size_t)(Bt * L * N), ns = (size_t)(Bt * Di * N);
    const size_t nc = (size_t)(Bt * (K - 1) * Di);
    double *h = arr(nt, -1, 1), *a = arr(nt, 3, 7), *b = arr(nt, -3, -1), *B = arr(nb, -1, 1);
    double *C = arr(nb, -1, 1), *D = arr((size_t)Di, -1, 1), *z = arr(nt, -1, 1);
    double *w = arr((size_t)(Di * K), -0.5, 0.5), *g = arr(nt, -1, 1);
    double *x0 = with_opt ? arr(ns, -1, 1) : NULL, *dxf = with_opt ? arr(ns, -1, 1) : NULL;
    double *cs = with_opt ? arr(nc, -1, 1) : NULL;
    double *y = arr(nt, 0, 0), *xf = arr(ns, 0, 0), *pre = arr(nt, 0, 0), *hh = arr(nt, 0, 0);
    double *cso = with_opt ? arr(nc, 0, 0) : NULL;
    double *d1 = arr(nt, 0, 0), *d2 = arr(nt, 0, 0), *d3 = arr(nt, 0, 0), *d4 = arr(nt, 0, 0);
    double *dB = arr(nb, 0, 0), *dC = arr(nb, 0, 0), *dD = arr((size_t)Di, 0, 0);
    double *dx0 = with_opt ? arr(ns, 0, 0) : NULL, *dw = arr((size_t)(Di * K), 0, 0);
    double *dcs = with_opt ? arr(nc, 0, 0) : NULL;
    int ok = 1;

    naju_oracle_scan_fwd(Bt, L, Di, N, h, a, b, B, C, D, x0, y, with_opt ? xf : NULL);
    ok &= finite_all("scan y", y, nt) && finite_all("scan x_final", xf, ns);
    naju_oracle_scan_bwd(Bt, L, Di, N, h, a, b, B, C, D, x0, g, dxf, d1, d2, d3, dB, dC, dD, dx0);
    ok &= finite_all("scan dh", d1, nt) && finite_all("scan da", d2, nt) &&
          finite_all("scan db", d3, nt) && finite_all("scan dB", dB, nb) &&
          finite_all("scan dC", dC, nb) && finite_all("scan dD", dD, (size_t)Di);
    if (dx0) ok &= finite_all("scan dx0", dx0, ns);
    naju_oracle_conv_silu(Bt, L, Di, K, h, w, cs, pre, hh);
    ok &= finite_all("conv pre", pre, nt) && finite_all("conv h", hh, nt);
    naju_oracle_block_fwd(Bt, L, Di, N, K, h, z, w, cs, a, b, B, C, D, x0, y, xf, cso);
    ok &= finite_all("block y", y, nt) && finite_all("block x_final", xf, ns);
    if (cso) ok &= finite_all("block conv_state_out", cso, nc);
    naju_oracle_block_bwd(Bt, L, Di, N, K, h, z, w, cs, a, b, B, C, D, x0, g, dxf, d1, d4, dw, dcs,
                          d2, d3, dB, dC, dD, dx0);
    ok &= finite_all("block du", d1, nt) && finite_all("block dz", d4, nt) &&
          finite_all("block dw", dw, (size_t)(Di * K)) && finite_all("block da", d2, nt) &&
          finite_all("block db", d3, nt) && finite_all("block dB", dB, nb) &&
          finite_all("block dC", dC, nb) && finite_all("block dD", dD, (size_t)Di);
    if (dcs) ok &= finite_all("block dconv_state", dcs, nc);

    double *all[] = {h, a, b, B, C, D, z, w, g, x0, dxf, cs, y, xf, pre, hh, cso,
                     d1, d2, d3, d4, dB, dC, dD, dx0, dw, dcs};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
    return ok;
}

int main(void)
{
    /* Bt, L, Di, N: ragged lengths, one token, a single channel, both state sizes */
    static const int64_t shapes[][4] = {{2, 37, 5, 16}, {1, 1, 3, 64}, {3, 5, 1, 16},
                                        {1, 70, 8, 64}, {2, 0, 4, 16}};
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
        for (int opt = 0; opt < 2; ++opt)
            if (!run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], opt)) return 2;
    printf("oracle driver: ok\n");
    return 0;
}

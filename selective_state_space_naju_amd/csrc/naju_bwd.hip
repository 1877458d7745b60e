// naju_bwd.hip -- reverse mode of the Naju selective scan (scan and block).
//
// Differentiates the "Core equations" of the Naju reproduction README
// (arXiv 2607.21000) and the block flowchart of that page.  With
// g_n = dLoss/dys_n (block: dy_n SiLU(z_n)) the state adjoint
// lam_n = dLoss/dx_n obeys the reverse-time affine recurrence
//     lam_n = f_{n+1} lam_{n+1} + g_n C_n / sqrt(N),   lam_{L-1} += dx_final,
// and per token
//     dLoss/df_n = <lam_n, x_{n-1}>,  dLoss/dw_n = <lam_n, B_n>  (w_n = i_n h_n),
//     dB_n = sum_c lam_n[c,:] w_n[c],  dC_n = sum_c g_n[c] x_n[c,:] / sqrt(N),
//     dD = sum g h,  dx0 = f_0 lam_0.
//
// Decomposition (same waves as the forward; tickets run from the last chunk
// to the first so that look-back goes towards the end of the sequence):
//   pass F  each wave starts from its checkpointed entering state, runs the
//           recurrence over its T tokens and keeps the states at every TB-th
//           token; in the same sweep it accumulates the reverse pair
//           (Q, R): mu_out = Q mu_in + R, where mu_in = f_{t1} lam_{t1} is the
//           adjoint flowing in from after the wave and mu_out = f_{t0} lam_{t0};
//   carry   the pairs are composed across the workgroup's waves (LDS) and across
//           workgroups (decoupled look-back in reverse), giving every wave mu_in;
//   pass G  sub-blocks of TB tokens are visited last to first: their states are
//           recomputed from the kept ones, then the adjoint runs backwards over
//           them producing the per-token gradients.  Channel sums (dB, dC) are
//           reduced across the wave's lanes and written as per-tile partials;
//           token sums (dD, dconv_w) as per-wave partials.  Small follow-up
//           kernels reduce the partials in a fixed order (deterministic) and
//           complete the convolution transpose across wave boundaries.
#include <stdlib.h>

#include "naju_device.h"
#include "naju_launch.h"

namespace naju {

// Reduce-scatter of v[16] over the lanes that differ in bits 2..5 (and, when
// FULL, also bits 0..1).  Afterwards v[0] of lane l holds the sum of original
// index  8*b5 + 4*b4 + 2*b3 + b2  (bK = bit K of l).
template <bool FULL>
__device__ __forceinline__ float reduce_scatter16(float (&v)[16], int lane)
{
#pragma unroll
    for (int lvl = 0; lvl < 4; ++lvl) {
        const int m = 32 >> lvl;  // 32, 16, 8, 4
        const int h = 8 >> lvl;   // 8, 4, 2, 1
        const bool hi = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float send = hi ? v[i] : v[i + h];
            const float keep = hi ? v[i + h] : v[i];
            v[i] = keep + __shfl_xor(send, m);
        }
    }
    float r = v[0];
    if constexpr (FULL) {
        r += __shfl_xor(r, 2);
        r += __shfl_xor(r, 1);
    }
    return r;
}

template <typename IO, int N, bool BLOCK>
__global__ __launch_bounds__(64 * kBwdW) void bwd_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_chunks,
    const int64_t n_waves, const float scale, const IO *__restrict__ hu,
    const IO *__restrict__ a, const IO *__restrict__ bg, const IO *__restrict__ Bm,
    const IO *__restrict__ Cm, const float *__restrict__ D, const IO *__restrict__ z,
    const float *__restrict__ conv_w, const IO *__restrict__ conv_state,
    const float *__restrict__ ckpt, const IO *__restrict__ dy,
    const float *__restrict__ dx_final, IO *__restrict__ dhu, IO *__restrict__ da,
    IO *__restrict__ db, IO *__restrict__ dz, float *__restrict__ dx0, WsHeader *hdr,
    uint32_t *flags, float *agg, float *incl, float *__restrict__ bc_part,
    float *__restrict__ dd_part, float *__restrict__ dw_part, float *__restrict__ edge)
{
    constexpr int T = kBwdT, W = kBwdW, TB = kBwdTB, NSB = T / TB;
    constexpr int LPC = N / 16;
    constexpr int CPW = 64 / LPC;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;

    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ float sQ[W][64];
    __shared__ float sR[W][16][64];
    __shared__ float sMu[16][64];
    // states entering sub-blocks 1..NSB-1 of every wave (sub-block 0 starts
    // from the checkpoint itself)
    __shared__ float sXB[W][NSB - 1][16][64];

    if (threadIdx.x == 0) {
        s_ticket = add_agent(&hdr->ticket, 1u);
        s_epoch = (ld_agent(&hdr->epoch) + 1u) & 0x3FFFFFFFu;
    }
    __syncthreads();
    const uint32_t ticket = s_ticket;
    const uint32_t ep = s_epoch;
    const uint32_t per_chunk = (uint32_t)(Bt * n_tiles);
    const int chunk = n_chunks - 1 - (int)(ticket / per_chunk);
    const int rem = (int)(ticket % per_chunk);
    const int bi = rem / n_tiles;
    const int tile = rem % n_tiles;

    const int sg = lane % LPC;
    const int64_t c = (int64_t)tile * CPW + lane / LPC;
    const bool valid = c < Di;
    const int64_t n0 = (int64_t)chunk * (W * T) + (int64_t)wv * T;
    const int64_t wrow = (int64_t)chunk * W + wv;
    const bool active = n0 < L;
    const float Dc = valid ? D[c] : 0.f;
    const float *ck = ckpt + ((int64_t)bi * n_waves + wrow) * N * Di + (int64_t)sg * 16 * Di + c;

    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
    if constexpr (BLOCK) {
        if (valid) {
            w0 = conv_w[c * 4 + 0];
            w1 = conv_w[c * 4 + 1];
            w2 = conv_w[c * 4 + 2];
            w3 = conv_w[c * 4 + 3];
        }
    }
    // u at absolute token m (conv_state for m < 0, zero without it)
    auto u_at = [&](int64_t m) -> float {
        if (!valid) return 0.f;
        if (m >= 0) return (m < L) ? to_f(hu[((int64_t)bi * L + m) * Di + c]) : 0.f;
        if (m >= -3 && conv_state) return to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
        return 0.f;
    };

    // -------------------------------------------------------------- pass F
    float x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = (active && valid) ? ck[(int64_t)s * Di] : 0.f;
    float Q = 1.f, R[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) R[s] = 0.f;
    {
        float um1 = 0.f, um2 = 0.f, um3 = 0.f;
        if constexpr (BLOCK) {
            um1 = u_at(n0 - 1);
            um2 = u_at(n0 - 2);
            um3 = u_at(n0 - 3);
        }
#pragma unroll
        for (int j = 0; j < T; ++j) {
            if (j % TB == 0 && j > 0) {
#pragma unroll
                for (int s = 0; s < 16; ++s) sXB[wv][j / TB - 1][s][lane] = x[s];
            }
            const int64_t n = n0 + j;
            if (n < L) {
                const int64_t t = ((int64_t)bi * L + n) * Di + c;
                float av = 0.f, bv = 0.f, hv = 0.f, gv = 0.f;
                if (valid) {
                    av = to_f(a[t]);
                    bv = to_f(bg[t]);
                    gv = to_f(dy[t]);
                    if constexpr (BLOCK) {
                        const float uv = to_f(hu[t]);
                        const float pre = w0 * um3 + w1 * um2 + w2 * um1 + w3 * uv;
                        um3 = um2;
                        um2 = um1;
                        um1 = uv;
                        hv = pre * sigm(pre);
                        const float zv = to_f(z[t]);
                        gv *= zv * sigm(zv);
                    } else {
                        hv = to_f(hu[t]);
                    }
                }
                const float f = sigm(av);
                const float wr = sigm(bv) * hv;
                const IO *Bn = Bm + ((int64_t)bi * L + n) * N + sg * 16;
                const IO *Cn = Cm + ((int64_t)bi * L + n) * N + sg * 16;
                Q *= f;
                const float qg = Q * gv * scale;
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    x[s] = fmaf(f, x[s], wr * to_f(Bn[s]));
                    R[s] = fmaf(qg, to_f(Cn[s]), R[s]);
                }
            }
        }
    }

    // ------------------------------------------ carry: compose reverse pairs
    sQ[wv][lane] = Q;
#pragma unroll
    for (int s = 0; s < 16; ++s) sR[wv][s][lane] = R[s];
    __syncthreads();

    // suffix of the waves after this one: mu_in(wave) = Qs mu_in(workgroup) + Rs
    float Qs = 1.f, Rs[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) Rs[s] = 0.f;
    for (int w = W - 1; w > wv; --w) {
        const float qw = sQ[w][lane];
#pragma unroll
        for (int s = 0; s < 16; ++s) Rs[s] = fmaf(qw, Rs[s], sR[w][s][lane]);
        Qs *= qw;
    }

    if (wv == 0) {
        float Qt = 1.f, Rt[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) Rt[s] = 0.f;
        for (int w = W - 1; w >= 0; --w) {
            const float qw = sQ[w][lane];
#pragma unroll
            for (int s = 0; s < 16; ++s) Rt[s] = fmaf(qw, Rt[s], sR[w][s][lane]);
            Qt *= qw;
        }
        const size_t me = ((size_t)bi * n_tiles + tile) * n_chunks + chunk;
        float mu[16];
        if (chunk == n_chunks - 1) {
#pragma unroll
            for (int s = 0; s < 16; ++s)
                mu[s] = (dx_final && valid) ? dx_final[(bi * Di + c) * N + sg * 16 + s] : 0.f;
        } else {
            float *ag = agg + me * (17 * 64);
            st_agent(ag + lane, Qt);
#pragma unroll
            for (int s = 0; s < 16; ++s) st_agent(ag + (1 + s) * 64 + lane, Rt[s]);
            wait_mem();
            if (lane == 0) st_agent(&flags[me], make_flag(ep, kFlagAgg));
            float accQ = 1.f, accR[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) accR[s] = 0.f;
            size_t j = me + 1;
            for (;;) {
                const uint32_t st = wait_flag(&flags[j], ep, hdr);
                if (st == kFlagIncl) {
                    const float *in = incl + j * (16 * 64);
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        mu[s] = fmaf(accQ, ld_agent(in + s * 64 + lane), accR[s]);
                    break;
                }
                const float *pa = agg + j * (17 * 64);
                const float qj = ld_agent(pa + lane);
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    accR[s] = fmaf(accQ, ld_agent(pa + (1 + s) * 64 + lane), accR[s]);
                accQ *= qj;
                ++j;  // the last chunk always publishes an inclusive value
            }
        }
        float *ic = incl + me * (16 * 64);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const float mo = fmaf(Qt, mu[s], Rt[s]);
            st_agent(ic + s * 64 + lane, mo);
            if (chunk == 0 && dx0 && valid) dx0[(bi * Di + c) * N + sg * 16 + s] = mo;
        }
        wait_mem();
        if (lane == 0) st_agent(&flags[me], make_flag(ep, kFlagIncl));
#pragma unroll
        for (int s = 0; s < 16; ++s) sMu[s][lane] = mu[s];
    }
    __syncthreads();

    float mu[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) mu[s] = fmaf(Qs, sMu[s][lane], Rs[s]);

    // -------------------------------------------------------------- pass G
    float dD_acc = 0.f;
    float dw_acc0 = 0.f, dw_acc1 = 0.f, dw_acc2 = 0.f, dw_acc3 = 0.f;
    float dp1 = 0.f, dp2 = 0.f, dp3 = 0.f;  // dpre at n+1, n+2, n+3
    if (active) {
        for (int k = NSB - 1; k >= 0; --k) {
            const int64_t nb = n0 + k * TB;
            float uw_[TB + 3];  // u at nb-3 .. nb+TB-1 (block)
            if constexpr (BLOCK) {
#pragma unroll
                for (int q = 0; q < TB + 3; ++q) uw_[q] = u_at(nb - 3 + q);
            }
            // recompute the sub-block's states; xs[jj] = state after token jj
            float xs[TB][16];
            float f_[TB], wr_[TB];
            {
                float xc[16];
                if (k == 0) {
#pragma unroll
                    for (int s = 0; s < 16; ++s) xc[s] = valid ? ck[(int64_t)s * Di] : 0.f;
                } else {
#pragma unroll
                    for (int s = 0; s < 16; ++s) xc[s] = sXB[wv][k - 1][s][lane];
                }
#pragma unroll
                for (int jj = 0; jj < TB; ++jj) {
                    const int64_t n = nb + jj;
                    f_[jj] = 1.f;
                    wr_[jj] = 0.f;
                    if (n < L) {
                        if (valid) {
                            const int64_t t = ((int64_t)bi * L + n) * Di + c;
                            float hv;
                            if constexpr (BLOCK) {
                                const float pre = w0 * uw_[jj] + w1 * uw_[jj + 1] +
                                                  w2 * uw_[jj + 2] + w3 * uw_[jj + 3];
                                hv = pre * sigm(pre);
                            } else {
                                hv = to_f(hu[t]);
                            }
                            f_[jj] = sigm(to_f(a[t]));
                            wr_[jj] = sigm(to_f(bg[t])) * hv;
                        }
                        const IO *Bn = Bm + ((int64_t)bi * L + n) * N + sg * 16;
#pragma unroll
                        for (int s = 0; s < 16; ++s)
                            xc[s] = fmaf(f_[jj], xc[s], wr_[jj] * to_f(Bn[s]));
                    }
#pragma unroll
                    for (int s = 0; s < 16; ++s) xs[jj][s] = xc[s];
                }
            }
            // reverse sweep over the sub-block
#pragma unroll
            for (int jj = TB - 1; jj >= 0; --jj) {
                const int64_t n = nb + jj;
                if (n < L) {
                    const int64_t t = ((int64_t)bi * L + n) * Di + c;
                    const IO *Bn = Bm + ((int64_t)bi * L + n) * N + sg * 16;
                    const IO *Cn = Cm + ((int64_t)bi * L + n) * N + sg * 16;
                    // per-token factors, recomputed from the inputs
                    float sa = 0.f, ig = 0.f, sb = 0.f, hv = 0.f, gs = 0.f;
                    float dyv = 0.f, dpre_f = 0.f, dzs = 0.f;
                    if (valid) {
                        float fa, fam, ibm;
                        sigm2(to_f(a[t]), fa, fam);
                        sigm2(to_f(bg[t]), ig, ibm);
                        sa = fa * fam;
                        sb = ig * ibm;
                        gs = to_f(dy[t]);
                        if constexpr (BLOCK) {
                            const float pre = w0 * uw_[jj] + w1 * uw_[jj + 1] +
                                              w2 * uw_[jj + 2] + w3 * uw_[jj + 3];
                            float sp, sm;
                            sigm2(pre, sp, sm);
                            hv = pre * sp;
                            dpre_f = sp * fmaf(pre, sm, 1.f);  // SiLU'(pre)
                            const float zv = to_f(z[t]);
                            float zp, zm;
                            sigm2(zv, zp, zm);
                            dzs = zp * fmaf(zv, zm, 1.f);  // SiLU'(z)
                            dyv = gs;
                            gs *= zv * zp;  // dy SiLU(z)
                        } else {
                            hv = to_f(hu[t]);
                        }
                    }
                    const float gsc = gs * scale;
                    float lam[16], cb[16], cc[16];
                    float df = 0.f, dwv = 0.f, yc = 0.f;
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        const float cv = to_f(Cn[s]);
                        lam[s] = fmaf(gsc, cv, mu[s]);
                        float xp;
                        if (jj > 0)
                            xp = xs[jj > 0 ? jj - 1 : 0][s];
                        else if (k == 0)
                            xp = valid ? ck[(int64_t)s * Di] : 0.f;
                        else
                            xp = sXB[wv][k > 0 ? k - 1 : 0][s][lane];
                        df = fmaf(lam[s], xp, df);
                        dwv = fmaf(lam[s], to_f(Bn[s]), dwv);
                        cb[s] = lam[s] * wr_[jj];
                        cc[s] = gsc * xs[jj][s];
                        if constexpr (BLOCK) yc = fmaf(xs[jj][s], cv, yc);
                    }
                    if constexpr (LPC > 1) {
                        df += __shfl_xor(df, 1);
                        df += __shfl_xor(df, 2);
                        dwv += __shfl_xor(dwv, 1);
                        dwv += __shfl_xor(dwv, 2);
                        if constexpr (BLOCK) {
                            yc += __shfl_xor(yc, 1);
                            yc += __shfl_xor(yc, 2);
                        }
                    }
                    // channel sums of this wave -> per-tile partials
                    const float rb = reduce_scatter16<(LPC == 1)>(cb, lane);
                    const float rc = reduce_scatter16<(LPC == 1)>(cc, lane);
                    const int idx = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 +
                                    ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
                    if (LPC > 1 || (lane & 3) == 0) {
                        float *pp = bc_part + (((int64_t)bi * L + n) * n_tiles + tile) * (2 * N);
                        pp[sg * 16 + idx] = rb;
                        pp[N + sg * 16 + idx] = rc;
                    }
                    const float dav = df * sa;
                    const float dbv = dwv * hv * sb;
                    const float dhv = fmaf(dwv, ig, Dc * gs);
                    dD_acc = fmaf(gs, hv, dD_acc);
                    if (valid && sg == 0) {
                        da[t] = from_f<IO>(dav);
                        db[t] = from_f<IO>(dbv);
                    }
                    if constexpr (BLOCK) {
                        const float dpre = dhv * dpre_f;
                        const float du = w3 * dpre + w2 * dp1 + w1 * dp2 + w0 * dp3;
                        dp3 = dp2;
                        dp2 = dp1;
                        dp1 = dpre;
                        dw_acc0 = fmaf(dpre, uw_[jj], dw_acc0);
                        dw_acc1 = fmaf(dpre, uw_[jj + 1], dw_acc1);
                        dw_acc2 = fmaf(dpre, uw_[jj + 2], dw_acc2);
                        dw_acc3 = fmaf(dpre, uw_[jj + 3], dw_acc3);
                        const int r = k * TB + jj;  // position inside the wave
                        if (valid && sg == 0) {
                            const float ysv = fmaf(scale, yc, Dc * hv);
                            dz[t] = from_f<IO>(dyv * ysv * dzs);
                            float *eg = edge + (((int64_t)bi * n_waves + wrow) * 6) * Di + c;
                            if (r >= T - 3)
                                eg[(3 + (r - (T - 3))) * Di] = du;  // completed by the fix-up
                            else
                                dhu[t] = from_f<IO>(du);
                            if (r < 3) eg[r * Di] = dpre;
                        }
                    } else {
                        if (valid && sg == 0) dhu[t] = from_f<IO>(dhv);
                    }
#pragma unroll
                    for (int s = 0; s < 16; ++s) mu[s] = f_[jj] * lam[s];
                }
            }
        }
        if (valid && sg == 0) {
            dd_part[((int64_t)bi * n_waves + wrow) * Di + c] = dD_acc;
            if constexpr (BLOCK) {
                float *pw = dw_part + (((int64_t)bi * n_waves + wrow) * Di + c) * 4;
                pw[0] = dw_acc0;
                pw[1] = dw_acc1;
                pw[2] = dw_acc2;
                pw[3] = dw_acc3;
                // first-token dpre rows of a wave shorter than 3 tokens
                float *eg = edge + (((int64_t)bi * n_waves + wrow) * 6) * Di + c;
                for (int r = (int)(L - n0); r < 3; ++r) eg[r * Di] = 0.f;
            }
        }
    }

    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t total = per_chunk * (uint32_t)n_chunks;
        const uint32_t old = add_agent(&hdr->done, 1u);
        if (old == total - 1) {
            st_agent(&hdr->ticket, 0u);
            st_agent(&hdr->done, 0u);
            st_agent(&hdr->epoch, ep);
        }
    }
}

// The finish of a backward call: three independent jobs, each too small to
// fill the device alone, run as block ranges of one launch (finish_kernel),
// then the second dD / dconv_w pass.  Every job keeps its fixed summation order.

// dB / dC: sum the per-tile partials in tile order.
template <typename IO>
__device__ __forceinline__ void bc_reduce_block(int blk, const int64_t rows, const int n_tiles,
                                                const int N2, const float *__restrict__ part,
                                                IO *__restrict__ dB, IO *__restrict__ dC)
{
    const int64_t i = (int64_t)blk * 256 + threadIdx.x;  // over rows * N2
    if (i >= rows * N2) return;
    const int64_t row = i / N2;
    const int s = (int)(i % N2);
    const float *p = part + row * (int64_t)n_tiles * N2 + s;
    // eight partials in flight at a time, added in tile order (missing ones add 0)
    float acc = 0.f;
    for (int t0 = 0; t0 < n_tiles; t0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = t0 + k < n_tiles ? p[(int64_t)(t0 + k) * N2] : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += v[k];
    }
    const int N = N2 / 2;
    if (s < N)
        dB[row * N + s] = from_f<IO>(acc);
    else
        dC[row * N + (s - N)] = from_f<IO>(acc);
}

// dD[c] = sum over (batch, wave) rows, dconv_w likewise, in two passes with a
// fixed order (deterministic).  Pass 1: row group g of RG (consecutive rows)
// for 64 channels, its four waves taking every fourth row, summed in wave order.

__device__ __forceinline__ void dd_reduce1_block(int bx, int g, const int64_t rows,
                                                 const int64_t Di, const int RG,
                                                 const float *__restrict__ dd_part,
                                                 const float *__restrict__ dw_part,
                                                 float *__restrict__ part2)
{
    __shared__ float red[4][5][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t c = (int64_t)bx * 64 + lane;
    const int64_t r0 = rows * g / RG, r1 = rows * (g + 1) / RG;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f, s4 = 0.f;
    if (c < Di) {
        for (int64_t r = r0 + wv; r < r1; r += 4) {
            s0 += dd_part[r * Di + c];
            if (dw_part) {
                const float4 q = *(const float4 *)(dw_part + (r * Di + c) * 4);
                s1 += q.x;
                s2 += q.y;
                s3 += q.z;
                s4 += q.w;
            }
        }
    }
    red[wv][0][lane] = s0;
    red[wv][1][lane] = s1;
    red[wv][2][lane] = s2;
    red[wv][3][lane] = s3;
    red[wv][4][lane] = s4;
    __syncthreads();
    if (wv == 0 && c < Di) {
#pragma unroll
        for (int k = 0; k < 5; ++k)
            part2[((int64_t)g * Di + c) * 5 + k] =
                ((red[0][k][lane] + red[1][k][lane]) + red[2][k][lane]) + red[3][k][lane];
    }
}

// Pass 2: the RG row-group partials of each (channel, quantity), in group
// order; one thread per (channel, quantity) -- consecutive in memory -- with
// the group loads issued before the ordered sum.
__global__ __launch_bounds__(256) void dd_reduce2_kernel(const int64_t Di, const int RG,
                                                         const float *__restrict__ part2,
                                                         float *__restrict__ dD,
                                                         float *__restrict__ dconv_w)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // c * 5 + k
    if (i >= Di * 5) return;
    float v[kDdGroups];
#pragma unroll
    for (int g = 0; g < kDdGroups; ++g) v[g] = g < RG ? part2[(int64_t)g * Di * 5 + i] : 0.f;
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < kDdGroups; ++g)
        if (g < RG) t += v[g];
    const int64_t c = i / 5;
    const int k = (int)(i % 5);
    if (k == 0)
        dD[c] = t;
    else if (dconv_w)
        dconv_w[c * 4 + (k - 1)] = t;
}

// Completes du for the last three tokens of every wave with the dpre of the
// next wave's first tokens, and writes dconv_state (inputs before u_0).
//   du_m = sum_k w[k] dpre_{m+3-k}
template <typename IO>
__device__ __forceinline__ void edge_fix_block(int blk, const int64_t Bt, const int64_t L,
                                               const int64_t Di, const int64_t n_waves,
                                               const float *__restrict__ conv_w,
                                               const float *__restrict__ edge, IO *__restrict__ du,
                                               IO *__restrict__ dconv_state)
{
    constexpr int T = kBwdT;
    const int64_t i = (int64_t)blk * 256 + threadIdx.x;  // over Bt*n_waves*Di
    if (i >= Bt * n_waves * Di) return;
    const int64_t c = i % Di;
    const int64_t wrow = (i / Di) % n_waves;
    const int64_t bi = i / (Di * n_waves);
    const float w[4] = {conv_w[c * 4 + 0], conv_w[c * 4 + 1], conv_w[c * 4 + 2],
                        conv_w[c * 4 + 3]};
    const float *eg = edge + ((bi * n_waves + wrow) * 6) * Di + c;
    const int64_t n0 = wrow * T;
    // the next wave's dpre at its first three tokens (rows 0..2 of its record)
    float en[3] = {0.f, 0.f, 0.f};
    if (n0 + T < L) {
        const float *ep = edge + ((bi * n_waves + wrow + 1) * 6) * Di + c;
#pragma unroll
        for (int k = 0; k < 3; ++k) en[k] = n0 + T + k < L ? ep[k * Di] : 0.f;
    }
    // this wave's partial du at its last three tokens (rows 3..5)
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const int64_t m = n0 + T - 3 + q;
        if (m < L) {
            float acc = eg[(3 + q) * Di];
            // du_m gets w[k] dpre_{m+3-k} for m+3-k = n0+T+q-k in the next wave
#pragma unroll
            for (int k = 0; k <= q; ++k) acc += w[k] * en[q - k];
            du[(bi * L + m) * Di + c] = from_f<IO>(acc);
        }
    }
    if (wrow == 0 && dconv_state) {
        // inputs before u_0: dconv_state[q] (token q - 3) gets w[k] dpre_{q-k}
        float e0[3];
#pragma unroll
        for (int n = 0; n < 3; ++n) e0[n] = n < L ? eg[n * Di] : 0.f;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k <= q; ++k) acc += w[k] * e0[q - k];
            dconv_state[(bi * 3 + q) * Di + c] = from_f<IO>(acc);
        }
    }
}

// Blocks [0, nb_bc): dB/dC; then nb_dd blocks of the first dD/dconv_w pass
// (nbx channel blocks per row group); then nb_edge blocks of the edge fix.
template <typename IO>
__global__ __launch_bounds__(256) void finish_kernel(
    const int nb_bc, const int64_t bc_rows, const int n_parts, const int N2,
    const float *__restrict__ bc, IO *__restrict__ dB, IO *__restrict__ dC, const int nb_dd,
    const int nbx, const int64_t dd_rows, const int RG, const float *__restrict__ dd_part,
    const float *__restrict__ dw_part, float *__restrict__ part2, const int64_t Bt,
    const int64_t L, const int64_t Di, const int64_t n_waves, const float *__restrict__ conv_w,
    const float *__restrict__ edge, IO *__restrict__ du, IO *__restrict__ dconv_state)
{
    int b = blockIdx.x;  // block-uniform job selection
    if (b < nb_bc) {
        bc_reduce_block<IO>(b, bc_rows, n_parts, N2, bc, dB, dC);
        return;
    }
    b -= nb_bc;
    if (b < nb_dd) {
        dd_reduce1_block(b % nbx, b / nbx, dd_rows, Di, RG, dd_part, dw_part, part2);
        return;
    }
    b -= nb_dd;
    edge_fix_block<IO>(b, Bt, L, Di, n_waves, conv_w, edge, du, dconv_state);
}

template <typename IO>
static hipError_t launch_bwd_finish(const BwdArgs &g, int n_parts, hipStream_t stream);

template <typename IO, int N, bool BLOCK>
static hipError_t launch_bwd_t(const BwdArgs &g, hipStream_t stream)
{
    const BwdPlan pl = bwd_plan(g.Bt, g.L, g.Di, g.N, g.block);
    char *ws = (char *)g.ws;
    WsHeader *hdr = (WsHeader *)ws;
    uint32_t *flags = (uint32_t *)(ws + pl.off_flags);
    float *agg = (float *)(ws + pl.off_agg);
    float *incl = (float *)(ws + pl.off_incl);
    float *bc = (float *)(ws + pl.off_bc);
    float *dd = (float *)(ws + pl.off_dd);
    float *dw = (float *)(ws + pl.off_dw);
    float *edge = (float *)(ws + pl.off_edge);
    hipLaunchKernelGGL((bwd_kernel<IO, N, BLOCK>), dim3(pl.n_wg), dim3(64 * kBwdW), 0, stream,
                       g.Bt, g.L, g.Di, pl.n_tiles, pl.n_chunks, pl.n_waves, g.scale,
                       (const IO *)g.hu, (const IO *)g.a, (const IO *)g.b, (const IO *)g.B,
                       (const IO *)g.C, g.D, (const IO *)g.z, g.conv_w,
                       (const IO *)g.conv_state, g.ckpt, (const IO *)g.dy, g.dx_final,
                       (IO *)g.dhu, (IO *)g.da, (IO *)g.db, (IO *)g.dz, g.dx0, hdr, flags, agg,
                       incl, bc, dd, dw, edge);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwd_finish<IO>(g, pl.n_tiles, stream);
}

// dB/dC from the n_parts per-token partials, dD/dconv_w from the per-wave
// partials, and the conv transpose at wave edges (all in a fixed order).
template <typename IO>
static hipError_t launch_bwd_finish(const BwdArgs &g, int n_parts, hipStream_t stream)
{
    const int N = g.N;
    const BwdPlan pl = bwd_plan(g.Bt, g.L, g.Di, g.N, g.block);
    char *ws = (char *)g.ws;
    float *bc = (float *)(ws + pl.off_bc);
    float *dd = (float *)(ws + pl.off_dd);
    float *dw = (float *)(ws + pl.off_dw);
    float *edge = (float *)(ws + pl.off_edge);
    hipError_t e;
    const int64_t bc_rows = g.Bt * g.L;
    const int nb_bc = (int)((bc_rows * 2 * N + 255) / 256);
    const int64_t dd_rows = g.Bt * pl.n_waves;
    const int RG = (int)(dd_rows / 8 < 1 ? 1 : dd_rows / 8 > kDdGroups ? kDdGroups : dd_rows / 8);
    const int nbx = (int)((g.Di + 63) / 64);
    const int nb_dd = nbx * RG;
    const int nb_edge = g.block ? (int)((g.Bt * pl.n_waves * g.Di + 255) / 256) : 0;
    float *part2 = (float *)(ws + pl.off_dd2);
    hipLaunchKernelGGL((finish_kernel<IO>), dim3((unsigned)(nb_bc + nb_dd + nb_edge)), dim3(256), 0,
                       stream, nb_bc, bc_rows, n_parts, 2 * N, (const float *)bc, (IO *)g.dB,
                       (IO *)g.dC, nb_dd, nbx, dd_rows, RG, (const float *)dd,
                       g.block ? (const float *)dw : (const float *)nullptr, part2, g.Bt, g.L,
                       g.Di, pl.n_waves, g.conv_w, (const float *)edge, (IO *)g.dhu,
                       (IO *)g.dconv_state);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(dd_reduce2_kernel, dim3((unsigned)((g.Di * 5 + 255) / 256)), dim3(256), 0,
                       stream, g.Di, RG, (const float *)part2, g.dD,
                       g.block ? g.dconv_w : (float *)nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return hipSuccess;
}

// The matrix-core variant serves bf16 activations with d_state 16 when B and C
// allow 16-byte loads; NAJU_BWD_VARIANT=rr forces the register recurrence.
static bool use_bwd_mfma(const BwdArgs &g)
{
    static const bool forced_rr = [] {
        const char *v = getenv("NAJU_BWD_VARIANT");
        return v && v[0] == 'r' && v[1] == 'r';
    }();
    // (the carry pass loads channel pairs as 4-byte words: whole 8-channel groups,
    // as in the forward's matrix-core path)
    if (forced_rr || g.io != 1 || g.N != 16 || g.Di % 8 != 0 || ((uintptr_t)g.B % 16) != 0 ||
        ((uintptr_t)g.C % 16) != 0)
        return false;
    // buffer ranges of 32 token rows and 32-bit fix-list keys
    const MfmaBwdShape m = mfma_bwd_shape(g.Bt, g.L, g.Di);
    return g.Di < ((int64_t)1 << 24) &&
           (double)g.Bt * m.n_super * (double)((g.L + 31) / 32) < 4.0e9;
}

hipError_t launch_bwd(const BwdArgs &g, hipStream_t stream)
{
    if (use_bwd_mfma(g)) {
        hipError_t e = launch_bwd_mfma(g, stream);
        if (e != hipSuccess) return e;
        return launch_bwd_finish<bf16>(g, mfma_bwd_shape(g.Bt, g.L, g.Di).n_super, stream);
    }
    if (g.io == 0) {
        if (g.N == 16) return g.block ? launch_bwd_t<float, 16, true>(g, stream)
                                      : launch_bwd_t<float, 16, false>(g, stream);
        return g.block ? launch_bwd_t<float, 64, true>(g, stream)
                       : launch_bwd_t<float, 64, false>(g, stream);
    }
    if (g.N == 16) return g.block ? launch_bwd_t<bf16, 16, true>(g, stream)
                                  : launch_bwd_t<bf16, 16, false>(g, stream);
    return g.block ? launch_bwd_t<bf16, 64, true>(g, stream)
                   : launch_bwd_t<bf16, 64, false>(g, stream);
}

}  // namespace naju

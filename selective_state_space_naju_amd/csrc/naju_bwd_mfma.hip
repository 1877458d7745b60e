// naju_bwd_mfma.hip -- matrix-core reverse mode of the Naju selective scan for
// bf16 activations and d_state 16 (scan and block).
//
// Differentiates the "Core equations" of the Naju reproduction README (arXiv
// 2607.21000) and its block flowchart.  Inside a wave's 32-token chunk, with
// the chunk-local running product P_n = prod_{j<=n} f_j, the rescaled writes
// W' = w/P, the rescaled readout gradients Gp = g P (g = dLoss/dys), the
// shared token-by-token matrix G[m,k] = C_m.B_k/sqrt(N), the entering state
// x_in (forward checkpoint) and Mu = P_last mu_in (the adjoint flowing in from
// after the chunk, rescaled), every gradient is a product of token x token
// matrices with per-channel columns, or a contraction over channels:
//
//   dw_k  = (1/P_k) [ (G^T_{m>=k} Gp)_k + U_k ],        U_k = B_k . Mu
//   f_n dLoss/df_n = T1_n + T24_n + T3                  (da = sigma(-a) * that)
//     T1_n  = sum_{m>=n} Gp_m V_m,                       V_m = C_m . x_in / sqrt(N)
//     T24_n = sum_{j<n} ( c_j - r_j + W'_j U_j )
//       r_n = Gp_n (G_{k<n} W')_n,   c_n = W'_n (G^T_{m>n} Gp)_n
//     T3    = Mu . x_in
//   dC_m  = ( Gp X_in + tril(H) B )_m / sqrt(N),         H = Gp W'^T (over channels)
//   dB_k  = ( tril(H)^T C )_k / sqrt(N) + (W' Mu)_k
//   mu_out = Gp^T C / sqrt(N) + P_last mu_in             (the reverse carry)
//
// All of these run on v_mfma_f32_32x32x16_bf16 with the same lane/K-slot
// order as the forward (lane l owns column l%32 and the 16 chunk tokens
// {8q + 4h + r}, h = l/32).  Carried quantities (x_in, Mu, the carry's Gp)
// use bf16 hi + lo operand pairs; per-token products use one bf16 operand.
//
// A wave whose chunk has prod(1/f) > 2^64 or a non-finite input cannot use the
// rescaled form.  It still publishes its exact reverse carry (which only needs
// Gp = g P), records itself in a list with its entering adjoint, and a small
// follow-up kernel recomputes its gradients with the plain reverse recurrence.
#include "naju_device.h"
#include "naju_launch.h"

namespace naju {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

__device__ __forceinline__ f32x16 mma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split2(float v, __bf16 &hi, __bf16 &lo)
{
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

__device__ __forceinline__ __bf16 asbf(bf16 v) { return __builtin_bit_cast(__bf16, v); }

// Bit pattern of element s of a bf16x8.  Goes through the whole vector: a
// bit_cast of a single __bf16 vector element to an integer is mis-lowered by
// this compiler (every element reads as element 0).
__device__ __forceinline__ bf16 bits_of(const bf16x8 &v, int s)
{
    const uint4 q = __builtin_bit_cast(uint4, v);
    const uint32_t w = (s >> 1) == 0 ? q.x : (s >> 1) == 1 ? q.y : (s >> 1) == 2 ? q.z : q.w;
    return (bf16)(w >> (16 * (s & 1)));
}

constexpr int kTW = 4;  // token-waves per workgroup (128 tokens)
constexpr int kCG = 2;  // channel groups of 32 per workgroup (64 channels)

}  // namespace

template <bool BLOCK>
__global__ __launch_bounds__(512, 1) void bwd_mfma_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_chunks,
    const int64_t n_waves, const float scale, const bf16 *__restrict__ hu,
    const bf16 *__restrict__ a, const bf16 *__restrict__ bg, const bf16 *__restrict__ Bm,
    const bf16 *__restrict__ Cm, const float *__restrict__ D, const bf16 *__restrict__ z,
    const float *__restrict__ conv_w, const bf16 *__restrict__ conv_state,
    const float *__restrict__ ckpt, const bf16 *__restrict__ dy,
    const float *__restrict__ dx_final, bf16 *__restrict__ dhu, bf16 *__restrict__ da,
    bf16 *__restrict__ db, bf16 *__restrict__ dz, float *__restrict__ dx0, WsHeader *hdr,
    uint32_t *flags, float *agg, float *incl, float *__restrict__ bc_part,
    float *__restrict__ dd_part, float *__restrict__ dw_part, float *__restrict__ edge,
    uint32_t *fix_mask, uint32_t *fix_list, float *fix_mu)
{
    constexpr int N = 16, T = 32;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int tw = wv & (kTW - 1);  // token-wave
    const int grp = wv / kTW;       // channel group
    const int col = lane & 31;
    const int hh = lane >> 5;

    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ float sQ[kTW][64];
    __shared__ float sR[kTW][16][64];
    __shared__ float sMu[16][64];
    __shared__ __attribute__((aligned(16))) bf16 sGpT[8][32][32];  // [wave][token][channel]
    __shared__ __attribute__((aligned(16))) bf16 sWpT[8][32][32];
    __shared__ float sXin[8][32][17];  // [wave][channel][state] (+1 pad)
    __shared__ float sMuw[8][32][17];
    __shared__ float sDiag[kTW][32];
    __shared__ float sDBC[kTW][32][32];  // group-1 partial dB|dC per token

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
    const int64_t n0 = (int64_t)chunk * (kTW * T) + (int64_t)tw * T;
    const int64_t wrow = (int64_t)chunk * kTW + tw;
    const bool active = n0 < L;
    const int64_t c = (int64_t)tile * 64 + grp * 32 + col;
    const bool valid = c < Di;
    const int64_t tokbase = (int64_t)bi * L;
    const float Dc = valid ? D[c] : 0.f;
    auto tok = [&](int i) -> int { return 8 * (i >> 2) + 4 * hh + (i & 3); };
    auto tval = [&](int i) -> bool { return n0 + tok(i) < L; };

    float cw0 = 0.f, cw1 = 0.f, cw2 = 0.f, cw3 = 0.f;
    if (BLOCK && valid) {
        cw0 = conv_w[c * 4 + 0];
        cw1 = conv_w[c * 4 + 1];
        cw2 = conv_w[c * 4 + 2];
        cw3 = conv_w[c * 4 + 3];
    }
    // u at absolute token m (conv_state for m < 0, zero past the end)
    auto u_at = [&](int64_t m) -> float {
        if (!valid || m >= L) return 0.f;
        if (m >= 0) return to_f(hu[(tokbase + m) * Di + c]);
        if (m >= -3 && conv_state) return to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
        return 0.f;
    };

    // ------------------------------------------------ token-shared operands
    bf16x8 Bop, Cop, Csc, Bsv[2], Csv[2];
    {
        const int64_t n = n0 + col;
        if (n < L) {
            Bop = __builtin_bit_cast(bf16x8, *(const uint4 *)(Bm + (tokbase + n) * N + 8 * hh));
            Cop = __builtin_bit_cast(bf16x8, *(const uint4 *)(Cm + (tokbase + n) * N + 8 * hh));
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) Bop[s] = Cop[s] = (__bf16)0.f;
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) Csc[s] = (__bf16)((float)Cop[s] * scale);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            bf16 vb = 0, vc = 0;
            if (col < N && tval(i)) {
                vb = Bm[(tokbase + n0 + tok(i)) * N + col];
                vc = Cm[(tokbase + n0 + tok(i)) * N + col];
            }
            Bsv[i >> 3][i & 7] = asbf(vb);
            Csv[i >> 3][i & 7] = (__bf16)(to_f(vc) * scale);
        }
    }
    // G in A-layout (rows = this lane's column token): g1[i] = B_tok(i).C_col,
    // g2[i] = C_tok(i).B_col
    bf16x8 GA[2], GTA[2];
    {
        f32x16 zero = {};
        const f32x16 g1 = mma(Bop, Cop, zero);
        const f32x16 g2 = mma(Cop, Bop, zero);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            GA[i >> 3][i & 7] = (__bf16)((tok(i) <= col) ? g1[i] * scale : 0.f);
            GTA[i >> 3][i & 7] = (__bf16)((tok(i) >= col) ? g2[i] * scale : 0.f);
            if (grp == 0 && tok(i) == col) sDiag[tw][col] = g1[i] * scale;
        }
    }

    // ------------------------------------------------------------ gates
    float Pv[16];
    bf16x8 WB[2], GpH[2], GpL[2];
    bool ok = true;
    {
        float invf[16], wr[16], gg[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t g0 = n0 + 8 * q + 4 * hh;
            float uw[7];
            if (BLOCK) {
#pragma unroll
                for (int k = 0; k < 7; ++k) uw[k] = u_at(g0 - 3 + k);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * q + r;
                const int64_t n = g0 + r;
                float e = 0.f, ib = 0.f, h = 0.f, gv = 0.f;
                if (valid && n < L) {
                    const int64_t t = (tokbase + n) * Di + c;
                    e = ex2(-to_f(a[t]) * kLog2e);
                    ib = sigm(to_f(bg[t]));
                    gv = to_f(dy[t]);
                    if (BLOCK) {
                        const float pre = cw0 * uw[r] + cw1 * uw[r + 1] + cw2 * uw[r + 2] +
                                          cw3 * uw[r + 3];
                        h = pre * sigm(pre);
                        const float zv = to_f(z[t]);
                        gv *= zv * sigm(zv);
                    } else {
                        h = to_f(hu[t]);
                    }
                }
                invf[i] = 1.f + e;
                wr[i] = ib * h;
                gg[i] = gv;
                ok = ok && (__builtin_fabsf(h) < 1e30f) && (__builtin_fabsf(gv) < 1e30f);
            }
        }
        float tot[4], cum[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float run = 1.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                run *= invf[4 * q + r];
                cum[4 * q + r] = run;
            }
            tot[q] = run;
        }
        float ptot[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) ptot[q] = __shfl_xor(tot[q], 32);
        float E[4], acc = 1.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const bool mine = (g & 1) == hh;
            const float Tg = mine ? tot[g >> 1] : ptot[g >> 1];
            if (mine) E[g >> 1] = acc;
            acc *= Tg;
        }
        ok = ok && (acc <= 18446744073709551616.f);  // 2^64; false for NaN
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float invP = E[i >> 2] * cum[i];
            const float P = rcp(invP);
            Pv[i] = P;
            const float wp = wr[i] * invP;
            ok = ok && (__builtin_fabsf(wp) < 1e30f);
            WB[i >> 3][i & 7] = (__bf16)wp;
            __bf16 hi, lo;
            split2(gg[i] * P, hi, lo);
            GpH[i >> 3][i & 7] = hi;
            GpL[i >> 3][i & 7] = lo;
        }
    }
    const bool wave_ok = __all(ok);

    // ---------------------------- reverse carry pair (Q, R) of this wave -> LDS
    {
        f32x16 r = {};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            r = mma(GpH[kb], Csv[kb], r);
            r = mma(GpL[kb], Csv[kb], r);
        }
        if (col < N) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sR[tw][col][grp * 32 + tok(i)] = r[i];
        }
        if (hh == 1) sQ[tw][grp * 32 + col] = Pv[15];  // P at the chunk's last token
    }
    // staging for the channel contractions and the entering state
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        sGpT[wv][tok(i)][col] = bits_of(GpH[i >> 3], i & 7);
        sWpT[wv][tok(i)][col] = bits_of(WB[i >> 3], i & 7);
    }
    {
        const float *ck = ckpt + ((int64_t)bi * n_waves + wrow) * N * Di + c;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            sXin[wv][col][8 * hh + k] = (active && valid) ? ck[(int64_t)(8 * hh + k) * Di] : 0.f;
    }
    __syncthreads();

    // ----------------------------------- reverse look-back (wave 0, 64 channels)
    if (wv == 0) {
        float Qt = 1.f, Rt[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) Rt[s] = 0.f;
        for (int w = kTW - 1; w >= 0; --w) {
            const float qw = sQ[w][lane];
#pragma unroll
            for (int s = 0; s < 16; ++s) Rt[s] = fmaf(qw, Rt[s], sR[w][s][lane]);
            Qt *= qw;
        }
        const int64_t cl = (int64_t)tile * 64 + lane;
        const bool vl = cl < Di;
        const size_t me = ((size_t)bi * n_tiles + tile) * n_chunks + chunk;
        float mu[16];
        if (chunk == n_chunks - 1) {
#pragma unroll
            for (int s = 0; s < 16; ++s) mu[s] = (dx_final && vl) ? dx_final[(bi * Di + cl) * N + s] : 0.f;
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
                    for (int s = 0; s < 16; ++s) mu[s] = fmaf(accQ, ld_agent(in + s * 64 + lane), accR[s]);
                    break;
                }
                const float *pa = agg + j * (17 * 64);
                const float qj = ld_agent(pa + lane);
#pragma unroll
                for (int s = 0; s < 16; ++s) accR[s] = fmaf(accQ, ld_agent(pa + (1 + s) * 64 + lane), accR[s]);
                accQ *= qj;
                ++j;
            }
        }
        float *ic = incl + me * (16 * 64);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const float mo = fmaf(Qt, mu[s], Rt[s]);
            st_agent(ic + s * 64 + lane, mo);
            if (chunk == 0 && dx0 && vl) dx0[(bi * Di + cl) * N + s] = mo;
        }
        wait_mem();
        if (lane == 0) st_agent(&flags[me], make_flag(ep, kFlagIncl));
#pragma unroll
        for (int s = 0; s < 16; ++s) sMu[s][lane] = mu[s];
    }
    __syncthreads();

    // --------------- this wave's entering adjoint, Mu = P_last mu_in, T3 = Mu.x_in
    float T3;
    {
        const int ch = grp * 32 + col;
        float mu[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) mu[k] = sMu[8 * hh + k][ch];
        for (int w = kTW - 1; w > tw; --w) {  // adjoint passes the later waves first
            const float qw = sQ[w][ch];
#pragma unroll
            for (int k = 0; k < 8; ++k) mu[k] = fmaf(qw, mu[k], sR[w][8 * hh + k][ch]);
        }
        const float pl = sQ[tw][ch];
        float t3 = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float m = pl * mu[k];
            sMuw[wv][col][8 * hh + k] = m;
            t3 = fmaf(m, sXin[wv][col][8 * hh + k], t3);
            if (!wave_ok && active && valid)
                fix_mu[(((int64_t)bi * n_waves + wrow) * N + 8 * hh + k) * Di + c] = mu[k];
        }
        T3 = t3 + __shfl_xor(t3, 32);
    }
    __builtin_amdgcn_wave_barrier();

    f32x16 dBr = {}, dCr = {};
    if (!wave_ok) {
        if (lane == 0 && active) {
            const uint32_t key = (uint32_t)(((int64_t)bi * n_tiles + tile) * n_waves + wrow);
            const uint32_t old = __hip_atomic_fetch_or(&fix_mask[key], 1u << grp, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            if (old == 0) {
                const uint32_t idx = add_agent(&hdr->pad[0], 1u);
                fix_list[idx] = key;
            }
        }
    } else if (active) {
        // operands carrying the entering state / adjoint (hi + lo)
        bf16x8 Xh, Xl, Mh, Ml;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            __bf16 h1, l1, h2, l2;
            split2(sXin[wv][col][8 * hh + k], h1, l1);
            split2(sMuw[wv][col][8 * hh + k], h2, l2);
            Xh[k] = h1;
            Xl[k] = l1;
            Mh[k] = h2;
            Ml[k] = l2;
        }
        f32x16 zero = {};
        f32x16 V = mma(Csc, Xh, zero);
        V = mma(Csc, Xl, V);
        f32x16 U = mma(Bop, Mh, zero);
        U = mma(Bop, Ml, U);
        f32x16 P1 = zero, P2 = zero;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            P1 = mma(GTA[kb], GpH[kb], P1);
            P1 = mma(GTA[kb], GpL[kb], P1);
            P2 = mma(GA[kb], WB[kb], P2);
        }

        // per-token factors, recomputed from the inputs
        bf16x8 GVb[2], X4b[2];
        float dwv[16], dhv[16], dpre[16], dsp[16];
        float dDp = 0.f;
        float dwa0 = 0.f, dwa1 = 0.f, dwa2 = 0.f, dwa3 = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t g0 = n0 + 8 * q + 4 * hh;
            float uw[7];
            if (BLOCK) {
#pragma unroll
                for (int k = 0; k < 7; ++k) uw[k] = u_at(g0 - 3 + k);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * q + r;
                const int64_t n = g0 + r;
                float fa = 1.f, sa = 0.f, ib = 0.f, ibm = 0.f, h = 0.f, gv = 0.f, dyv = 0.f;
                float zs = 0.f, zd = 0.f, pre_d = 0.f, pre = 0.f;
                if (valid && n < L) {
                    const int64_t t = (tokbase + n) * Di + c;
                    sigm2(to_f(a[t]), fa, sa);
                    sigm2(to_f(bg[t]), ib, ibm);
                    gv = to_f(dy[t]);
                    if (BLOCK) {
                        pre = cw0 * uw[r] + cw1 * uw[r + 1] + cw2 * uw[r + 2] + cw3 * uw[r + 3];
                        float sp, sm;
                        sigm2(pre, sp, sm);
                        h = pre * sp;
                        pre_d = sp * fmaf(pre, sm, 1.f);  // SiLU'(pre)
                        const float zv = to_f(z[t]);
                        float zp, zm;
                        sigm2(zv, zp, zm);
                        zs = zv * zp;
                        zd = zp * fmaf(zv, zm, 1.f);  // SiLU'(z)
                        dyv = gv;
                        gv *= zs;
                    } else {
                        h = to_f(hu[t]);
                    }
                }
                const float P = Pv[i];
                const float invP = rcp(P);
                const float wp = ib * h * invP;
                const float gp = gv * P;
                const float dg = sDiag[tw][tok(i)];
                const float dw = invP * (P1[i] + U[i]);
                const float rr = gp * (P2[i] - dg * wp);
                const float cc = wp * (P1[i] - dg * gp);
                X4b[i >> 3][i & 7] = (__bf16)(cc - rr + wp * U[i]);
                GVb[i >> 3][i & 7] = (__bf16)(gp * V[i]);
                dwv[i] = dw;
                dsp[i] = sa;  // sigma(-a) kept for da
                const float dbv = dw * h * ib * ibm;
                const float dh = fmaf(dw, ib, Dc * gv);
                dDp = fmaf(gv, h, dDp);
                if (valid && n < L) {
                    const int64_t t = (tokbase + n) * Di + c;
                    db[t] = from_f<bf16>(dbv);
                    if (BLOCK) {
                        const float ys = fmaf(P, P2[i] + V[i], Dc * h);
                        dz[t] = from_f<bf16>(dyv * ys * zd);
                    } else {
                        dhu[t] = from_f<bf16>(dh);
                    }
                }
                dhv[i] = dh;
                dpre[i] = BLOCK ? dh * pre_d : 0.f;
                if (BLOCK) {
                    dwa0 = fmaf(dpre[i], uw[r], dwa0);
                    dwa1 = fmaf(dpre[i], uw[r + 1], dwa1);
                    dwa2 = fmaf(dpre[i], uw[r + 2], dwa2);
                    dwa3 = fmaf(dpre[i], uw[r + 3], dwa3);
                }
            }
        }
        (void)dwv;
        (void)dhv;
        // da = sigma(-a) (T1 + T24 + T3)
        {
            f32x16 T = zero;
            bf16x8 ONEU[2], ONEL[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                ONEU[i >> 3][i & 7] = (__bf16)(tok(i) >= col ? 1.f : 0.f);
                ONEL[i >> 3][i & 7] = (__bf16)(tok(i) < col ? 1.f : 0.f);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                T = mma(ONEU[kb], GVb[kb], T);
                T = mma(ONEL[kb], X4b[kb], T);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (valid && tval(i)) {
                    const int64_t t = (tokbase + n0 + tok(i)) * Di + c;
                    da[t] = from_f<bf16>(dsp[i] * (T[i] + T3));
                }
            }
        }
        // block: conv transpose du_m = sum_k w_k dpre_{m+3-k} (next group's
        // first three dpre come from the partner half; wave edges via the workspace)
        if (BLOCK) {
            float nx[4][3];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const float mine = dpre[4 * q + k];
                    const float nxt = (q < 3) ? dpre[4 * (q + 1) + k] : 0.f;
                    const float send = hh ? mine : nxt;
                    nx[q][k] = __shfl_xor(send, 32);
                }
            }
            float *eg = edge + (((int64_t)bi * n_waves + wrow) * 6) * Di + c;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float d0 = dpre[4 * q], d1 = dpre[4 * q + 1], d2 = dpre[4 * q + 2],
                            d3 = dpre[4 * q + 3];
                const float e0 = nx[q][0], e1 = nx[q][1], e2 = nx[q][2];
                const bool last = (q == 3 && hh == 1);  // next group is in the next wave
                const float du0 = cw3 * d0 + cw2 * d1 + cw1 * d2 + cw0 * d3;
                const float du1 = cw3 * d1 + cw2 * d2 + cw1 * d3 + (last ? 0.f : cw0 * e0);
                const float du2 = cw3 * d2 + cw2 * d3 + (last ? 0.f : cw1 * e0 + cw0 * e1);
                const float du3 = cw3 * d3 + (last ? 0.f : cw2 * e0 + cw1 * e1 + cw0 * e2);
                const float dus[4] = {du0, du1, du2, du3};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    if (valid && tval(i)) {
                        const int64_t t = (tokbase + n0 + tok(i)) * Di + c;
                        if (last && r >= 1)
                            eg[(3 + (r - 1)) * Di] = dus[r];
                        else
                            dhu[t] = from_f<bf16>(dus[r]);
                    }
                }
            }
            if (hh == 0 && valid) {
#pragma unroll
                for (int k = 0; k < 3; ++k) eg[k * Di] = (n0 + k < L) ? dpre[k] : 0.f;
            }
        }
        // token sums of this wave (dD, dconv_w)
        {
            dDp += __shfl_xor(dDp, 32);
            if (hh == 0 && valid) dd_part[((int64_t)bi * n_waves + wrow) * Di + c] = dDp;
            if (BLOCK) {
                dwa0 += __shfl_xor(dwa0, 32);
                dwa1 += __shfl_xor(dwa1, 32);
                dwa2 += __shfl_xor(dwa2, 32);
                dwa3 += __shfl_xor(dwa3, 32);
                if (hh == 0 && valid) {
                    float *pw = dw_part + (((int64_t)bi * n_waves + wrow) * Di + c) * 4;
                    pw[0] = dwa0;
                    pw[1] = dwa1;
                    pw[2] = dwa2;
                    pw[3] = dwa3;
                }
            }
        }
        // channel contractions: H = Gp W'^T, dC = (Gp X_in + tril(H) B)/sqrt N,
        // dB = tril(H)^T C / sqrt N + W' Mu
        {
            bf16x8 GpT[2], WpT[2], XK[2][2], MK[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                GpT[kb] = __builtin_bit_cast(bf16x8, *(const uint4 *)&sGpT[wv][col][16 * kb + 8 * hh]);
                WpT[kb] = __builtin_bit_cast(bf16x8, *(const uint4 *)&sWpT[wv][col][16 * kb + 8 * hh]);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    __bf16 h1, l1, h2, l2;
                    const int chn = 16 * kb + 8 * hh + k;
                    split2(col < N ? sXin[wv][chn][col] : 0.f, h1, l1);
                    split2(col < N ? sMuw[wv][chn][col] : 0.f, h2, l2);
                    XK[kb][0][k] = h1;
                    XK[kb][1][k] = l1;
                    MK[kb][0][k] = h2;
                    MK[kb][1][k] = l2;
                }
            }
            f32x16 HA = zero, HTA = zero;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                HA = mma(WpT[kb], GpT[kb], HA);   // lane m=col: H[col][tok(i)]
                HTA = mma(GpT[kb], WpT[kb], HTA); // lane k=col: H[tok(i)][col]
            }
            bf16x8 HAb[2], HTAb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                HAb[i >> 3][i & 7] = (__bf16)(tok(i) <= col ? HA[i] : 0.f);
                HTAb[i >> 3][i & 7] = (__bf16)(tok(i) >= col ? HTA[i] : 0.f);
            }
            f32x16 c1 = zero, c2 = zero, b1 = zero, b2 = zero;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                c1 = mma(GpT[kb], XK[kb][0], c1);
                c1 = mma(GpT[kb], XK[kb][1], c1);
                c2 = mma(HAb[kb], Bsv[kb], c2);
                b1 = mma(HTAb[kb], Csv[kb], b1);
                b2 = mma(WpT[kb], MK[kb][0], b2);
                b2 = mma(WpT[kb], MK[kb][1], b2);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                dCr[i] = scale * (c1[i] + c2[i]);
                dBr[i] = b1[i] + b2[i];
            }
        }
    }

    // ---------------- combine the two channel groups, write per-tile partials
    if (grp == 1 && col < N) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sDBC[tw][tok(i)][col] = dBr[i];
            sDBC[tw][tok(i)][16 + col] = dCr[i];
        }
    }
    __syncthreads();
    if (grp == 0 && col < N && active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (tval(i)) {
                float *pp = bc_part + ((tokbase + n0 + tok(i)) * n_tiles + tile) * (2 * N);
                pp[col] = dBr[i] + sDBC[tw][tok(i)][col];
                pp[N + col] = dCr[i] + sDBC[tw][tok(i)][16 + col];
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

// ---------------------------------------------------------------- fix-up
// Recomputes, with the plain reverse recurrence, the gradients of the waves the
// matrix-core kernel listed.  One 64-lane workgroup per list entry (a 32-token
// chunk of one 64-channel tile); lanes are channels, 16 fp32 states each; the
// chunk's states are kept in LDS.  Channel groups that were not listed only
// contribute zeros (their results are already written).
template <bool BLOCK>
__global__ __launch_bounds__(64) void bwd_fix_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles,
    const int64_t n_waves, const float scale, const bf16 *__restrict__ hu,
    const bf16 *__restrict__ a, const bf16 *__restrict__ bg, const bf16 *__restrict__ Bm,
    const bf16 *__restrict__ Cm, const float *__restrict__ D, const bf16 *__restrict__ z,
    const float *__restrict__ conv_w, const bf16 *__restrict__ conv_state,
    const float *__restrict__ ckpt, const bf16 *__restrict__ dy, bf16 *__restrict__ dhu,
    bf16 *__restrict__ da, bf16 *__restrict__ db, bf16 *__restrict__ dz, WsHeader *hdr,
    float *__restrict__ bc_part, float *__restrict__ dd_part, float *__restrict__ dw_part,
    float *__restrict__ edge, uint32_t *fix_mask, const uint32_t *fix_list,
    const float *__restrict__ fix_mu)
{
    constexpr int N = 16, T = 32;
    const int lane = threadIdx.x;
    __shared__ float sx[T][16][64];  // state after each token of the chunk
    const uint32_t cnt = ld_agent(&hdr->pad[0]);
    for (uint32_t e = blockIdx.x; e < cnt; e += gridDim.x) {
        const uint32_t key = fix_list[e];
        const uint32_t gmask = fix_mask[key];
        const int64_t wrow = key % n_waves;
        const int64_t bt = key / n_waves;
        const int tile = (int)(bt % n_tiles);
        const int bi = (int)(bt / n_tiles);
        const int64_t c = (int64_t)tile * 64 + lane;
        const bool mine = ((gmask >> (lane >> 5)) & 1u) != 0;
        const bool valid = c < Di && mine;
        const int64_t n0 = wrow * T;
        const int64_t tokbase = (int64_t)bi * L;
        const float Dc = valid ? D[c] : 0.f;
        float cw0 = 0.f, cw1 = 0.f, cw2 = 0.f, cw3 = 0.f;
        if (BLOCK && valid) {
            cw0 = conv_w[c * 4 + 0];
            cw1 = conv_w[c * 4 + 1];
            cw2 = conv_w[c * 4 + 2];
            cw3 = conv_w[c * 4 + 3];
        }
        auto u_at = [&](int64_t m) -> float {
            if (!valid || m >= L) return 0.f;
            if (m >= 0) return to_f(hu[(tokbase + m) * Di + c]);
            if (m >= -3 && conv_state) return to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
            return 0.f;
        };
        // per-token values (recomputed as needed)
        auto gate = [&](int64_t n, float &f, float &fm, float &ib, float &ibm, float &h,
                        float &gs, float &dyv, float &zd, float &pre_d, float &zs) {
            f = 1.f; fm = 0.f; ib = 0.f; ibm = 0.f; h = 0.f; gs = 0.f; dyv = 0.f; zd = 0.f;
            pre_d = 0.f; zs = 0.f;
            if (!valid || n >= L) return;
            const int64_t t = (tokbase + n) * Di + c;
            sigm2(to_f(a[t]), f, fm);
            sigm2(to_f(bg[t]), ib, ibm);
            gs = to_f(dy[t]);
            if (BLOCK) {
                const float pre = cw0 * u_at(n - 3) + cw1 * u_at(n - 2) + cw2 * u_at(n - 1) +
                                  cw3 * u_at(n);
                float sp, sm;
                sigm2(pre, sp, sm);
                h = pre * sp;
                pre_d = sp * fmaf(pre, sm, 1.f);
                const float zv = to_f(z[t]);
                float zp, zm;
                sigm2(zv, zp, zm);
                zs = zv * zp;
                zd = zp * fmaf(zv, zm, 1.f);
                dyv = gs;
                gs *= zs;
            } else {
                h = to_f(hu[t]);
            }
        };
        float x[16];
        const float *ck = ckpt + ((int64_t)bi * n_waves + wrow) * N * Di + c;
#pragma unroll
        for (int s = 0; s < 16; ++s) x[s] = valid ? ck[(int64_t)s * Di] : 0.f;
        float xin[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) xin[s] = x[s];
        for (int j = 0; j < T; ++j) {
            const int64_t n = n0 + j;
            float f, fm, ib, ibm, h, gs, dyv, zd, pd, zs;
            gate(n, f, fm, ib, ibm, h, gs, dyv, zd, pd, zs);
            if (n < L) {
                const bf16 *Bn = Bm + (tokbase + n) * N;
#pragma unroll
                for (int s = 0; s < 16; ++s) x[s] = fmaf(f, x[s], ib * h * to_f(Bn[s]));
            }
#pragma unroll
            for (int s = 0; s < 16; ++s) sx[j][s][lane] = x[s];
        }
        float mu[16];
#pragma unroll
        for (int s = 0; s < 16; ++s)
            mu[s] = valid ? fix_mu[(((int64_t)bi * n_waves + wrow) * N + s) * Di + c] : 0.f;
        float dDp = 0.f, dwa[4] = {0.f, 0.f, 0.f, 0.f};
        float dp1 = 0.f, dp2 = 0.f, dp3 = 0.f;
        for (int j = T - 1; j >= 0; --j) {
            const int64_t n = n0 + j;
            if (n >= L) continue;
            float f, fm, ib, ibm, h, gs, dyv, zd, pd, zs;
            gate(n, f, fm, ib, ibm, h, gs, dyv, zd, pd, zs);
            const bf16 *Bn = Bm + (tokbase + n) * N;
            const bf16 *Cn = Cm + (tokbase + n) * N;
            const float gsc = gs * scale;
            float lam[16], cb[16], cc[16], df = 0.f, dwv = 0.f, yc = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float cv = to_f(Cn[s]);
                lam[s] = fmaf(gsc, cv, mu[s]);
                const float xp = j > 0 ? sx[j - 1][s][lane] : xin[s];
                const float xn = sx[j][s][lane];
                df = fmaf(lam[s], xp, df);
                dwv = fmaf(lam[s], to_f(Bn[s]), dwv);
                cb[s] = valid ? lam[s] * ib * h : 0.f;
                cc[s] = valid ? gsc * xn : 0.f;
                yc = fmaf(xn, cv, yc);
            }
            // dB, dC contributions of the listed channels, added to the partials
            float vb[16], vc[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                vb[s] = cb[s];
                vc[s] = cc[s];
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    vb[s] += __shfl_xor(vb[s], m);
                    vc[s] += __shfl_xor(vc[s], m);
                }
            }
            if (lane < 16) {
                float *pp = bc_part + ((tokbase + n) * n_tiles + tile) * (2 * N);
                float tb = 0.f, tc = 0.f;
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    tb = (s == lane) ? vb[s] : tb;
                    tc = (s == lane) ? vc[s] : tc;
                }
                pp[lane] += tb;
                pp[N + lane] += tc;
            }
            const float dav = df * f * fm;
            const float dbv = dwv * h * ib * ibm;
            const float dh = fmaf(dwv, ib, Dc * gs);
            dDp = fmaf(gs, h, dDp);
            if (valid) {
                const int64_t t = (tokbase + n) * Di + c;
                da[t] = from_f<bf16>(dav);
                db[t] = from_f<bf16>(dbv);
                if (BLOCK) {
                    const float ys = fmaf(scale, yc, Dc * h);
                    dz[t] = from_f<bf16>(dyv * ys * zd);
                    const float dpre = dh * pd;
                    const float du = cw3 * dpre + cw2 * dp1 + cw1 * dp2 + cw0 * dp3;
                    dp3 = dp2;
                    dp2 = dp1;
                    dp1 = dpre;
                    dwa[0] = fmaf(dpre, u_at(n - 3), dwa[0]);
                    dwa[1] = fmaf(dpre, u_at(n - 2), dwa[1]);
                    dwa[2] = fmaf(dpre, u_at(n - 1), dwa[2]);
                    dwa[3] = fmaf(dpre, u_at(n), dwa[3]);
                    float *eg = edge + (((int64_t)bi * n_waves + wrow) * 6) * Di + c;
                    if (j >= T - 3)
                        eg[(3 + (j - (T - 3))) * Di] = du;
                    else
                        dhu[t] = from_f<bf16>(du);
                    if (j < 3) eg[j * Di] = dpre;
                } else {
                    dhu[t] = from_f<bf16>(dh);
                }
            }
#pragma unroll
            for (int s = 0; s < 16; ++s) mu[s] = f * lam[s];
        }
        if (valid) {
            dd_part[((int64_t)bi * n_waves + wrow) * Di + c] = dDp;
            if (BLOCK) {
                float *pw = dw_part + (((int64_t)bi * n_waves + wrow) * Di + c) * 4;
                pw[0] = dwa[0];
                pw[1] = dwa[1];
                pw[2] = dwa[2];
                pw[3] = dwa[3];
                float *eg = edge + (((int64_t)bi * n_waves + wrow) * 6) * Di + c;
                for (int r = (int)(L - n0); r < 3; ++r) eg[r * Di] = 0.f;
            }
        }
        __syncthreads();
        if (lane == 0) fix_mask[key] = 0u;  // leave the workspace clean
        __syncthreads();
    }
    // the last workgroup to finish clears the list
    if (cnt > 0 && lane == 0) {
        const uint32_t old = add_agent(&hdr->done2, 1u);
        if (old == gridDim.x - 1) {
            st_agent(&hdr->pad[0], 0u);
            st_agent(&hdr->done2, 0u);
        }
    }
}

template <bool BLOCK>
static hipError_t launch_bwd_mfma_t(const BwdArgs &g, hipStream_t stream)
{
    const BwdPlan pl = bwd_plan(g.Bt, g.L, g.Di, g.N, g.block);
    char *ws = (char *)g.ws;
    WsHeader *hdr = (WsHeader *)ws;
    const int n_tiles = (int)((g.Di + 63) / 64);
    const int n_chunks = (int)((g.L + 127) / 128);
    const int64_t n_wg = g.Bt * n_tiles * n_chunks;
    const int64_t n_waves = (g.L + 31) / 32;
    uint32_t *flags = (uint32_t *)(ws + pl.off_flags);
    float *agg = (float *)(ws + pl.off_agg);
    float *incl = (float *)(ws + pl.off_incl);
    float *bc = (float *)(ws + pl.off_bc);
    float *dd = (float *)(ws + pl.off_dd);
    float *dw = (float *)(ws + pl.off_dw);
    float *edge = (float *)(ws + pl.off_edge);
    uint32_t *fmask = (uint32_t *)(ws + pl.off_fixmask);
    uint32_t *flist = (uint32_t *)(ws + pl.off_fixlist);
    float *fmu = (float *)(ws + pl.off_fixmu);
    hipLaunchKernelGGL((bwd_mfma_kernel<BLOCK>), dim3(n_wg), dim3(512), 0, stream, g.Bt, g.L, g.Di,
                       n_tiles, n_chunks, n_waves, g.scale, (const bf16 *)g.hu,
                       (const bf16 *)g.a, (const bf16 *)g.b, (const bf16 *)g.B,
                       (const bf16 *)g.C, g.D, (const bf16 *)g.z, g.conv_w,
                       (const bf16 *)g.conv_state, g.ckpt, (const bf16 *)g.dy, g.dx_final,
                       (bf16 *)g.dhu, (bf16 *)g.da, (bf16 *)g.db, (bf16 *)g.dz, g.dx0, hdr, flags,
                       agg, incl, bc, dd, dw, edge, fmask, flist, fmu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_fix_kernel<BLOCK>), dim3(256), dim3(64), 0, stream, g.Bt, g.L, g.Di,
                       n_tiles, n_waves, g.scale, (const bf16 *)g.hu, (const bf16 *)g.a,
                       (const bf16 *)g.b, (const bf16 *)g.B, (const bf16 *)g.C, g.D,
                       (const bf16 *)g.z, g.conv_w, (const bf16 *)g.conv_state, g.ckpt,
                       (const bf16 *)g.dy, (bf16 *)g.dhu, (bf16 *)g.da, (bf16 *)g.db,
                       (bf16 *)g.dz, hdr, bc, dd, dw, edge, fmask, (const uint32_t *)flist,
                       (const float *)fmu);
    return hipGetLastError();
}

hipError_t launch_bwd_mfma(const BwdArgs &g, hipStream_t stream)
{
    return g.block ? launch_bwd_mfma_t<true>(g, stream) : launch_bwd_mfma_t<false>(g, stream);
}

}  // namespace naju

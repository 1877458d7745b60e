// naju_bwd_mfma.hip -- matrix-core reverse mode of the Naju selective scan for
// bf16 activations and d_state 16 (scan and block).
//
// Differentiates the "Core equations" of the Naju reproduction README (arXiv
// 2607.21000) and its block flowchart.  Inside a wave's 32-token chunk, per
// channel, with the chunk-local running product P_n = prod_{j<=n} f_j, the
// rescaled writes W' = w/P, the readout gradients g = dLoss/dys and Gp = g P,
// the token x token matrix G[m,k] = C_m.B_k/sqrt(N) (shared by all channels),
// the entering state x_in (forward checkpoint), the adjoint mu_in arriving
// after the chunk's last token and Mu = P_last mu_in:
//
//   Z_n    = (G_{k<=n} W')_n + C_n.x_in/sqrt(N)          (ys_n = P_n Z_n + D h_n)
//   dw_k   = (1/P_k) [ (G^T_{m>=k} Gp)_k + B_k.Mu ]      (adjoint of w = sigma(b) h)
//   mu_out = Gp^T C/sqrt(N) + Mu                          (adjoint entering the chunk)
//   dC_m   = ( Gp X_in + tril(H) B )_m / sqrt(N),          H = Gp W'^T over channels
//   dB_k   = ( tril(H)^T C )_k / sqrt(N) + (W' Mu)_k
//
// and the gate gradient follows from Phi_n = f_n dLoss/df_n, which obeys
//   Phi_0 = mu_out . x_in,   Phi_{n+1} = Phi_n - ( g_n (ys_n - D h_n) - w_n dw_n )
// (from lambda_n . x_n = g_n (ys_n - D h_n) + Phi_{n+1} and x_n - f_n x_{n-1} =
// w_n B_n), so da_n = sigma(-a_n) Phi_n is an exclusive prefix sum over the
// chunk.  Every contraction runs on v_mfma_f32_32x32x16_bf16 with the forward's
// lane order (lane l owns column l%32 and the 16 chunk tokens {8q + 4h + r},
// h = l/32), every operand as a bf16 hi + lo pair (three products per pair).
//
// The products take the decay pivoted at the wave's token 16, as the forward
// does: with p = 15 they use W'' = w P_p / P_k, Gp'' = g P_n / P_p,
// X = P_p x_in and Mu'' = (P_last / P_p) mu_in, which give the same Z P, dw,
// H, dB and dC (each P_p cancels per channel) while every scale factor spans
// at most one 16-token half of the wave.  The rescaled form holds while each
// half's product of 1/f stays below 2^96 (forget pre-activations down to about
// -4 on average).
//
// A workgroup owns 128 tokens (four token-waves) of a super-tile of n_sub
// 32-channel tiles, visited in turn; its dB/dC partial over those channels is
// accumulated in the matrix registers and written once.  Activations are read
// and written through buffer resources whose range ends at the last valid
// token, so ragged tails need no branches.  A wave with a half past the bound,
// or a non-finite value, cannot use the rescaled form: it still publishes its
// exact reverse carry (from the plain running product, which underflows
// instead of overflowing), records itself with its entering adjoint, and a
// follow-up kernel recomputes its gradients with the plain reverse recurrence.
#include "naju_device.h"
#include "naju_launch.h"
#include "naju_mfma.h"

namespace naju {

namespace {

constexpr int kTW = 4;  // token-waves per workgroup (128 tokens)

__device__ __forceinline__ f32x16 mma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// bf16 element at byte offset off
__device__ __forceinline__ float ldb(rsrc_t r, uint32_t off)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16);
}
__device__ __forceinline__ void stb(rsrc_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b16(from_f<bf16>(v), r, off, 0, 0);
}

// sigma(-v) in (0, 1) (v = a or b) is parked as fp16 scaled by 2^15: normal (2^-11
// relative) for sigma(-v) >= 2^-29, i.e. v up to about 20; beyond that it underflows
// gradually towards 0 (a gradient factor below 2e-9 there)
constexpr float kSigScale = 32768.f, kSigUnscale = 1.f / 32768.f;

// Workgroups b and b + 8 run on the same XCD (round-robin dispatch) and start
// together; they are paired on the two halves of 128-byte rows (two adjacent
// 32-channel tiles), so each line is fetched once into that XCD's L2 and used
// by both.  Groups of 16 workgroups hold 8 pairs: pair index p, half h.
__device__ __forceinline__ void pair_of(uint32_t b, uint32_t &p, int &h)
{
    p = (b >> 4) * 8 + (b & 7);
    h = (int)((b >> 3) & 1);
}

}  // namespace

template <bool BLOCK>
#ifndef NAJU_BWD_MINB
#define NAJU_BWD_MINB 2
#endif
__global__ __launch_bounds__(64 * kTW, NAJU_BWD_MINB) void bwd_mfma_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_sub,
    const int n_super, const int n_chunks, const int64_t n_waves, const float scale,
    const bf16 *__restrict__ hu, const bf16 *__restrict__ a, const bf16 *__restrict__ bg,
    const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm, const float *__restrict__ D,
    const bf16 *__restrict__ z, const float *__restrict__ conv_w,
    const bf16 *__restrict__ conv_state, const float *__restrict__ ckpt,
    const bf16 *__restrict__ dy, const float *__restrict__ muin, bf16 *__restrict__ dhu,
    bf16 *__restrict__ da, bf16 *__restrict__ db, bf16 *__restrict__ dz, WsHeader *hdr,
    float *__restrict__ bc_part, float *__restrict__ dd_part, float *__restrict__ dw_part,
    float *__restrict__ edge, uint32_t *fix_mask, uint32_t *fix_list, float *fix_mu)
{
    constexpr int N = 16, T = 32;
    const int lane = threadIdx.x & 63;
    // token-wave (wave-uniform; readfirstlane lets the compiler keep everything
    // derived from it -- token ranges, buffer descriptors -- in scalar registers)
    const int tw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;
    const int hh = lane >> 5;
    const bool upper = hh != 0;

    // reverse carries of the four waves
    __shared__ float sQ[kTW][32];
    __shared__ float sR[kTW][16][32];
    // per-token factors consumed once, after the matrix products: sigma(-a),
    // sigma(b), sigma(-b) and dy SiLU'(z)  [wave][slot][lane]
    __shared__ _Float16 sSA[kTW][16][64];  // sigma(-a) * kSigScale
    __shared__ float sEB[kTW][16][64];     // e^{-b}
    __shared__ float sGZ[BLOCK ? kTW : 1][16][64];
    __shared__ bf16 sUw[BLOCK ? kTW : 1][35][32];  // u: three tokens before the wave, then its 32
    __shared__ __attribute__((aligned(16))) bf16 sBr[kTW * 32][16];  // B rows of the 128 tokens
    __shared__ __attribute__((aligned(16))) bf16 sCr[kTW * 32][16];  // C rows / sqrt(N)

    // a pair of workgroups covers 2 n_sub consecutive tiles, half h taking
    // tiles 2 st + h; sup = 2 (pair's tile group) + h indexes the dB/dC partials
    uint32_t pr;
    int hf;
    pair_of(blockIdx.x, pr, hf);
    const uint32_t n_ps = (uint32_t)(n_super / 2);
    if (pr >= (uint32_t)n_chunks * (uint32_t)Bt * n_ps) return;
    const int ps = (int)(pr % n_ps);
    const int bi = (int)((pr / n_ps) % (uint32_t)Bt);
    const int chunk = (int)(pr / n_ps / (uint32_t)Bt);
    const int sup = 2 * ps + hf;
    auto tile_of = [&](int st) -> int { return ps * 2 * n_sub + 2 * st + hf; };
    const int64_t n0 = (int64_t)chunk * (kTW * T) + (int64_t)tw * T;
    const int64_t wrow = (int64_t)chunk * kTW + tw;
    const bool active = n0 < L;
    const int Lw = active ? (int)(L - n0 < T ? L - n0 : T) : 0;  // valid tokens of this wave
    const int64_t tokbase = (int64_t)bi * L;
    auto tok = [&](int i) -> int { return 8 * (i >> 2) + 4 * hh + (i & 3); };
    auto tval = [&](int i) -> bool { return tok(i) < Lw; };

    // ------------------------------------------------ token-shared operands
    // The wave's B and C rows (C pre-scaled: scale = 1/4 is exact in bf16),
    // zero past the last token, staged once in LDS; the token-shared operands
    // are read from there where they are used rather than held in registers.
    {
        const rsrc_t rB = make_rsrc(Bm + (tokbase + (active ? n0 : 0)) * N, (uint32_t)Lw * N * 2);
        const rsrc_t rC = make_rsrc(Cm + (tokbase + (active ? n0 : 0)) * N, (uint32_t)Lw * N * 2);
        const uint32_t ro = (uint32_t)(col * N + 8 * hh) * 2;
        const bf16x8 Bq = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rB, ro, 0, 0));
        const bf16x8 Cq = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rC, ro, 0, 0));
        bf16x8 Cs;
#pragma unroll
        for (int s = 0; s < 8; ++s) Cs[s] = (__bf16)((float)Cq[s] * scale);
        *(uint4 *)&sBr[32 * tw + col][8 * hh] = __builtin_bit_cast(uint4, Bq);
        *(uint4 *)&sCr[32 * tw + col][8 * hh] = __builtin_bit_cast(uint4, Cs);
    }

    f32x16 dBC = {};  // dB (columns 0..15) | dC / scale (columns 16..31) of this wave's tokens
    // The tile's work in two forms (the same barriers in the same order): FULL
    // for a wave of 32 valid tokens, and the ragged form for the last wave of a
    // sequence (see the element access below).
    auto tile_body = [&](const int st, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        // lane-derived values are re-derived every tile: kept out of loop-invariant
        // code motion, which would pin dozens of them (masks, offsets) in registers
        // across the whole loop
        int ln = threadIdx.x & 63;
        asm volatile("" : "+v"(ln));
        const int lane = ln, col = ln & 31, hh = ln >> 5;
        const bool upper = hh != 0;
        auto tok = [&](int i) -> int { return 8 * (i >> 2) + 4 * hh + (i & 3); };
        auto tval = [&](int i) -> bool { return FULL || tok(i) < Lw; };
        // token-shared operands: Bop / Csc are A/B-operand rows (token col, states
        // 8h..8h+7); Bsv / Csv the transposed operands over tokens tok(i), Csv
        // holding state col in columns 0..15 and Bsv state col-16 in columns
        // 16..31, so dB and dC accumulate into the two halves of one matrix
        auto rows = [&](const bf16 (*r)[16]) -> bf16x8 {
            return __builtin_bit_cast(bf16x8, *(const uint4 *)&r[32 * tw + col][8 * hh]);
        };
        auto trans = [&](const bf16 (*r)[16], int kb, bool on) -> bf16x8 {
            bf16x8 v;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bf16 e = r[32 * tw + tok(8 * kb + s)][col & 15];
                v[s] = as_bf(on ? e : (bf16)0);
            }
            return v;
        };
        const int tile = tile_of(st);
        const int64_t c = (int64_t)tile * 32 + col;
        const bool valid = c < Di;
        const int64_t ebase = (tokbase + (active ? n0 : 0)) * Di + (int64_t)tile * 32;
        // Element access of every [Bt][L][Di] tensor: slot i = 4q + r is token
        // 8q + 4h + r, at lane offset vr[r] (row 4h + r) plus group q's row offset.
        // A full wave passes the group offset as the wave-uniform soffset: every
        // row is in range, and the lanes of channels past Di carry kOOB, past the
        // range with or without it.  The ragged wave uses one buffer per tensor
        // and group, starting at the group's first row and ending at the wave's
        // last valid token, so the range check sees the whole offset.
        const uint32_t row2 = (uint32_t)Di * 2;
        uint32_t vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) vr[r] = valid ? (uint32_t)((4 * hh + r) * Di + col) * 2 : kOOB;
        auto trs = [&](const bf16 *t) -> rsrc_t { return make_rsrc(t + ebase, (uint32_t)Lw * row2); };
        auto trq = [&](const bf16 *t, int q) -> rsrc_t {
            const int left = Lw - 8 * q;  // valid rows from the group's first
            return make_rsrc(t + ebase + (int64_t)(8 * q) * Di, left > 0 ? (uint32_t)left * row2 : 0u);
        };
        auto LD16 = [&](const bf16 *t, int i) -> uint16_t {
            if constexpr (FULL)
                return __builtin_amdgcn_raw_buffer_load_b16(trs(t), vr[i & 3],
                                                            (uint32_t)(8 * (i >> 2)) * row2, 0);
            else
                return __builtin_amdgcn_raw_buffer_load_b16(trq(t, i >> 2), vr[i & 3], 0, 0);
        };
        auto LD = [&](const bf16 *t, int i) -> float {
            return __uint_as_float((uint32_t)LD16(t, i) << 16);
        };
        auto ST = [&](bf16 *t, int i, float v) {
            if constexpr (FULL)
                __builtin_amdgcn_raw_buffer_store_b16(from_f<bf16>(v), trs(t), vr[i & 3],
                                                      (uint32_t)(8 * (i >> 2)) * row2, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b16(from_f<bf16>(v), trq(t, i >> 2), vr[i & 3], 0, 0);
        };

        // ------------------------------------------------------- phase A
        // The loads the gates need (a, dy, z, the three rows of u before the wave, D
        // and the conv taps) are issued first, b and h|u once the gates are under way:
        // a wave keeps at most 63 memory operations in flight, so issuing all 86 at
        // once would wait out a round trip before the last of them.
        uint16_t ra[16], rdy[16], rz[BLOCK ? 16 : 1], rb[16], ru[16], rpv[3];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            ra[i] = LD16(a, i);
            rdy[i] = LD16(dy, i);
            if (BLOCK) rz[i] = LD16(z, i);
        }
        if (BLOCK) {
            // u at the three tokens before the wave: the previous rows of u, or the
            // carried conv state before the sequence start
            const bool first = n0 == 0;
            const bf16 *pbase = first ? conv_state : hu;
            const int64_t poff = first ? (int64_t)bi * 3 * Di : (tokbase + n0 - 3) * Di;
            const uint32_t pbytes = ((first && !conv_state) || !active) ? 0u : 3u * (uint32_t)Di * 2;
            const rsrc_t rp = make_rsrc(pbytes ? (const void *)(pbase + poff + tile * 32)
                                               : (const void *)a,
                                        pbytes);
            const uint32_t po = valid ? (uint32_t)col * 2 : kOOB;
#pragma unroll
            for (int k = 0; k < 3; ++k)
                rpv[k] = __builtin_amdgcn_raw_buffer_load_b16(rp, po + (uint32_t)(k * Di) * 2, 0, 0);
        }
        // inputs of w = sigma(b) h
        float cw0 = 0.f, cw1 = 0.f, cw2 = 0.f, cw3 = 0.f, Dc = 0.f;
        if (valid) {
            Dc = D[c];
            if (BLOCK) {
                cw0 = conv_w[c * 4 + 0];
                cw1 = conv_w[c * 4 + 1];
                cw2 = conv_w[c * 4 + 2];
                cw3 = conv_w[c * 4 + 3];
            }
        }
        auto bf = [](uint16_t v) -> float { return __uint_as_float((uint32_t)v << 16); };

        // gates and readout gradients; the wave's reverse carry (P_last, R).  The
        // decay is pivoted at the wave's token 16, as in the forward: invP holds
        // P_p / P_k, Gp = g P_n / P_p, W' = w P_p / P_k, and the products take
        // X = P_p x_in and Mu = (P_last / P_p) mu_in, so that every scale factor spans
        // at most 16 tokens.
        float invP[16], g[16];
        bf16x8 GpH[2], GpL[2];
        bool ok = true;
        float rQ, plp;  // P_p, and P_last / P_p of the lane's channel
        {
            float invf[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float av = bf(ra[i]);
                float dv = bf(rdy[i]);
                const float e = tval(i) ? ex2(-av * kLog2e) : 0.f;
                invf[i] = 1.f + e;
                sSA[tw][i][lane] = (_Float16)(e * rcp(invf[i]) * kSigScale);  // sigma(-a)
                if (BLOCK) {
                    const float zv = bf(rz[i]);
                    const float ez = ex2(-zv * kLog2e);
                    const float sz = rcp(1.f + ez);
                    const float szm = 1.f - sz;  // sigma(-z): only z sigma(-z) is used, absolute error suffices
                    sGZ[tw][i][lane] = dv * sz * fmaf(zv, szm, 1.f);  // dy SiLU'(z)
                    dv *= zv * sz;                                     // dy SiLU(z)
                }
                g[i] = dv;
            }
            // b and h|u, issued once the first loads are in use (a wave keeps at most
            // 63 loads in flight)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                rb[i] = LD16(bg, i);
                ru[i] = LD16(hu, i);
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
            float E[4], acc = 1.f, Q = 1.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q == 2) {  // restart the running product at the pivot
                    Q = acc;
                    acc = 1.f;
                }
                const float pt = xhalf(tot[q], upper);  // partner group (q, 1-h)
                // token order of the groups: (0,0) (0,1) (1,0) (1,1) ...
                E[q] = upper ? acc * pt : acc;
                acc *= tot[q] * pt;
            }
            ok = (Q <= 0x1p96f) && (acc <= 0x1p96f);  // both halves; false for NaN
            rQ = rcp(Q);
            E[0] *= rQ;
            E[1] *= rQ;
            float gp[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                invP[i] = E[i >> 2] * cum[i];
                gp[i] = g[i] * rcp(invP[i]);
                ok = ok && (__builtin_fabsf(gp[i]) < 0x1p110f);
            }
            split16(gp, GpH, GpL);
        }
        // the u window: the wave's 32 tokens and the three before, staged in LDS
        // (row 3 + t is token n0 + t); window u_{n-3..n} of slot 4q+r is rows
        // 8q + 4h + r .. 8q + 4h + r + 3
        auto win = [&](int q, int k) -> float { return to_f(sUw[tw][8 * q + 4 * hh + k][col]); };
        auto fill_window = [&]() {
#pragma unroll
            for (int i = 0; i < 16; ++i) sUw[tw][3 + tok(i)][col] = (bf16)ru[i];
            if (!upper) {
#pragma unroll
                for (int k = 0; k < 3; ++k) sUw[tw][k][col] = (bf16)rpv[k];
            }
        };
        // the seven u values behind group q's windows
        auto window = [&](int q, float (&uw)[7]) {
#pragma unroll
            for (int k = 0; k < 7; ++k) uw[k] = win(q, k);
        };
        // h = SiLU(pre) of the block and its derivative, from the group's u values
        auto silu_at = [&](const float (&uw)[7], int r, float &hd) -> float {
            const float pre = cw0 * uw[r] + cw1 * uw[r + 1] + cw2 * uw[r + 2] + cw3 * uw[r + 3];
            const float sp = rcp(1.f + ex2(-pre * kLog2e));
            hd = sp * fmaf(pre, 1.f - sp, 1.f);  // SiLU'(pre); 1 - sp enters only as pre (1 - sp)
            return pre * sp;
        };
        float h[16], hdk[BLOCK ? 16 : 1];  // h and (block) SiLU'(pre)
        bf16x8 WB[2], WBl[2];     // W' as bf16 hi + lo parts
        {
            float wp[16];
            // sigma(b), and sigma(-b) = e^{-b} sigma(b) (not 1 - sigma(b), which cancels
            // for large b), parked for the epilogue
            float ib[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float eb = ex2(-bf(rb[i]) * kLog2e);
                ib[i] = rcp(1.f + eb);
                sEB[tw][i][lane] = eb;
            }
            if (BLOCK) fill_window();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float uw[7];
                if (BLOCK) window(q, uw);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    float hv;
                    if constexpr (BLOCK)
                        hv = silu_at(uw, r, hdk[i]);
                    else
                        hv = bf(ru[i]);
                    h[i] = hv;
                    wp[i] = ib[i] * hv * invP[i];
                    ok = ok && (__builtin_fabsf(wp[i]) < 0x1p110f);
                }
            }
            split16(wp, WB, WBl);
        }
        const bool wave_ok = __all(ok);
        // x_in (forward checkpoint): states 8h..8h+7 of channel col; and the
        // workgroup's entering adjoint, loaded here so that both round trips
        // overlap the products and the barrier below
        float xin[8], mu0[8];
        const size_t me = ((size_t)bi * n_tiles + tile) * n_chunks + chunk;
        {
            const float *ck = ckpt + (((int64_t)bi * n_waves + wrow) * N + 8 * hh) * Di + c;
#pragma unroll
            for (int k = 0; k < 8; ++k) xin[k] = (active && valid) ? ck[(int64_t)k * Di] : 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) mu0[k] = muin[me * (16 * 32) + (8 * hh + k) * 32 + col];
        }
        if (wave_ok) {
            f32x16 r = {};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 Cv = trans(sCr, kb, col < N);
                r = mma(Cv, GpH[kb], r);  // rows: state, columns: channel
                r = mma(Cv, GpL[kb], r);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) sR[tw][tok(i)][col] = r[i] * rQ;  // R = P_p C^T Gp
            // P_last / P_p from the token-31 lane (the upper half), and the true P_last
            const float pl_own = rcp(invP[15]);
            const float pl_other = xhalf(pl_own, upper);
            plp = upper ? pl_own : pl_other;
            if (upper) sQ[tw][col] = pl_own * rQ;
        } else {
            // A wave outside the rescaled form still owes the earlier waves its exact
            // carry.  The pivoted factors can overflow here (a half-chunk's product of
            // 1/f past the float range, or f = 0), so the carry is formed from the
            // plain running product P_n = prod_{j<=n} f_j, which underflows to 0
            // instead.  a is read again (an L2 hit) rather than kept live.
            float cum[16], tot[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float run = 1.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    run *= tval(i) ? 1.f + ex2(-LD(a, i) * kLog2e) : 1.f;
                    cum[i] = run;
                }
                tot[q] = run;
            }
            float acc = 1.f, gpt[16];
            bf16x8 PH[2], PL[2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float pt = xhalf(tot[q], upper);
                const float Eq = upper ? acc * pt : acc;
                acc *= tot[q] * pt;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    cum[i] *= Eq;  // 1 / P at token tok(i)
                    gpt[i] = g[i] * rcp(cum[i]);
                }
            }
            split16(gpt, PH, PL);
            f32x16 r = {};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 Cv = trans(sCr, kb, col < N);
                r = mma(Cv, PH[kb], r);
                r = mma(Cv, PL[kb], r);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) sR[tw][tok(i)][col] = r[i];
            if (upper) sQ[tw][col] = rcp(cum[15]);
            plp = 0.f;
        }
        __syncthreads();

        // ------------------------------------------------------- phase B
        // this wave's entering adjoint (the later waves pass it first), Mu,
        // x_in and Phi_0 = mu_out . x_in
        // mu_in of this wave: the workgroup's entering adjoint passed through the
        // later waves (states 8h..8h+7 of channel col)
        auto entering = [&](float (&mu)[8]) {
#pragma unroll
            for (int k = 0; k < 8; ++k) mu[k] = mu0[k];
            for (int w = kTW - 1; w > tw; --w) {
                const float qw = sQ[w][col];
#pragma unroll
                for (int k = 0; k < 8; ++k) mu[k] = fmaf(qw, mu[k], sR[w][8 * hh + k][col]);
            }
        };
        float Mu[8];
        float phi0;
        {
            float mu[8];
            entering(mu);
            const float pl = sQ[tw][col];
            float t = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                // Phi_0 = mu_out . x_in with the true Mu = P_last mu_in and R; the
                // products take the pivoted Mu and X
                t = fmaf(fmaf(pl, mu[k], sR[tw][8 * hh + k][col]), xin[k], t);
                Mu[k] = plp * mu[k];
                xin[k] *= rQ;
            }
            phi0 = t + xhalf(t, upper);
        }


        if (!wave_ok) {
            // leave this (wave, tile) to the fix-up kernel: it needs the entering adjoint
            if (active && valid) {
                float mu[8];
                entering(mu);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    fix_mu[(((int64_t)bi * n_waves + wrow) * N + 8 * hh + k) * Di + c] = mu[k];
            }
            if (lane == 0 && active) {
                const uint32_t key = (uint32_t)(((int64_t)bi * n_super + sup) * n_waves + wrow);
                const uint32_t old = __hip_atomic_fetch_or(&fix_mask[key], 1u << st,
                                                           __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                if (old == 0) {
                    const uint32_t idx = add_agent(&hdr->pad[0], 1u);
                    fix_list[idx] = key;
                }
            }
        } else if (active) {
            const f32x16 zero = {};
            bf16x8 XH, XL, MH, ML;  // x_in and Mu (states 8h..8h+7) as A operands
            split8(xin, XH, XL);
            split8(Mu, MH, ML);

            f32x16 Z, PU;  // PU = G^T_{m>=n} Gp + B.Mu, so dw = PU / P
            {
                const bf16x8 Bop = rows(sBr), Csc = rows(sCr);
                // tril(G) and its transpose as A operands (C pre-scaled, so G =
                // Csc.B), each in bf16 hi + lo parts: the gate gradient is a prefix
                // sum of products whose difference it takes, so their rounding must
                // stay near fp32.  One at a time, to keep the registers low.
                {
                    bf16x8 GA[2], GAl[2];
                    const f32x16 g1 = mma(Bop, Csc, zero);  // g1[i] = G[col][tok(i)]
                    float gm[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) gm[i] = (tok(i) <= col) ? g1[i] : 0.f;
                    split16(gm, GA, GAl);
                    Z = mma(Csc, XH, zero);
                    Z = mma(Csc, XL, Z);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        Z = mma(GA[kb], WB[kb], Z);
                        Z = mma(GA[kb], WBl[kb], Z);
                        Z = mma(GAl[kb], WB[kb], Z);
                    }
                }
                {
                    bf16x8 GTA[2], GTAl[2];
                    const f32x16 g2 = mma(Csc, Bop, zero);  // g2[i] = G[tok(i)][col]
                    float gm[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) gm[i] = (tok(i) >= col) ? g2[i] : 0.f;
                    split16(gm, GTA, GTAl);
                    PU = mma(Bop, MH, zero);
                    PU = mma(Bop, ML, PU);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        PU = mma(GTA[kb], GpH[kb], PU);
                        PU = mma(GTA[kb], GpL[kb], PU);
                        PU = mma(GTAl[kb], GpH[kb], PU);
                    }
                }
            }

            // per 4-token group q: outputs, the exclusive prefix for da, the conv
            // transpose (the upper half finishes its previous group once the
            // partner's first three dpre of this group arrive) and dconv_w partials
            float dDp = 0.f, dwa0 = 0.f, dwa1 = 0.f, dwa2 = 0.f, dwa3 = 0.f;
            float base = 0.f;              // prefix of ph over the groups before
            float dprev[4] = {0.f, 0.f, 0.f, 0.f};  // upper half: previous group's dpre
            float *eg = edge + (((int64_t)bi * n_waves + wrow) * 6) * Di + c;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float ph[4], dp[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    const float dw = invP[i] * PU[i];
                    const float ysd = rcp(invP[i]) * Z[i];
                    const float eb = sEB[tw][i][lane];
                    const float ibv = rcp(1.f + eb);
                    const float sbm = eb < __builtin_huge_valf() ? eb * ibv : 1.f;
                    const float hv = h[i];
                    ph[r] = fmaf(g[i], ysd, -ibv * hv * dw);
                    ST(db, i, dw * hv * ibv * sbm);
                    const float dh = fmaf(dw, ibv, Dc * g[i]);
                    dDp = fmaf(g[i], hv, dDp);
                    if (BLOCK) {
                        ST(dz, i, sGZ[tw][i][lane] * fmaf(Dc, hv, ysd));
                        dp[r] = dh * hdk[i];
                    } else {
                        ST(dhu, i, dh);
                    }
                }
                {
                    const float sq = (ph[0] + ph[1]) + (ph[2] + ph[3]);
                    const float ps = xhalf(sq, upper);
                    float run = upper ? base + ps : base;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * q + r;
                        ST(da, i, (float)sSA[tw][i][lane] * kSigUnscale * (phi0 - run));
                        run += ph[r];
                    }
                    base += sq + ps;
                }
                if (BLOCK) {
                    float uw[7];
                    window(q, uw);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        dwa0 = fmaf(dp[r], uw[r], dwa0);
                        dwa1 = fmaf(dp[r], uw[r + 1], dwa1);
                        dwa2 = fmaf(dp[r], uw[r + 2], dwa2);
                        dwa3 = fmaf(dp[r], uw[r + 3], dwa3);
                    }
                    // du_m = sum_k w_k dpre_{m+3-k}.  Lower half: group q followed by the
                    // partner's group q.  Upper half: group q-1 followed by the partner's
                    // group q (its first three dpre are what arrives here).
                    float e[3];
#pragma unroll
                    for (int k = 0; k < 3; ++k) e[k] = xhalf(dp[k], upper);
                    const float *d = upper ? dprev : dp;
                    const float du[4] = {cw3 * d[0] + cw2 * d[1] + cw1 * d[2] + cw0 * d[3],
                                         cw3 * d[1] + cw2 * d[2] + cw1 * d[3] + cw0 * e[0],
                                         cw3 * d[2] + cw2 * d[3] + cw1 * e[0] + cw0 * e[1],
                                         cw3 * d[3] + cw2 * e[0] + cw1 * e[1] + cw0 * e[2]};
                    const int qo = upper ? q - 1 : q;  // the group finished here
                    if (qo >= 0) {
                        // qo differs between the halves, so its row offset joins the lane
                        // offset: as a scalar offset or a per-group buffer it would be
                        // lane-dependent, and each store a loop over its distinct values
                        const rsrc_t rdu = trs(dhu);
                        const uint32_t go = (uint32_t)(8 * qo) * row2;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            __builtin_amdgcn_raw_buffer_store_b16(from_f<bf16>(du[r]), rdu,
                                                                  vr[r] + go, 0, 0);
                    }
                    if (q == 0 && !upper && valid) {
                        // the wave's first three dpre, for the previous wave's last tokens
#pragma unroll
                        for (int k = 0; k < 3; ++k) eg[k * Di] = (k < Lw) ? dp[k] : 0.f;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) dprev[r] = dp[r];
                }
            }
            if (BLOCK && upper) {
                // the upper half's last group: token 28 is complete, tokens 29..31 wait
                // for the next wave's first dpre (finished from the workspace)
                const float *d = dprev;
                const float du[4] = {cw3 * d[0] + cw2 * d[1] + cw1 * d[2] + cw0 * d[3],
                                     cw3 * d[1] + cw2 * d[2] + cw1 * d[3],
                                     cw3 * d[2] + cw2 * d[3],
                                     cw3 * d[3]};
                ST(dhu, 12, du[0]);
                if (valid) {
#pragma unroll
                    for (int r = 1; r < 4; ++r)
                        if (tval(12 + r)) eg[(3 + (r - 1)) * Di] = du[r];
                }
            }
            // token sums of this wave (dD, dconv_w)
            dDp += xhalf(dDp, upper);
            if (BLOCK) {
                dwa0 += xhalf(dwa0, upper);
                dwa1 += xhalf(dwa1, upper);
                dwa2 += xhalf(dwa2, upper);
                dwa3 += xhalf(dwa3, upper);
            }
            if (!upper && valid) {
                dd_part[((int64_t)bi * n_waves + wrow) * Di + c] = dDp;
                if (BLOCK)
                    *(float4 *)(dw_part + (((int64_t)bi * n_waves + wrow) * Di + c) * 4) =
                        make_float4(dwa0, dwa1, dwa2, dwa3);
            }
            // Channel contractions: H = Gp W'^T; columns 0..15 of dBC gather
            // tril(H)^T C + W' Mu (C pre-scaled), columns 16..31 Gp X_in + tril(H) B.
            // Every operand and H itself enter as bf16 hi + lo parts: H sums products
            // over the channels of values whose rounding does not cancel, so a single
            // bf16 part would leave dB and dC about 1% of their own scale off.
            // The channel-major operands come from the register layout through a
            // product with a 0/1 selection matrix on the matrix cores (each output is
            // one input times 1, so exact): afterwards lane (col, h) holds, for token
            // (or state) col, the channels tok(i) of the tile in K order.  Gp, W', x_in
            // and Mu all come out in that one channel order, which is all that a
            // contraction over channels needs.
            {
                // selection over tokens: element s of block kb in lane (col, h) stands
                // for token 16 kb + 8 (s >> 2) + 4 h + (s & 3), i.e. tok(8 kb + s)
                // a 0/1 operand with a single 1 (bf16 0x3f80) at element s, if on
                auto one_hot = [](bool on, int s) -> bf16x8 {
                    const uint32_t v = on ? (0x3f80u << (16 * (s & 1))) : 0u;
                    const int d = s >> 1;
                    const uint4 q = {d == 0 ? v : 0u, d == 1 ? v : 0u, d == 2 ? v : 0u,
                                     d == 3 ? v : 0u};
                    return __builtin_bit_cast(bf16x8, q);
                };
                // tok(8 kb + s) == col  <=>  kb = col / 16, h = (col / 4) % 2 and
                // s = 4 ((col / 8) % 2) + col % 4
                auto sel_tok = [&](int kb) -> bf16x8 {
                    return one_hot((col >> 4) == kb && ((col >> 2) & 1) == hh,
                                   4 * ((col >> 3) & 1) + (col & 3));
                };
                const bf16x8 S0 = sel_tok(0), S1 = sel_tok(1);
                // transpose of a 32 x 32 operand pair held with rows by lane and
                // columns by slot: afterwards rows by slot, columns by lane (exact)
                auto chan_major = [&](const bf16x8 (&v)[2], bf16x8 (&out)[2]) {
                    f32x16 t = mma(v[0], S0, zero);
                    t = mma(v[1], S1, t);
#pragma unroll
                    for (int i = 0; i < 16; ++i) out[i >> 3][i & 7] = (__bf16)t[i];
                };
                bf16x8 GTh[2], GTl[2], WTh[2], WTl[2];
                chan_major(GpH, GTh);
                chan_major(GpL, GTl);
                chan_major(WB, WTh);
                chan_major(WBl, WTl);
                // Mu (state col, columns 0..15) and x_in (state col - 16, columns
                // 16..31) over the same channels: states 8h + s select column 8h + s
                // of the first half or of the second
                bf16x8 XMh[2], XMl[2];
                {
                    // 8 h + s == col (columns 0..15), 8 h + s + 16 == col (16..31)
                    const bf16x8 sm = one_hot(col < 16 && ((col >> 3) & 1) == hh, col & 7);
                    const bf16x8 sx = one_hot(col >= 16 && ((col >> 3) & 1) == hh, col & 7);
                    f32x16 t = mma(MH, sm, zero);
                    t = mma(ML, sm, t);
                    t = mma(XH, sx, t);
                    t = mma(XL, sx, t);
                    float tv[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) tv[i] = t[i];
                    split16(tv, XMh, XMl);
                }
                // the A operand of the Mu / x_in term: W' for dB, Gp for dC -- one
                // product per column half, the other half of XM zeroed
                const uint4 z4 = {0u, 0u, 0u, 0u};
                const bf16x8 zb = __builtin_bit_cast(bf16x8, z4);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 bh = col < N ? XMh[kb] : zb, bl = col < N ? XMl[kb] : zb;
                    const bf16x8 ch = col < N ? zb : XMh[kb], cl = col < N ? zb : XMl[kb];
                    dBC = mma(WTh[kb], bh, dBC);  // columns 0..15
                    dBC = mma(WTh[kb], bl, dBC);
                    dBC = mma(WTl[kb], bh, dBC);
                    dBC = mma(GTh[kb], ch, dBC);  // columns 16..31
                    dBC = mma(GTh[kb], cl, dBC);
                    dBC = mma(GTl[kb], ch, dBC);
                }
                // tril(H) (token m >= k), hi + lo: rows k by lane for tril(H)^T C, then
                // its transpose (rows m by lane) for tril(H) B
                {
                    f32x16 HT = zero;  // HT[i] = H[tok(i)][col]
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        HT = mma(GTh[kb], WTh[kb], HT);
                        HT = mma(GTh[kb], WTl[kb], HT);
                        HT = mma(GTl[kb], WTh[kb], HT);
                    }
                    bf16x8 Hh[2], Hl[2];
                    float hm[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) hm[i] = tok(i) >= col ? HT[i] : 0.f;
                    split16(hm, Hh, Hl);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const bf16x8 Ct = trans(sCr, kb, col < N);
                        dBC = mma(Hh[kb], Ct, dBC);  // columns 0..15
                        dBC = mma(Hl[kb], Ct, dBC);
                    }
                    bf16x8 Th[2], Tl[2];
                    chan_major(Hh, Th);
                    chan_major(Hl, Tl);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const bf16x8 Bt = trans(sBr, kb, col >= N);
                        dBC = mma(Th[kb], Bt, dBC);  // columns 16..31
                        dBC = mma(Tl[kb], Bt, dBC);
                    }
                }
            }

        }
        __syncthreads();  // sQ and sR are rewritten by the next tile
    };
    for (int st = 0; st < n_sub && tile_of(st) < n_tiles; ++st) {
        if (Lw == T)
            tile_body(st, std::true_type{});
        else
            tile_body(st, std::false_type{});
    }

    // ------------------------- dB/dC partial of this super-tile, per token
    if (active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (tval(i)) {
                float *pp = bc_part + ((tokbase + n0 + tok(i)) * n_super + sup) * (2 * N);
                pp[col] = col < N ? dBC[i] : dBC[i] * scale;
            }
        }
    }

}

// ----------------------------------------------------- reverse carry pass
// The adjoint crossing a chunk boundary only needs, per 128-token chunk of a
// 32-channel tile, the chunk's reverse carry  mu_out = Q mu_in + R  with
// Q = P_last (per channel) and R = Gp^T C / sqrt(N) (per channel and state).
// A workgroup takes 64 channels (two tiles, whole 128-byte rows) of one chunk;
// its four waves compute their 32-token carries with the same products as the
// gradient kernel and compose them (the adjoint passes the later waves first).
// Lane (col, h) holds the channel pair 64p + 2 col, 64p + 2 col + 1 (one 4-byte
// load per token and tensor); MFMA column tile j takes the channels 64p + 2 col + j.
template <bool BLOCK>
__global__ __launch_bounds__(64 * kTW) void bwd_carry_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_chunks,
    const float scale, const bf16 *__restrict__ a, const bf16 *__restrict__ Cm,
    const bf16 *__restrict__ z, const bf16 *__restrict__ dy, float *__restrict__ agg)
{
    constexpr int N = 16, T = 32;
    const int lane = threadIdx.x & 63;
    const int tw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;
    const int hh = lane >> 5;
    const bool upper = hh != 0;
    __shared__ float sQ[kTW][2][32];
    __shared__ float sR[kTW][2][16][32];

    const int n_pairs = (n_tiles + 1) / 2;  // 64-channel groups
    const int pr = (int)(blockIdx.x % (uint32_t)n_pairs);
    const int chunk = (int)((blockIdx.x / (uint32_t)n_pairs) % (uint32_t)n_chunks);
    const int bi = (int)(blockIdx.x / (uint32_t)n_pairs / (uint32_t)n_chunks);
    const int64_t n0 = (int64_t)chunk * (kTW * T) + (int64_t)tw * T;
    const bool active = n0 < L;
    const int Lw = active ? (int)(L - n0 < T ? L - n0 : T) : 0;
    const int64_t tokbase = (int64_t)bi * L;
    const int64_t c0 = (int64_t)pr * 64 + 2 * col;  // channel of column tile j: c0 + j
    const bool valid = c0 < Di;                      // Di is even: both or neither
    auto tok = [&](int i) -> int { return 8 * (i >> 2) + 4 * hh + (i & 3); };

    // the loads go out first among the CU's workgroups (wave priority 2 until the
    // last is issued): a carry is one round trip and then arithmetic
    __builtin_amdgcn_s_setprio(2);
    bf16x8 Csv[2];
    {
        const rsrc_t rC = make_rsrc(Cm + (tokbase + (active ? n0 : 0)) * N, (uint32_t)Lw * N * 2);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t o = col < N ? (uint32_t)(tok(i) * N + col) * 2 : kOOB;
            Csv[i >> 3][i & 7] = (__bf16)(ldb(rC, o) * scale);
        }
    }
    const int64_t ebase = (tokbase + (active ? n0 : 0)) * Di + (int64_t)pr * 64;
    const uint32_t row2 = (uint32_t)Di * 2;
    uint32_t vr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vr[r] = valid ? (uint32_t)((4 * hh + r) * Di + 2 * col) * 2 : kOOB;
    // the two channels of slot i as one 4-byte load
    auto LD2 = [&](const bf16 *t, int i) -> uint32_t {
        return __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(t + ebase, (uint32_t)Lw * row2),
                                                    vr[i & 3] + (uint32_t)(8 * (i >> 2)) * row2,
                                                    0, 0);
    };
    float invf[2][16], g[2][16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t av = LD2(a, i), dv = LD2(dy, i);
        uint32_t zv = 0;
        if (BLOCK) zv = LD2(z, i);
        const bool tv = tok(i) < Lw;  // tokens past the end keep the state (f = 1)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float aj = __uint_as_float(j ? (av & 0xffff0000u) : (av << 16));
            float dj = __uint_as_float(j ? (dv & 0xffff0000u) : (dv << 16));
            invf[j][i] = 1.f + (tv ? ex2(-aj * kLog2e) : 0.f);
            if (BLOCK) {
                const float zj = __uint_as_float(j ? (zv & 0xffff0000u) : (zv << 16));
                dj *= zj * rcp(1.f + ex2(-zj * kLog2e));  // dy SiLU(z)
            }
            g[j][i] = dj;
        }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float tot[4], cum[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float run = 1.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                run *= invf[j][4 * q + r];
                cum[4 * q + r] = run;
            }
            tot[q] = run;
        }
        float E[4], acc = 1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float pt = xhalf(tot[q], upper);
            E[q] = upper ? acc * pt : acc;
            acc *= tot[q] * pt;
        }
        bf16x8 GpH[2], GpL[2];
        float gp[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) gp[i] = g[j][i] * rcp(E[i >> 2] * cum[i]);
        split16(gp, GpH, GpL);
        f32x16 r = {};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            r = mma(Csv[kb], GpH[kb], r);  // rows: state, columns: channel
            r = mma(Csv[kb], GpL[kb], r);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sR[tw][j][tok(i)][col] = r[i];
        if (upper) sQ[tw][j][col] = rcp(E[3] * cum[15]);
    }
    __syncthreads();
    if (tw == 0 && valid) {
        // lane (col, h) composes states 8h..8h+7 of its two channels
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float Qt = 1.f, Rt[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) Rt[k] = 0.f;
            for (int w = kTW - 1; w >= 0; --w) {
                const float qw = sQ[w][j][col];
#pragma unroll
                for (int k = 0; k < 8; ++k) Rt[k] = fmaf(qw, Rt[k], sR[w][j][8 * hh + k][col]);
                Qt *= qw;
            }
            const int64_t ch = c0 + j;  // its 32-channel tile and column there
            const int tile = (int)(ch >> 5), cc = (int)(ch & 31);
            float *ag = agg + (((size_t)bi * n_tiles + tile) * n_chunks + chunk) * (17 * 32);
            if (!upper) ag[cc] = Qt;
#pragma unroll
            for (int k = 0; k < 8; ++k) ag[(1 + 8 * hh + k) * 32 + cc] = Rt[k];
        }
    }
}

// Reverse scan of the chunk carries: the adjoint arriving after each chunk's
// last token (dx_final after the sequence), and dx0 before the first token.
// One thread per (channel, state); a workgroup per (batch row, tile).
__global__ __launch_bounds__(512) void bwd_carry_scan_kernel(
    const int64_t Di, const int n_tiles, const int n_chunks, const float *__restrict__ agg,
    const float *__restrict__ dx_final, float *__restrict__ muin, float *__restrict__ dx0)
{
    constexpr int N = 16;
    const int s = threadIdx.x >> 5, col = threadIdx.x & 31;
    const int tile = (int)(blockIdx.x % (uint32_t)n_tiles);
    const int64_t bi = blockIdx.x / (uint32_t)n_tiles;
    const int64_t c = (int64_t)tile * 32 + col;
    const bool valid = c < Di;
    float mu = (dx_final && valid) ? dx_final[(bi * Di + c) * N + s] : 0.f;
    const size_t e0 = (size_t)blockIdx.x * n_chunks;
#pragma unroll 4
    for (int ch = n_chunks - 1; ch >= 0; --ch) {
        muin[(e0 + ch) * (16 * 32) + s * 32 + col] = mu;
        const float *ag = agg + (e0 + ch) * (17 * 32);
        mu = fmaf(ag[col], mu, ag[(1 + s) * 32 + col]);
    }
    if (dx0 && valid) dx0[(bi * Di + c) * N + s] = mu;
}

// ---------------------------------------------------------------- fix-up
// Recomputes, with the plain reverse recurrence, the gradients of the waves the
// matrix-core kernel listed.  A list entry is one 32-token chunk of one
// super-tile; a 64-lane workgroup walks its listed 32-channel tiles two at a
// time (lane = channel, 16 fp32 states each, the chunk's states kept in LDS).
// Tiles that were not listed only contribute zeros (their results are already
// written).
template <bool BLOCK>
__global__ __launch_bounds__(64) void bwd_fix_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_sub,
    const int n_super, const int64_t n_waves, const float scale, const bf16 *__restrict__ hu,
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
        const uint32_t tmask = fix_mask[key];
        const int64_t wrow = key % n_waves;
        const int64_t bs = key / n_waves;
        const int sup = (int)(bs % n_super);
        const int bi = (int)(bs / n_super);
        const int64_t n0 = wrow * T;
        const int64_t tokbase = (int64_t)bi * L;
        for (int pr = 0; 2 * pr < n_sub; ++pr) {
            const int st = 2 * pr + (lane >> 5);
            const int tile = (sup >> 1) * 2 * n_sub + 2 * st + (sup & 1);
            const int64_t c = (int64_t)tile * 32 + (lane & 31);
            const bool mine = st < n_sub && tile < n_tiles && ((tmask >> st) & 1u) != 0;
            const bool valid = c < Di && mine;
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
                if (m >= -3 && conv_state)
                    return to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
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
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        cb[s] += __shfl_xor(cb[s], m);
                        cc[s] += __shfl_xor(cc[s], m);
                    }
                }
                if (lane < 16) {
                    float *pp = bc_part + ((tokbase + n) * n_super + sup) * (2 * N);
                    float tb = 0.f, tc = 0.f;
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        tb = (s == lane) ? cb[s] : tb;
                        tc = (s == lane) ? cc[s] : tc;
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
            __syncthreads();  // sx is rewritten by the next tile pair
        }
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
    const MfmaBwdShape m = mfma_bwd_shape(g.Bt, g.L, g.Di);
    char *ws = (char *)g.ws;
    WsHeader *hdr = (WsHeader *)ws;
    const int64_t n_waves = (g.L + 31) / 32;
    float *agg = (float *)(ws + pl.off_magg);
    float *muin = (float *)(ws + pl.off_mincl);
    float *bc = (float *)(ws + pl.off_bc);
    float *dd = (float *)(ws + pl.off_dd);
    float *dw = (float *)(ws + pl.off_dw);
    float *edge = (float *)(ws + pl.off_edge);
    uint32_t *fmask = (uint32_t *)(ws + pl.off_fixmask);
    uint32_t *flist = (uint32_t *)(ws + pl.off_fixlist);
    float *fmu = (float *)(ws + pl.off_fixmu);
    hipError_t e;
    const int64_t k1_wgs = g.Bt * m.n_chunks * ((m.n_tiles + 1) / 2);
    hipLaunchKernelGGL((bwd_carry_kernel<BLOCK>), dim3((unsigned)k1_wgs),
                       dim3(64 * kTW), 0, stream, g.Bt, g.L, g.Di, m.n_tiles, m.n_chunks, g.scale,
                       (const bf16 *)g.a, (const bf16 *)g.C, (const bf16 *)g.z, (const bf16 *)g.dy,
                       agg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_carry_scan_kernel, dim3((unsigned)(g.Bt * m.n_tiles)), dim3(512), 0,
                       stream, g.Di, m.n_tiles, m.n_chunks, (const float *)agg, g.dx_final, muin,
                       g.dx0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t k3_pairs = m.n_wg / 2;
    hipLaunchKernelGGL((bwd_mfma_kernel<BLOCK>), dim3((unsigned)(16 * ((k3_pairs + 7) / 8))), dim3(64 * kTW), 0, stream,
                       g.Bt, g.L, g.Di, m.n_tiles, m.n_sub, m.n_super, m.n_chunks, n_waves,
                       g.scale, (const bf16 *)g.hu, (const bf16 *)g.a, (const bf16 *)g.b,
                       (const bf16 *)g.B, (const bf16 *)g.C, g.D, (const bf16 *)g.z, g.conv_w,
                       (const bf16 *)g.conv_state, g.ckpt, (const bf16 *)g.dy, (const float *)muin,
                       (bf16 *)g.dhu, (bf16 *)g.da, (bf16 *)g.db, (bf16 *)g.dz, hdr, bc, dd, dw,
                       edge, fmask, flist, fmu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_fix_kernel<BLOCK>), dim3(256), dim3(64), 0, stream, g.Bt, g.L, g.Di,
                       m.n_tiles, m.n_sub, m.n_super, n_waves, g.scale, (const bf16 *)g.hu,
                       (const bf16 *)g.a, (const bf16 *)g.b, (const bf16 *)g.B, (const bf16 *)g.C,
                       g.D, (const bf16 *)g.z, g.conv_w, (const bf16 *)g.conv_state, g.ckpt,
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

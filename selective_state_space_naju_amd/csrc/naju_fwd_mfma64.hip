// naju_fwd_mfma64.hip -- matrix-core forward of the Naju selective scan for
// bf16 activations and d_state 64 (scan and block).
//
// Recurrence and readout: "Core equations" of the Naju reproduction README
// (arXiv 2607.21000); block front end and output modulation: that page's block
// flowchart.  Inside a wave's 32 tokens the chunk algebra is that of the
// d_state-16 matrix-core forward: with P_n = prod_{j<=n} f_j (per channel) and
// W'_k = w_k / P_k,
//     y_n = P_n ( sum_{k<=n} G[n,k] W'_k + C_n x_in / sqrt(N) ) + D h_n,
//     G   = tril(C B^T) / sqrt(N),      x_out = P_T (x_in + W'^T B),
// where G now contracts over 64 states (four MFMA K-blocks) and a wave's
// state (32 channels) is 64 x 32.
//
// Decomposition.  A workgroup of eight waves owns one row (batch row,
// 64-channel tile) at a time and walks its 128-token chunks in order, so the
// state entering a chunk is the one its own previous chunk left: no
// cross-workgroup look-back and no workspace.  Wave (t, c) takes token block t
// (32 tokens) of channel half c (32 channels); the four waves of a channel half
// carry its state in registers (token block t: states 16 t .. 16 t + 15) and
// compose it with their chunk aggregates through LDS.  A 64-channel row is a
// whole 128-byte line, so the tile copies fetch no half lines; one workgroup
// fills a CU (136 KB of LDS).
//
// The decay is pivoted at the wave's token 16: with P_p = prod_{j<=15} f_j the
// products take W'' = w P_p / P_k, the outputs P_n / P_p, the entering state
// P_p x_in and the aggregate the factor P_T / P_p, so every scale factor spans at
// most one 16-token half.  A wave with a half whose product of 1/f passes 2^96,
// or a non-finite gate or h, runs the plain register recurrence for its chunk
// instead.  The host uses this kernel when the rows alone keep a good part of
// the device busy (Bt * d_inner / 64 >= 32).
#include <type_traits>

#include "naju_device.h"
#include "naju_launch.h"
#include "naju_mfma.h"

namespace naju {

namespace {
constexpr int kN = 64;          // d_state
constexpr int kCT = 64;         // channels per tile
constexpr int kCW = 32;         // channels per wave
constexpr int kTk = 32;         // tokens per wave
constexpr int kWv = 8;          // waves per workgroup: 4 token blocks x 2 channel halves
constexpr int kRw = kTk * 4;    // tokens per chunk
constexpr int kHl = 16;         // rows of u kept before the chunk (block)
constexpr int kSP = kN + 4;     // padded per-channel state row of the LDS aggregates
}  // namespace

// ------------------------------------------------------------------ fallback
// Register recurrence of one wave's 32 tokens for lane (channel c, state half
// sh), states 32 sh .. 32 sh + 31.  Conv window of the block from memory.
template <bool BLOCK>
__device__ __forceinline__ void rr64_window(int64_t L, int64_t Di, int bi, int64_t c, bool valid,
                                            int64_t n0, const bf16 *hu, const float *conv_w,
                                            const bf16 *conv_state, float (&cw)[4], float (&um)[3])
{
    cw[0] = cw[1] = cw[2] = cw[3] = 0.f;
    um[0] = um[1] = um[2] = 0.f;
    if (!BLOCK || !valid) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) cw[k] = conv_w[c * 4 + k];
    for (int k = 1; k <= 3; ++k) {  // um[k-1] = u_{n0-k}
        const int64_t m = n0 - k;
        float v = 0.f;
        if (m >= 0 && m < L)
            v = to_f(hu[((int64_t)bi * L + m) * Di + c]);
        else if (m < 0 && conv_state)
            v = to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
        um[k - 1] = v;
    }
}

// h, f and the write gate of token t for the fallback (block: advances the window)
template <bool BLOCK>
__device__ __forceinline__ void rr64_token(bool valid, int64_t t, const bf16 *hu, const bf16 *a,
                                           const bf16 *bg, const float (&cw)[4], float (&um)[3],
                                           float &h, float &f, float &wr)
{
    float av = 0.f, bv = 0.f;
    h = 0.f;
    if (valid) {
        av = to_f(a[t]);
        bv = to_f(bg[t]);
        if (BLOCK) {
            const float uv = to_f(hu[t]);
            const float pre = cw[0] * um[2] + cw[1] * um[1] + cw[2] * um[0] + cw[3] * uv;
            um[2] = um[1];
            um[1] = um[0];
            um[0] = uv;
            h = pre * sigm(pre);
        } else {
            h = to_f(hu[t]);
        }
    }
    f = valid ? sigm(av) : 1.f;
    wr = valid ? sigm(bv) * h : 0.f;
}

// 32 consecutive bf16 of a B or C row (64-byte aligned) as fp32
__device__ __forceinline__ void row32(const bf16 *p, float (&v)[32])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 u = ((const uint4 *)p)[q];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
            v[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
}

// Aggregate from a zero state: x -> P x + S over the wave's tokens.
template <bool BLOCK>
__device__ void rr64_aggregate(int64_t L, int64_t Di, int bi, int64_t c, bool valid, int sh,
                               int64_t n0, const bf16 *hu, const bf16 *a, const bf16 *bg,
                               const bf16 *Bm, const float *conv_w, const bf16 *conv_state,
                               float &P, float (&S)[32])
{
    float cw[4], um[3];
    rr64_window<BLOCK>(L, Di, bi, c, valid, n0, hu, conv_w, conv_state, cw, um);
    P = 1.f;
#pragma unroll
    for (int s = 0; s < 32; ++s) S[s] = 0.f;
    for (int j = 0; j < kTk; ++j) {
        const int64_t n = n0 + j;
        if (n >= L) break;
        float h, f, wr, Bv[32];
        rr64_token<BLOCK>(valid, ((int64_t)bi * L + n) * Di + c, hu, a, bg, cw, um, h, f, wr);
        row32(Bm + ((int64_t)bi * L + n) * kN + 32 * sh, Bv);
#pragma unroll
        for (int s = 0; s < 32; ++s) S[s] = fmaf(f, S[s], wr * Bv[s]);
        P *= f;
    }
}

// Full recurrence from the entering state xin with the readout; the two state
// halves of a channel (lanes l and l ^ 32) add their partial dot products and
// the lower one stores y.  Every lane of the wave takes part (cross-lane swap).
template <bool BLOCK>
__device__ void rr64_output(int64_t L, int64_t Di, int bi, int64_t c, bool valid, int sh,
                            int64_t n0, float scale, const bf16 *hu, const bf16 *a,
                            const bf16 *bg, const bf16 *Bm, const bf16 *Cm, const float *D,
                            const bf16 *z, const float *conv_w, const bf16 *conv_state,
                            const float (&xin)[32], bf16 *y)
{
    float cw[4], um[3];
    rr64_window<BLOCK>(L, Di, bi, c, valid, n0, hu, conv_w, conv_state, cw, um);
    const float Dc = valid ? D[c] : 0.f;
    float x[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) x[s] = xin[s];
    for (int j = 0; j < kTk; ++j) {
        const int64_t n = n0 + j;
        if (n >= L) break;
        const int64_t t = ((int64_t)bi * L + n) * Di + c;
        float h, f, wr, Bv[32], Cv[32];
        rr64_token<BLOCK>(valid, t, hu, a, bg, cw, um, h, f, wr);
        row32(Bm + ((int64_t)bi * L + n) * kN + 32 * sh, Bv);
        row32(Cm + ((int64_t)bi * L + n) * kN + 32 * sh, Cv);
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            x[s] = fmaf(f, x[s], wr * Bv[s]);
            acc = fmaf(x[s], Cv[s], acc);
        }
        acc += xhalf(acc, sh != 0);
        float yv = fmaf(scale, acc, Dc * h);
        if (valid && sh == 0) {
            if (BLOCK) {
                const float zv = to_f(z[t]);
                yv *= zv * sigm(zv);
            }
            y[t] = from_f<bf16>(yv);
        }
    }
}

// ------------------------------------------------------------------- kernel
template <bool BLOCK>
__global__ __launch_bounds__(64 * kWv, 1) void fwd_mfma64_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_chunks,
    const float scale, const bf16 *__restrict__ hu, const bf16 *__restrict__ a,
    const bf16 *__restrict__ bg, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ x0, const bf16 *__restrict__ z,
    const float *__restrict__ conv_w, const bf16 *__restrict__ conv_state, bf16 *__restrict__ y,
    float *__restrict__ x_final, bf16 *__restrict__ conv_state_out, float *__restrict__ ckpt)
{
    constexpr int N = kN, T = kTk, W = kWv, H = BLOCK ? kHl : 0;
    // wave-uniform (readfirstlane keeps what derives from it in scalar registers)
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tbw = wv & 3, chh = wv >> 2;  // token block, channel half

    __shared__ __attribute__((aligned(16))) bf16 sU[H + kRw][kCT];  // h (scan) or u (block)
    __shared__ __attribute__((aligned(16))) bf16 sAB[2][kRw][kCT];  // a, b
    __shared__ __attribute__((aligned(16))) bf16 sB[kRw][N];        // B rows
    __shared__ __attribute__((aligned(16))) float sS[W][kCW][kSP];  // wave aggregates / entering states
    __shared__ float sP[W][kCW];

    const int n_rows = (int)(Bt * n_tiles);
    const int64_t n_waves = (L + T - 1) / T;
    const uint32_t rowb = (uint32_t)Di * 2;

    // Copy the h|u, a, b tile and the B rows of chunk ch of row `row` into LDS
    // (wave w: token rows 16 w .. 16 w + 15; wave 0 also the 16 rows of u
    // before the chunk).  A 64-channel row is 128 bytes: eight lanes per row.
    // The range ends with the last row's channel Di, so rows past L read 0.
    auto prefetch = [&](int row, int ch, int lane) {
        const int b_ = row / n_tiles;
        const int64_t cb = (int64_t)(row % n_tiles) * kCT;
        const int r0 = 16 * wv;
        const int64_t n_0 = (int64_t)ch * kRw;
        const int rows = (int)(L - n_0 < kRw ? L - n_0 : kRw);
        const int64_t tb = ((int64_t)b_ * L + n_0) * Di + cb;  // the tile's first element
        const uint32_t range = (uint32_t)rows * rowb - (uint32_t)cb * 2;
        const uint32_t vo = ((uint32_t)(r0 + (lane >> 3)) * (uint32_t)Di + 8 * (lane & 7)) * 2;
        const rsrc_t rh = make_rsrc(hu + tb, range);
        const rsrc_t ra = make_rsrc(a + tb, range);
        const rsrc_t rb = make_rsrc(bg + tb, range);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t so = (uint32_t)(8 * k) * rowb;
            dma16b<false>(rh, vo, so, &sU[H + r0 + 8 * k][0]);
            dma16b<false>(ra, vo, so, &sAB[0][r0 + 8 * k][0]);
            dma16b<false>(rb, vo, so, &sAB[1][r0 + 8 * k][0]);
        }
        if (BLOCK && wv == 0) {
            // rows n0-16 .. n0-1 of u (the first chunk's are replaced after the copy)
            const rsrc_t rs = make_rsrc(hu + (ch > 0 ? tb - 16 * Di : tb),
                                        ch > 0 ? 16u * rowb - (uint32_t)cb * 2 : 0u);
            const uint32_t vh = ((uint32_t)(lane >> 3) * (uint32_t)Di + 8 * (lane & 7)) * 2;
            dma16b<false>(rs, vh, 0u, &sU[0][0]);
            dma16b<false>(rs, vh, 8u * rowb, &sU[8][0]);
        }
        // B rows: 128 bytes, eight lanes per row
        const rsrc_t rB = make_rsrc(Bm + ((int64_t)b_ * L + n_0) * N, (uint32_t)rows * (N * 2));
        const uint32_t vb = (uint32_t)((r0 + (lane >> 3)) * N + 8 * (lane & 7)) * 2;
#pragma unroll
        for (int k = 0; k < 2; ++k) dma16b<false>(rB, vb, (uint32_t)(8 * k * N * 2), &sB[r0 + 8 * k][0]);
    };
    // C rows of this wave's 32 tokens as MFMA operands: token lane % 32,
    // K-block kb = states 16 kb + 8 (lane / 32) .. + 7 (rows past L read 0)
    auto load_c = [&](int row, int ch, int lane, bf16x8 (&cv)[4]) {
        const int b_ = row / n_tiles;
        const int64_t nw = (int64_t)ch * kRw + (int64_t)tbw * T;
        const int rows = nw < L ? (int)(L - nw < T ? L - nw : T) : 0;
        const rsrc_t rc =
            make_rsrc(Cm + ((int64_t)b_ * L + (nw < L ? nw : 0)) * N, (uint32_t)rows * (N * 2));
        const uint32_t vc = (uint32_t)((lane & 31) * N + 8 * (lane >> 5)) * 2;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            cv[kb] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rc, vc + 32 * kb, 0, 0));
    };

    // workgroup w takes rows w, w + G, w + 2G, ...
    int row = blockIdx.x, chunk = 0;
    if (row < n_rows) prefetch(row, 0, threadIdx.x & 63);
    float xr[8];  // the state carried along the row: wave (t, c), lane (channel, half h)
                  // holds states 16 t + 8 h .. + 7 of channel 32 c + channel
    float Dc = 0.f, cw0 = 0.f, cw1 = 0.f, cw2 = 0.f, cw3 = 0.f;

    while (row < n_rows) {
        wait_mem();
        __syncthreads();  // the tile of (row, chunk) is in LDS
        // lane-dependent values are re-derived every chunk (kept out of
        // loop-invariant code motion, which would pin per-lane addresses)
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int col = lane & 31;
        const int hh = lane >> 5;
        const bool upper = hh != 0;

        const int bi = row / n_tiles;
        const int64_t cbase = (int64_t)(row % n_tiles) * kCT;
        const int64_t n0 = (int64_t)chunk * kRw + (int64_t)tbw * T;
        const int64_t tokbase = (int64_t)bi * L;
        const bool active = n0 < L;
        const int Lw = active ? (int)(L - n0 < T ? L - n0 : T) : 0;  // valid tokens of the wave
        auto tok = [&](int i) -> int { return 8 * (i >> 2) + 4 * hh + (i & 3); };
        const int64_t c_col = cbase + kCW * chh + col;

        if (chunk == 0) {
            // per-channel constants of the row
            const int64_t cc = c_col < Di ? c_col : 0;
            Dc = D[cc];
            if (BLOCK) {
                cw0 = conv_w[cc * 4 + 0];
                cw1 = conv_w[cc * 4 + 1];
                cw2 = conv_w[cc * 4 + 2];
                cw3 = conv_w[cc * 4 + 3];
            }
            {
                const int s0 = 16 * tbw + 8 * hh;
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    xr[k] = (x0 && c_col < Di) ? x0[((int64_t)bi * Di + c_col) * N + s0 + k] : 0.f;
            }
            if (BLOCK) {
                // the conv window before the sequence start: the carried conv state or zeros
                if (threadIdx.x < 3 * kCT) {
                    const int r = threadIdx.x / kCT, chn = threadIdx.x % kCT;
                    const int64_t c = cbase + chn;
                    sU[H - 3 + r][chn] = (conv_state && c < Di)
                                             ? conv_state[((int64_t)bi * 3 + r) * Di + c]
                                             : (bf16)0;
                }
                __syncthreads();
            }
        }

        // the next chunk (of this row, else the first of the next row)
        int nrow = row, nchunk = chunk + 1;
        if (nchunk == n_chunks) {
            nchunk = 0;
            nrow = row + gridDim.x;
        }
        const bool has_next = nrow < n_rows;
        bf16x8 Cop[4];
        load_c(row, chunk, lane, Cop);  // arrives during the gates

        // ------------------------------------------------------ gates, W', P
        // Tokens past the end of the sequence (only in the last chunk of a row)
        // get f = 1 and w = 0, so they leave the state and the aggregate alone.
        float Pv[16], FT[16], Ptot, rQ;  // Ptot = P_T / P_p, rQ = P_p
        bf16x8 Whi[2], Wlo[2];
        bool ok = true;
        auto gates = [&](auto tail_c) {
            constexpr bool TL = decltype(tail_c)::value;
            // e_a = e^{-a}, e_b = e^{-b}; invP_n = prod_{k<=n} (1 + e_a) = 1/P_n in
            // the wave's 32 tokens.  One reciprocal r = 1 / (invP (1 + e_b))
            // gives sigma(b) = r invP and P = r (1 + e_b).
            float cum[16], eb[16], hv[16], tot[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rg = 32 * tbw + 8 * q + 4 * hh;  // tile row of the group's first token
                float uw[7];
                if (BLOCK) {
#pragma unroll
                    for (int k = 0; k < 7; ++k) uw[k] = to_f(sU[H + rg - 3 + k][kCW * chh + col]);
                }
                float run = 1.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    float h;
                    if (BLOCK) {
                        const float pre =
                            cw0 * uw[r] + cw1 * uw[r + 1] + cw2 * uw[r + 2] + cw3 * uw[r + 3];
                        h = pre * sigm(pre);
                    } else {
                        h = to_f(sU[rg + r][kCW * chh + col]);
                    }
                    float ea = ex2(to_f(sAB[0][rg + r][kCW * chh + col]) * -kLog2e);
                    eb[i] = ex2(to_f(sAB[1][rg + r][kCW * chh + col]) * -kLog2e);
                    if (TL) {
                        const bool tv = tok(i) < Lw;
                        ea = tv ? ea : 0.f;
                        h = tv ? h : 0.f;
                    }
                    run = fmaf(run, ea, run);  // prod (1 + e^{-a})
                    cum[i] = run;
                    hv[i] = h;
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
            ok = ok && (Q <= 0x1p96f) && (acc <= 0x1p96f);  // both halves; false for NaN
            rQ = rcp(Q);
            E[0] *= rQ;
            E[1] *= rQ;
            Ptot = rcp(acc);
            float wp[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float invP = E[i >> 2] * cum[i];
                const float qv = fmaf(invP, eb[i], invP);  // invP (1 + e^{-b})
                const float r = rcp(qv);
                const float t = hv[i] * invP;
                wp[i] = t * (r * invP);        // h sigma(b) / P
                Pv[i] = fmaf(r, eb[i], r);     // P
                FT[i] = Dc * t;                // y = P (G W' + C x_in + D h / P)
                ok = ok && (__builtin_fabsf(wp[i]) < 0x1p110f) && (qv < 0x1p120f);
            }
            split16(wp, Whi, Wlo);
        };
        if (Lw < T)
            gates(std::true_type{});
        else
            gates(std::false_type{});
        const bool wave_ok = __all(ok);

        // --------------------------------------------- B operands, G = C B^T
        bf16x8 Bop[4], Bsv[2][2];  // Bsv: A operand of B^T W' (rows = states 32 rt + col)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            Bop[kb] = __builtin_bit_cast(bf16x8, *(const uint4 *)&sB[32 * tbw + col][16 * kb + 8 * hh]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                Bsv[rt][i >> 3][i & 7] = as_bf(sB[32 * tbw + tok(i)][32 * rt + col]);
        // (before the copy below: a wait for C issued after it would wait for the copy too)
        f32x16 g = {};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) g = mfma(Bop[kb], Cop[kb], g);  // g[i] = B_tok(i) . C_col
        if (chunk == 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) asm volatile("" ::"v"(xr[k]));  // x0 has arrived
        }
        __syncthreads();  // every wave is done with the tile
        if (has_next) prefetch(nrow, nchunk, lane);

        // ------------- wave aggregate (P_T, S = P_T W'^T B) -> LDS, and G @ W'
        f32x16 Y;
        if (wave_ok) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x16 sacc = {};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    sacc = mfma(Bsv[rt][kb], Whi[kb], sacc);  // rows: state, columns: channel
                    sacc = mfma(Bsv[rt][kb], Wlo[kb], sacc);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = {sacc[4 * q] * Ptot, sacc[4 * q + 1] * Ptot,
                                      sacc[4 * q + 2] * Ptot, sacc[4 * q + 3] * Ptot};
                    *(float4 *)&sS[wv][col][32 * rt + 8 * q + 4 * hh] = v;
                }
            }
            if (!upper) sP[wv][col] = Ptot * rQ;  // P_T
            bf16x8 Ghi[2], Glo[2];
            float gv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) gv[i] = (tok(i) <= col) ? g[i] * scale : 0.f;
            split16(gv, Ghi, Glo);
#pragma unroll
            for (int i = 0; i < 16; ++i) Y[i] = FT[i];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                Y = mfma(Ghi[kb], Whi[kb], Y);
                Y = mfma(Ghi[kb], Wlo[kb], Y);
                Y = mfma(Glo[kb], Whi[kb], Y);
            }
        } else {
            float P, S[32];
            rr64_aggregate<BLOCK>(L, Di, bi, c_col, c_col < Di, hh, n0, hu, a, bg, Bm, conv_w,
                                  conv_state, P, S);
#pragma unroll
            for (int k = 0; k < 32; k += 4)
                *(float4 *)&sS[wv][col][32 * hh + k] = float4{S[k], S[k + 1], S[k + 2], S[k + 3]};
            if (!upper) sP[wv][col] = P;
        }
        __syncthreads();

        // ----------------- compose: entering state of every wave, carried state
        // Wave w holds states 16 w .. 16 w + 15 (lane = channel, 8 states per
        // half).  Each wave's aggregate is replaced by the state entering that
        // wave; the carried state moves past the whole chunk.
        {
            const int s0 = 16 * tbw + 8 * hh;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                const int w = 4 * chh + w4;  // the token blocks of this channel half
                const float pw = sP[w][col];
                float4 t[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) t[m] = *(const float4 *)&sS[w][col][s0 + 4 * m];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    *(float4 *)&sS[w][col][s0 + 4 * m] =
                        float4{xr[4 * m], xr[4 * m + 1], xr[4 * m + 2], xr[4 * m + 3]};
                    xr[4 * m + 0] = fmaf(pw, xr[4 * m + 0], t[m].x);
                    xr[4 * m + 1] = fmaf(pw, xr[4 * m + 1], t[m].y);
                    xr[4 * m + 2] = fmaf(pw, xr[4 * m + 2], t[m].z);
                    xr[4 * m + 3] = fmaf(pw, xr[4 * m + 3], t[m].w);
                }
            }
            if (chunk == n_chunks - 1 && c_col < Di) {
                if (x_final) {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        x_final[((int64_t)bi * Di + c_col) * N + s0 + k] = xr[k];
                }
                if (BLOCK && tbw == 0 && !upper && conv_state_out) {
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        const int64_t m = L - 3 + k;
                        bf16 v = 0;
                        if (m >= 0)
                            v = hu[(tokbase + m) * Di + c_col];
                        else if (conv_state)
                            v = conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c_col];
                        conv_state_out[((int64_t)bi * 3 + k) * Di + c_col] = v;
                    }
                }
            }
        }
        __syncthreads();

        // --------------------- this wave's entering state, K-slots of the
        // B operand: channel col, states 16 kb + 8 hh + e
        float xs[4][8];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const float4 u0 = *(const float4 *)&sS[wv][col][16 * kb + 8 * hh];
            const float4 u1 = *(const float4 *)&sS[wv][col][16 * kb + 8 * hh + 4];
            xs[kb][0] = u0.x, xs[kb][1] = u0.y, xs[kb][2] = u0.z, xs[kb][3] = u0.w;
            xs[kb][4] = u1.x, xs[kb][5] = u1.y, xs[kb][6] = u1.z, xs[kb][7] = u1.w;
        }
        if (ckpt && active) {
            float *cp = ckpt + (((int64_t)bi * n_waves + (int64_t)chunk * 4 + tbw) * N) * Di + cbase + kCW * chh;
            const rsrc_t rc = make_rsrc(cp, (uint32_t)(N * Di * 4));
            // every offset in the lane's voffset (the rule for range-checked
            // offsets that every kernel here keeps)
            const uint32_t vo = c_col < Di ? (uint32_t)((8 * hh) * Di + col) * 4 : kOOB;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(xs[kb][e]), rc,
                        c_col < Di ? vo + (uint32_t)((16 * kb + e) * Di) * 4 : kOOB, 0, 0);
        }

        if (!wave_ok) {
            if (y) {
                // the fallback works in lane = (channel, state half) layout
                float xin[32];
#pragma unroll
                for (int k = 0; k < 32; k += 4) {
                    const float4 u = *(const float4 *)&sS[wv][col][32 * hh + k];
                    xin[k] = u.x, xin[k + 1] = u.y, xin[k + 2] = u.z, xin[k + 3] = u.w;
                }
                rr64_output<BLOCK>(L, Di, bi, c_col, c_col < Di, hh, n0, scale, hu, a, bg, Bm,
                                   Cm, D, z, conv_w, conv_state, xin, y);
            }
        } else if (y) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = xs[kb][e] * (scale * rQ);  // P_p x_in
                bf16x8 xh, xl;
                split8(v, xh, xl);
                Y = mfma(Cop[kb], xh, Y);
                Y = mfma(Cop[kb], xl, Y);
            }
            const int64_t ebase = (tokbase + (active ? n0 : 0)) * Di + cbase;
            const uint32_t row2 = (uint32_t)Di * 2;
            const rsrc_t ry = make_rsrc(y + ebase, (uint32_t)Lw * row2);
            const rsrc_t rz = make_rsrc(BLOCK ? (const void *)(z + ebase) : (const void *)y,
                                        BLOCK ? (uint32_t)Lw * row2 : 0u);
            const bool vc = c_col < Di;
            // z first, all at once: the y stores below may alias it as far as the
            // compiler can tell, so a load between them would wait out a round trip
            uint32_t zb[16];
            if (BLOCK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t vo = vc ? (uint32_t)((4 * hh + r) * Di + kCW * chh + col) * 2 : kOOB;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        zb[4 * q + r] = __builtin_amdgcn_raw_buffer_load_b16(
                            rz, vo + (uint32_t)(8 * q) * row2, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t vo = vc ? (uint32_t)((4 * hh + r) * Di + kCW * chh + col) * 2 : kOOB;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = 4 * q + r;
                    // the row offset joins the lane offset (the range, Lw rows, then
                    // drops rows past the wave's last token; kOOB drops channels past Di)
                    const uint32_t off = vo + (uint32_t)(8 * q) * row2;
                    float yv = Pv[i] * Y[i];
                    if (BLOCK) {
                        const float zv = __uint_as_float(zb[i] << 16);
                        yv *= zv * sigm(zv);
                    }
                    // (no nontemporal hint: L2 merges the 64-byte pieces into whole lines)
                    __builtin_amdgcn_raw_buffer_store_b16(from_f<bf16>(yv), ry, off, 0, 0);
                }
            }
        }
        row = nrow;
        chunk = nchunk;
    }
}

bool use_fwd_mfma64(const FwdArgs &g)
{
    const auto al16 = [](const void *p) { return ((uintptr_t)p % 16) == 0; };
    const int64_t rows = g.Bt * ((g.Di + kCT - 1) / kCT);
    // (buffer ranges of 128 token rows stay below 2^32 bytes)
    return g.io == 1 && g.N == kN && g.Di % 8 == 0 && g.Di < ((int64_t)1 << 24) && rows >= 32 &&
           al16(g.B) && al16(g.C) && al16(g.hu) && al16(g.a) && al16(g.b);
}

hipError_t launch_fwd_mfma64(const FwdArgs &g, hipStream_t stream)
{
    const int n_tiles = (int)((g.Di + kCT - 1) / kCT);
    const int n_chunks = (int)((g.L + kRw - 1) / kRw);
    const int64_t rows = g.Bt * n_tiles;
    const int64_t slots = (int64_t)device_cu_count();  // one workgroup per CU
    const int64_t grid = rows < slots ? rows : slots;
    if (g.block)
        hipLaunchKernelGGL(fwd_mfma64_kernel<true>, dim3(grid), dim3(64 * kWv), 0, stream, g.Bt,
                           g.L, g.Di, n_tiles, n_chunks, g.scale, (const bf16 *)g.hu,
                           (const bf16 *)g.a, (const bf16 *)g.b, (const bf16 *)g.B,
                           (const bf16 *)g.C, g.D, g.x0, (const bf16 *)g.z, g.conv_w,
                           (const bf16 *)g.conv_state, (bf16 *)g.y, g.x_final,
                           (bf16 *)g.conv_state_out, g.ckpt);
    else
        hipLaunchKernelGGL(fwd_mfma64_kernel<false>, dim3(grid), dim3(64 * kWv), 0, stream, g.Bt,
                           g.L, g.Di, n_tiles, n_chunks, g.scale, (const bf16 *)g.hu,
                           (const bf16 *)g.a, (const bf16 *)g.b, (const bf16 *)g.B,
                           (const bf16 *)g.C, g.D, g.x0, (const bf16 *)g.z, g.conv_w,
                           (const bf16 *)g.conv_state, (bf16 *)g.y, g.x_final,
                           (bf16 *)g.conv_state_out, g.ckpt);
    return hipGetLastError();
}

}  // namespace naju

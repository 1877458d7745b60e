// naju_fwd_mfma.hip -- matrix-core forward of the Naju selective scan for bf16
// activations and d_state 16 (scan and block).
//
// Same recurrence/readout ("Core equations" of the Naju reproduction README,
// arXiv 2607.21000), same workgroup decomposition and decoupled look-back as
// naju_fwd.hip; only the work inside a wave's 32-token chunk changes.  With
// the chunk-local running product P_n = prod_{j<=n} f_j (per channel) and the
// rescaled writes W'_k = w_k / P_k,
//     x_n = P_n (x_in + sum_{k<=n} W'_k B_k)
//     y_n = P_n ( sum_{k<=n} G[n,k] W'_k  +  C_n x_in / sqrt(N) ) + D h_n,
//     G  = tril(C B^T) / sqrt(N)   (32 x 32, shared by every channel)
// so the three contractions of a chunk -- G @ W', C @ x_in^T and the chunk's
// state increment W'^T B -- run on MFMA (v_mfma_f32_32x32x16_bf16), while the
// VALU only forms the gates, P and W' and applies the epilogue.  Operands are
// split into bf16 hi + lo parts (x = hi + lo to ~2^-17 relative), so the
// products keep close to fp32 accuracy with fp32 accumulation.
//
// Lane layout: lane l owns column l%32 of the two 32-wide MFMA column tiles,
// which are the adjacent channels 2(l%32) and 2(l%32) + 1 (so a lane's y, z and
// checkpoint values of a token are one 4- or 8-byte access), and, in its half
// h = l/32, the 16 chunk tokens {8q + 4h + r}.  That set is both the
// lane's row set in the 32x32 accumulator and (by choosing the K-slot order)
// its K-slots in the A/B operands, so gates, W', P and the outputs of a token
// all live in the lane that needs them.
//
// Safety: the factorisation needs 1/P over the chunk to stay in range.  A wave
// whose chunk has prod(1/f) > 2^64 or a non-finite input falls back to the
// plain register recurrence for that chunk (exact for any input).
#include <type_traits>

#include "naju_device.h"
#include "naju_launch.h"
#include "naju_mfma.h"

namespace naju {

// ------------------------------------------------------------------ fallback
// Register recurrence of one wave's chunk in lane = channel layout (64
// channels), used when the rescaled form is unsafe.  Aggregate from a zero
// state: x -> P x + S.
template <bool BLOCK>
__device__ __forceinline__ void rr_aggregate(int64_t L, int64_t Di, int bi, int64_t c, bool valid,
                                             int64_t n0, const bf16 *hu, const bf16 *a,
                                             const bf16 *bg, const bf16 *Bm, const float *conv_w,
                                             const bf16 *conv_state, float &P, float (&S)[16])
{
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, um1 = 0.f, um2 = 0.f, um3 = 0.f;
    if (BLOCK && valid) {
        w0 = conv_w[c * 4 + 0];
        w1 = conv_w[c * 4 + 1];
        w2 = conv_w[c * 4 + 2];
        w3 = conv_w[c * 4 + 3];
        float hv[3];
        for (int k = 1; k <= 3; ++k) {
            const int64_t m = n0 - k;
            float v = 0.f;
            if (m >= 0 && m < L)
                v = to_f(hu[((int64_t)bi * L + m) * Di + c]);
            else if (m < 0 && conv_state)
                v = to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
            hv[k - 1] = v;
        }
        um1 = hv[0];
        um2 = hv[1];
        um3 = hv[2];
    }
    P = 1.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) S[s] = 0.f;
    for (int j = 0; j < 32; ++j) {
        const int64_t n = n0 + j;
        if (n >= L) break;
        const int64_t t = ((int64_t)bi * L + n) * Di + c;
        float av = 0.f, bv = 0.f, hv = 0.f;
        if (valid) {
            av = to_f(a[t]);
            bv = to_f(bg[t]);
            if (BLOCK) {
                const float uv = to_f(hu[t]);
                const float pre = w0 * um3 + w1 * um2 + w2 * um1 + w3 * uv;
                um3 = um2;
                um2 = um1;
                um1 = uv;
                hv = pre * sigm(pre);
            } else {
                hv = to_f(hu[t]);
            }
        }
        const float f = valid ? sigm(av) : 1.f;
        const float wr = valid ? sigm(bv) * hv : 0.f;
        const bf16 *Bn = Bm + ((int64_t)bi * L + n) * 16;
#pragma unroll
        for (int s = 0; s < 16; ++s) S[s] = fmaf(f, S[s], wr * to_f(Bn[s]));
        P *= f;
    }
}

// Full recurrence with readout from the entering state; writes y.
template <bool BLOCK>
__device__ __forceinline__ void rr_output(int64_t L, int64_t Di, int bi, int64_t c, bool valid,
                                          int64_t n0, float scale, const bf16 *hu, const bf16 *a,
                                          const bf16 *bg, const bf16 *Bm, const bf16 *Cm,
                                          const float *D, const bf16 *z, const float *conv_w,
                                          const bf16 *conv_state, const float (&xin)[16], bf16 *y)
{
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, um1 = 0.f, um2 = 0.f, um3 = 0.f;
    if (BLOCK && valid) {
        w0 = conv_w[c * 4 + 0];
        w1 = conv_w[c * 4 + 1];
        w2 = conv_w[c * 4 + 2];
        w3 = conv_w[c * 4 + 3];
        float hv[3];
        for (int k = 1; k <= 3; ++k) {
            const int64_t m = n0 - k;
            float v = 0.f;
            if (m >= 0 && m < L)
                v = to_f(hu[((int64_t)bi * L + m) * Di + c]);
            else if (m < 0 && conv_state)
                v = to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
            hv[k - 1] = v;
        }
        um1 = hv[0];
        um2 = hv[1];
        um3 = hv[2];
    }
    const float Dc = valid ? D[c] : 0.f;
    float x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = xin[s];
    for (int j = 0; j < 32; ++j) {
        const int64_t n = n0 + j;
        if (n >= L) break;
        const int64_t t = ((int64_t)bi * L + n) * Di + c;
        float av = 0.f, bv = 0.f, hv = 0.f;
        if (valid) {
            av = to_f(a[t]);
            bv = to_f(bg[t]);
            if (BLOCK) {
                const float uv = to_f(hu[t]);
                const float pre = w0 * um3 + w1 * um2 + w2 * um1 + w3 * uv;
                um3 = um2;
                um2 = um1;
                um1 = uv;
                hv = pre * sigm(pre);
            } else {
                hv = to_f(hu[t]);
            }
        }
        const float f = valid ? sigm(av) : 1.f;
        const float wr = valid ? sigm(bv) * hv : 0.f;
        const bf16 *Bn = Bm + ((int64_t)bi * L + n) * 16;
        const bf16 *Cn = Cm + ((int64_t)bi * L + n) * 16;
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            x[s] = fmaf(f, x[s], wr * to_f(Bn[s]));
            acc = fmaf(x[s], to_f(Cn[s]), acc);
        }
        float yv = fmaf(scale, acc, Dc * hv);
        if (valid) {
            if (BLOCK) {
                const float zv = to_f(z[t]);
                yv *= zv * sigm(zv);
            }
            y[t] = from_f<bf16>(yv);
        }
    }
}

// ------------------------------------------------------------------- kernel
// Persistent: workgroup w of G takes tickets w, w + G, w + 2G, ... (workgroup
// chunks of 64 channels x 128 tokens, chunk-major, so a look-back predecessor
// always holds a smaller ticket, taken by a workgroup that is resident and in
// an earlier or the same round).  The static schedule needs no shared ticket
// counter; one count per workgroup at exit lets the last one advance the epoch.
// The h|u, a, b tile of the next ticket (and, for the block, the eight rows of
// u before it, for the conv window) is copied HBM -> LDS with
// global_load_lds_dwordx4 (no VGPRs involved) while the current one runs its
// matrix products, look-back and epilogue.
constexpr int kRows = kFwdT * kMfmaW;  // tokens per workgroup chunk
constexpr int kHalo = 8;               // rows of u kept before the chunk (block)


template <bool BLOCK>
__global__ __launch_bounds__(64 * kMfmaW, 2) void fwd_mfma_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_chunks,
    const float scale, const bf16 *__restrict__ hu, const bf16 *__restrict__ a,
    const bf16 *__restrict__ bg, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ x0, const bf16 *__restrict__ z,
    const float *__restrict__ conv_w, const bf16 *__restrict__ conv_state, bf16 *__restrict__ y,
    float *__restrict__ x_final, bf16 *__restrict__ conv_state_out, float *__restrict__ ckpt,
    WsHeader *hdr, uint64_t *agg, uint64_t *incl, const int lazy_agg)
{
    constexpr int N = 16, T = kFwdT, W = kMfmaW, H = BLOCK ? kHalo : 0;
    // Scan: each wave reads the second column tile's h, a, b into registers
    // (two tokens per register) before the first tile's gates, so the next
    // ticket's copy can start halfway through the gate arithmetic instead of
    // after it (holding all of the tile in registers spills).  The block's conv
    // window would need twice the registers, so it keeps the later start.
    constexpr bool EARLY = !BLOCK;
    static_assert(T == 32, "one 32x32 MFMA tile of tokens per wave");
    // wave-uniform (readfirstlane keeps what derives from it in scalar registers)
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    __shared__ __attribute__((aligned(16))) bf16 sU[H + kRows][64];  // h (scan) or u (block)
    __shared__ __attribute__((aligned(16))) bf16 sAB[2][kRows][64];  // a, b
    __shared__ __attribute__((aligned(16))) bf16 sBC[2][kRows][16];  // B, C rows
    __shared__ uint32_t s_epoch;
    __shared__ float sP[W][64];
    __shared__ float sS[W][16][64];
    __shared__ float sX[16][64];

    const uint32_t per_chunk = (uint32_t)(Bt * n_tiles);
    const uint32_t total = per_chunk * (uint32_t)n_chunks;
    const int64_t n_waves = (L + T - 1) / T;

    // Copy the h|u, a, b tile and the B, C rows of ticket tk into LDS.  Only
    // waves 2 and 3 copy (64 rows each; wave 2 also the rows of u before the
    // chunk and the B rows, wave 3 the C rows): a wave's wait for its own
    // memory operations covers every one it issued, and waves 0 and 1, which
    // run the look-back, must not wait for a tile copy on every flag read.
    // The copies carry the nontemporal hint (aux = 2): every byte is used once,
    // so it should not displace the look-back traffic in L2.  The y stores do
    // not: each store instruction writes 64-byte pieces of lines, which L2 merges
    // into whole lines before writing back (with the hint: scan forward 5 %
    // slower).
    auto prefetch = [&](uint32_t tk, int lane) {
        const int ch = (int)(tk / per_chunk);
        const int rm = (int)(tk % per_chunk);
        const int b_ = rm / n_tiles;
        const int64_t cbase_t = (int64_t)(rm % n_tiles) * 64;
        const int r0 = 64 * (wv - 2);
        const int64_t n_0 = (int64_t)ch * kRows;
        const int rows = (int)(L - n_0 < kRows ? L - n_0 : kRows);
        const uint32_t rowb = (uint32_t)Di * 2;
        const int64_t tb = ((int64_t)b_ * L + n_0) * Di + cbase_t;  // the tile's first element
        // lane: row lane / 8 of an 8-row group, 16-byte column chunk lane % 8,
        // relative to the tile's first channel; the range ends with the last
        // row's channel Di, so rows past L read 0 (channels past Di of the
        // other rows read the next row's first channels; no output uses them)
        const uint32_t range = (uint32_t)rows * rowb - (uint32_t)cbase_t * 2;
        const uint32_t vo = ((uint32_t)(r0 + (lane >> 3)) * (uint32_t)Di + 8 * (lane & 7)) * 2;
        const rsrc_t rh = make_rsrc(hu + tb, range);
        const rsrc_t ra = make_rsrc(a + tb, range);
        const rsrc_t rb = make_rsrc(bg + tb, range);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t so = (uint32_t)(8 * k) * rowb;
            dma16b(rh, vo, so, &sU[H + r0 + 8 * k][0]);
            dma16b(ra, vo, so, &sAB[0][r0 + 8 * k][0]);
            dma16b(rb, vo, so, &sAB[1][r0 + 8 * k][0]);
        }
        if (BLOCK && wv == 2) {
            // rows n0-8 .. n0-1 of u (the first chunk's are replaced after the copy)
            const rsrc_t rs = make_rsrc(hu + (ch > 0 ? tb - 8 * Di : tb),
                                        ch > 0 ? 8u * rowb - (uint32_t)cbase_t * 2 : 0u);
            const uint32_t vh = ((uint32_t)(lane >> 3) * (uint32_t)Di + 8 * (lane & 7)) * 2;
            dma16b(rs, vh, 0u, &sU[0][0]);
        }
        // B rows (wave 2) or C rows (wave 3): lane = row lane / 2 of a 32-row group
        // (no nontemporal hint: every channel tile of the batch row reads them)
        const uint32_t vb = (uint32_t)((lane >> 1) * N + 8 * (lane & 1)) * 2;
        if (wv == 2) {
            const rsrc_t rs = make_rsrc(Bm + ((int64_t)b_ * L + n_0) * N, (uint32_t)rows * (N * 2));
#pragma unroll
            for (int k = 0; k < 4; ++k) dma16b<false>(rs, vb, (uint32_t)(32 * k * N * 2), &sBC[0][32 * k][0]);
        } else {
            const rsrc_t rs = make_rsrc(Cm + ((int64_t)b_ * L + n_0) * N, (uint32_t)rows * (N * 2));
#pragma unroll
            for (int k = 0; k < 4; ++k) dma16b<false>(rs, vb, (uint32_t)(32 * k * N * 2), &sBC[1][32 * k][0]);
        }
    };

    // D of a ticket's channels (2 (lane % 32) + j), loaded one ticket ahead and
    // before the copy: a load issued after the copy would, when waited for, also
    // wait for the copy (memory operations complete in order)
    float Dn[2] = {0.f, 0.f};
    auto loadD = [&](uint32_t tk, int ln) {
        const int rm = (int)(tk % per_chunk);
        const int64_t cb = (int64_t)(rm % n_tiles) * 64;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t c = cb + 2 * (ln & 31) + j;
            Dn[j] = D[c < Di ? c : 0];
        }
    };
    if (threadIdx.x == 0) s_epoch = (ld_agent(&hdr->epoch) + 1u) & 0x3FFFFFFFu;
    uint32_t cur = blockIdx.x;
    if (EARLY && cur < total) loadD(cur, threadIdx.x & 63);
    if (cur < total && wv >= 2) prefetch(cur, threadIdx.x & 63);
    __syncthreads();
    const uint32_t ep = s_epoch;

    while (cur < total) {
        wait_mem();
        __syncthreads();  // the tile of `cur` is in LDS
        // lane-dependent values are re-derived every ticket (kept out of
        // loop-invariant code motion, which would otherwise pin dozens of
        // per-lane addresses in registers across the whole loop)
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int col = lane & 31;
        const int hh = lane >> 5;
        const bool upper = hh != 0;

        const int chunk = (int)(cur / per_chunk);
        const int rem = (int)(cur % per_chunk);
        const int bi = rem / n_tiles;
        const int tile = rem % n_tiles;
        const int64_t cbase = (int64_t)tile * 64;
        const int64_t n0 = (int64_t)chunk * kRows + (int64_t)wv * T;
        const int64_t tokbase = (int64_t)bi * L;
        const bool active = n0 < L;
        const int Lw = active ? (int)(L - n0 < T ? L - n0 : T) : 0;  // valid tokens of the wave
        auto tok = [&](int i) -> int { return 8 * (i >> 2) + 4 * hh + (i & 3); };

        if (BLOCK && chunk == 0) {
            // the conv window before the sequence start: the carried conv state or zeros
            if (threadIdx.x < 3 * 64) {
                const int r = threadIdx.x >> 6, chn = threadIdx.x & 63;
                const int64_t c = cbase + chn;
                sU[H - 3 + r][chn] = (conv_state && c < Di)
                                         ? conv_state[((int64_t)bi * 3 + r) * Di + c]
                                         : (bf16)0;
            }
            __syncthreads();
        }

        // ------------------------------------------------ token-shared operands
        bf16x8 Bop, Cop, Csc, Bsv[2];
        {
            const uint4 qb = *(const uint4 *)&sBC[0][32 * wv + col][8 * hh];
            const uint4 qc = *(const uint4 *)&sBC[1][32 * wv + col][8 * hh];
            const uint4 z4 = {0u, 0u, 0u, 0u};
            Bop = __builtin_bit_cast(bf16x8, col < Lw ? qb : z4);
            Cop = __builtin_bit_cast(bf16x8, col < Lw ? qc : z4);
#pragma unroll
            for (int s = 0; s < 8; ++s) Csc[s] = (__bf16)((float)Cop[s] * scale);
            // (the reads are made unconditional: a select after each read would
            // otherwise become a branch around it, with a wait of its own)
            uint32_t bv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) bv[i] = sBC[0][32 * wv + tok(i)][col & 15];
            asm volatile(""
                         : "+v"(bv[0]), "+v"(bv[1]), "+v"(bv[2]), "+v"(bv[3]), "+v"(bv[4]),
                           "+v"(bv[5]), "+v"(bv[6]), "+v"(bv[7]), "+v"(bv[8]), "+v"(bv[9]),
                           "+v"(bv[10]), "+v"(bv[11]), "+v"(bv[12]), "+v"(bv[13]),
                           "+v"(bv[14]), "+v"(bv[15]));
#pragma unroll
            for (int i = 0; i < 16; ++i)
                Bsv[i >> 3][i & 7] = as_bf((col < N && tok(i) < Lw) ? (bf16)bv[i] : (bf16)0);
        }

        // ------------------------------------------------------ gates, W', P
        // Tokens past the end of the sequence (only in the last wave of a row)
        // get f = 1 and w = 0, so they leave the state and the aggregate alone.
        const uint32_t nxt = cur + gridDim.x;
        const float Dcur[2] = {Dn[0], Dn[1]};
        uint32_t rw[3][8];  // h, a, b of column tile 1, tokens (2p, 2p + 1) in the two halves
        if constexpr (EARLY) {
            const int chn = 2 * col + 1;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int r0 = 32 * wv + tok(2 * p), r1 = 32 * wv + tok(2 * p + 1);
                rw[0][p] = (uint32_t)sU[r0][chn] | ((uint32_t)sU[r1][chn] << 16);
                rw[1][p] = (uint32_t)sAB[0][r0][chn] | ((uint32_t)sAB[0][r1][chn] << 16);
                rw[2][p] = (uint32_t)sAB[1][r0][chn] | ((uint32_t)sAB[1][r1][chn] << 16);
            }
        }
        auto raw = [&](int t, int i) -> float {
            const uint32_t v = rw[t][i >> 1];
            return __uint_as_float((i & 1) ? (v & 0xffff0000u) : (v << 16));
        };
        float Pv[2][16], FT[2][16];
        bf16x8 Whi[2][2], Wlo[2][2];
        float Ptot[2];
        bool ok = true;
        auto gates = [&](auto tail_c) {
            constexpr bool TL = decltype(tail_c)::value;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (EARLY && j == 1) {
                    __syncthreads();  // every wave holds what it needs of the tile
                    if (nxt < total) {
                        loadD(nxt, lane);
                        if (wv >= 2) prefetch(nxt, lane);
                    }
                }
                const bool rg1 = EARLY && j == 1;  // tile 1 from registers
                const int chn = 2 * col + j;
                const int64_t c = cbase + chn;
                const int64_t cc = c < Di ? c : 0;
                const float Dc = EARLY ? Dcur[j] : D[cc];
                float cw0 = 0.f, cw1 = 0.f, cw2 = 0.f, cw3 = 0.f;
                if (BLOCK) {
                    cw0 = conv_w[cc * 4 + 0];
                    cw1 = conv_w[cc * 4 + 1];
                    cw2 = conv_w[cc * 4 + 2];
                    cw3 = conv_w[cc * 4 + 3];
                }
                // e_a = e^{-a}, e_b = e^{-b}; invP_n = prod_{k<=n} (1 + e_a) = 1/P_n in
                // the wave's 32 tokens.  One reciprocal r = 1 / (invP (1 + e_b))
                // gives sigma(b) = r invP and P = r (1 + e_b).
                float cum[16], eb[16], hv[16], tot[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rg = 32 * wv + 8 * q + 4 * hh;  // tile row of the group's first token
                    float uw[7];
                    if (BLOCK) {
#pragma unroll
                        for (int k = 0; k < 7; ++k) uw[k] = to_f(sU[H + rg - 3 + k][chn]);
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
                            h = rg1 ? raw(0, i) : to_f(sU[rg + r][chn]);
                        }
                        float ea = ex2((rg1 ? raw(1, i) : to_f(sAB[0][rg + r][chn])) * -kLog2e);
                        eb[i] = ex2((rg1 ? raw(2, i) : to_f(sAB[1][rg + r][chn])) * -kLog2e);
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
                float E[4], acc = 1.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float pt = xhalf(tot[q], upper);  // partner group (q, 1-h)
                    // token order of the groups: (0,0) (0,1) (1,0) (1,1) ...
                    E[q] = upper ? acc * pt : acc;
                    acc *= tot[q] * pt;
                }
                ok = ok && (acc <= 18446744073709551616.f);  // 2^64; false for NaN
                Ptot[j] = rcp(acc);
                float wp[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float invP = E[i >> 2] * cum[i];
                    const float qv = fmaf(invP, eb[i], invP);  // invP (1 + e^{-b})
                    const float r = rcp(qv);
                    const float t = hv[i] * invP;
                    wp[i] = t * (r * invP);     // h sigma(b) / P
                    Pv[j][i] = fmaf(r, eb[i], r);  // P
                    FT[j][i] = Dc * t;          // y = P (G W' + C x_in + D h / P)
                    ok = ok && (__builtin_fabsf(wp[i]) < 1e30f) && (qv < 1.329228e36f);  // 2^120
                }
                split16(wp, Whi[j], Wlo[j]);
            }
        };
        if (Lw < T)
            gates(std::true_type{});
        else
            gates(std::false_type{});
        const bool wave_ok = __all(ok);
        if constexpr (!EARLY) {
            __syncthreads();  // every wave is done with the tile
            if (nxt < total && wv >= 2) prefetch(nxt, lane);
        }

        // ------------------------------------- chunk aggregates (P_T, S) -> LDS
        // S = P_T (W'^T B), formed as B^T W' so each lane holds its own channel
        f32x16 Y[2];
        if (wave_ok) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x16 sacc = {};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    sacc = mfma(Bsv[kb], Whi[j][kb], sacc);  // rows: state, columns: channel
                    sacc = mfma(Bsv[kb], Wlo[j][kb], sacc);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) sS[wv][tok(i)][2 * col + j] = sacc[i] * Ptot[j];
                if (!upper) sP[wv][2 * col + j] = Ptot[j];
            }
        } else {
            float P, S[16];
            rr_aggregate<BLOCK>(L, Di, bi, cbase + lane, cbase + lane < Di, n0, hu, a, bg, Bm,
                                conv_w, conv_state, P, S);
            sP[wv][lane] = P;
#pragma unroll
            for (int s = 0; s < 16; ++s) sS[wv][s][lane] = S[s];
        }
        __syncthreads();

        // ----------------------------------------- intra-chunk term G @ W'
        if (wave_ok) {
            f32x16 g = {};
            g = mfma(Bop, Cop, g);  // g[i] = C_{col} . B_{tok(i)} = G[col][tok(i)]
            bf16x8 Ghi[2], Glo[2];
            float gv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) gv[i] = (tok(i) <= col) ? g[i] * scale : 0.f;
            split16(gv, Ghi, Glo);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x16 acc;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = FT[j][i];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    acc = mfma(Ghi[kb], Whi[j][kb], acc);
                    acc = mfma(Ghi[kb], Wlo[j][kb], acc);
                    acc = mfma(Glo[kb], Whi[j][kb], acc);
                }
                Y[j] = acc;
            }
        }

        const int64_t c_lane = cbase + lane;
        const bool valid_lane = c_lane < Di;

        // -------------------------------- look-back for the entering state
        // Waves 0 and 1 (which issue no tile copies) carry states 8w..8w+7 of
        // the 64 channels (lane = channel); each publishes and reads its own
        // slots, so the two look back in parallel.  Every published value is a
        // tagged word (the call's epoch and the kind: aggregate or inclusive
        // state) written by one agent-scope store, so publishing needs no wait
        // and no flag, and a reader takes a predecessor's values once all 64
        // lanes' words carry the current tag: one round trip when the nearest
        // predecessor's inclusive state is out, else its aggregate is folded
        // and the look-back moves one chunk further.
        if (wv < 2) {
            constexpr int SG = 8;
            const int s0 = SG * wv;
            float Pt = 1.f, St[SG];
#pragma unroll
            for (int k = 0; k < SG; ++k) St[k] = 0.f;
            for (int w = 0; w < W; ++w) {
                const float pw = sP[w][lane];
#pragma unroll
                for (int k = 0; k < SG; ++k) St[k] = fmaf(pw, St[k], sS[w][s0 + k][lane]);
                Pt *= pw;
            }
            const size_t me = ((size_t)bi * n_tiles + tile) * n_chunks + chunk;
            const size_t mg = me * 2 + wv;  // this wave's payload slot
            const uint32_t tagA = make_flag(ep, kFlagAgg), tagI = make_flag(ep, kFlagIncl);
            float xin[SG];
            if (chunk == 0) {
#pragma unroll
                for (int k = 0; k < SG; ++k)
                    xin[k] = (x0 && valid_lane) ? x0[(bi * Di + c_lane) * N + s0 + k] : 0.f;
            } else {
                // The aggregate is published before the walk, or (lazy_agg) only
                // once this chunk finds it has to wait: a successor needs it only
                // while this chunk's inclusive state is not out, and the stores are
                // a sixth of the call's traffic.  Lazy publication pays when a round
                // of resident workgroups spans few chunks of each row (the nearest
                // predecessor is then usually done); with deep chains every chunk
                // waits, and publishing late delays the walks behind it.
                bool published = false;
                auto publish = [&]() {
                    uint64_t *ag = agg + mg * ((SG + 1) * 64);
                    st_tagged(ag + lane, Pt, tagA);
#pragma unroll
                    for (int k = 0; k < SG; ++k) st_tagged(ag + (1 + k) * 64 + lane, St[k], tagA);
                    published = true;
                };
                if (!lazy_agg) publish();
                float accP = 1.f, accS[SG];
#pragma unroll
                for (int k = 0; k < SG; ++k) accS[k] = 0.f;
                size_t jx = me - 1;  // nearest predecessor not folded in yet
                int left = chunk;    // predecessors of this row not folded in yet
                uint32_t spins = 0;
                for (;;) {
                    // the predecessor's inclusive state, else its aggregate (loading
                    // both together measured slower: the extra words cost more than
                    // the round trip they save; a row's first chunk publishes only
                    // its inclusive state, so the walk always ends at one)
                    const uint64_t *pi = incl + (jx * 2 + wv) * (SG * 64);
                    const uint64_t *pa = agg + (jx * 2 + wv) * ((SG + 1) * 64);
                    uint64_t iv[SG], av[SG + 1];
#pragma unroll
                    for (int k = 0; k < SG; ++k) iv[k] = ld_tagged(pi + k * 64 + lane);
                    bool ri = true;
#pragma unroll
                    for (int k = 0; k < SG; ++k) ri = ri && tagged_tag(iv[k]) == tagI;
                    if (__all(ri)) {
#pragma unroll
                        for (int k = 0; k < SG; ++k)
                            xin[k] = fmaf(accP, tagged_value(iv[k]), accS[k]);
                        break;
                    }
                    if (!published) publish();
#pragma unroll
                    for (int k = 0; k <= SG; ++k) av[k] = ld_tagged(pa + k * 64 + lane);
                    // (only the inclusive state of the row's first chunk ends the walk)
                    bool ra = left > 1;
#pragma unroll
                    for (int k = 0; k <= SG; ++k) ra = ra && tagged_tag(av[k]) == tagA;
                    if (__all(ra)) {
#pragma unroll
                        for (int k = 0; k < SG; ++k)
                            accS[k] = fmaf(accP, tagged_value(av[1 + k]), accS[k]);
                        accP *= tagged_value(av[0]);
                        --jx;
                        --left;
                        continue;
                    }
                    if (++spins > kSpinLimit) {
                        __hip_atomic_fetch_or(&hdr->error, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                        for (int k = 0; k < SG; ++k) xin[k] = 0.f;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            uint64_t *ic = incl + mg * (SG * 64);
            float xo[SG];
#pragma unroll
            for (int k = 0; k < SG; ++k) {
                xo[k] = fmaf(Pt, xin[k], St[k]);
                st_tagged(ic + k * 64 + lane, xo[k], tagI);
                sX[s0 + k][lane] = xin[k];
            }
            if (valid_lane && chunk == n_chunks - 1) {
                if (x_final) {
#pragma unroll
                    for (int k = 0; k < SG; ++k) x_final[(bi * Di + c_lane) * N + s0 + k] = xo[k];
                }
                if (BLOCK && wv == 0 && conv_state_out) {
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        const int64_t m = L - 3 + k;
                        bf16 v = 0;
                        if (m >= 0)
                            v = hu[(tokbase + m) * Di + c_lane];
                        else if (conv_state)
                            v = conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c_lane];
                        conv_state_out[((int64_t)bi * 3 + k) * Di + c_lane] = v;
                    }
                }
            }
        }
        __syncthreads();

        // --------------------- this wave's entering state, in the B-operand
        // layout (channel 2 col + j, states 8h..8h+7): the workgroup's entering
        // state carried through the waves before it
        float xs[2][8];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int chn = 2 * col + j;
#pragma unroll
            for (int k = 0; k < 8; ++k) xs[j][k] = sX[8 * hh + k][chn];
            for (int w = 0; w < wv; ++w) {
                const float pw = sP[w][chn];
#pragma unroll
                for (int k = 0; k < 8; ++k) xs[j][k] = fmaf(pw, xs[j][k], sS[w][8 * hh + k][chn]);
            }
        }
        if (ckpt && active) {
            float *cp = ckpt + (((int64_t)bi * n_waves + (int64_t)chunk * W + wv) * N) * Di + cbase;
            const rsrc_t rc = make_rsrc(cp, (uint32_t)(N * Di * 4));
            // channels 2 col and 2 col + 1 (both valid or neither: Di is even)
            const uint32_t vo = cbase + 2 * col < Di ? (uint32_t)((8 * hh) * Di + 2 * col) * 4 : kOOB;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const f32x2 v = {xs[0][k], xs[1][k]};
                // (nontemporal: read back only by the backward, much later)
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rc, vo,
                                                      (uint32_t)(k * Di) * 4, 2);
            }
        }

        if (!wave_ok) {
            if (y) {
                // the fallback works in lane = channel layout
                float xin[16];
#pragma unroll
                for (int s = 0; s < 16; ++s) xin[s] = sX[s][lane];
                for (int w = 0; w < wv; ++w) {
                    const float pw = sP[w][lane];
#pragma unroll
                    for (int s = 0; s < 16; ++s) xin[s] = fmaf(pw, xin[s], sS[w][s][lane]);
                }
                rr_output<BLOCK>(L, Di, bi, c_lane, valid_lane, n0, scale, hu, a, bg, Bm, Cm, D,
                                 z, conv_w, conv_state, xin, y);
            }
        } else if (y) {
            const int64_t ebase = (tokbase + (active ? n0 : 0)) * Di + cbase;
            const uint32_t row2 = (uint32_t)Di * 2;
            const rsrc_t ry = make_rsrc(y + ebase, (uint32_t)Lw * row2);
            const rsrc_t rz = make_rsrc(BLOCK ? (const void *)(z + ebase) : (const void *)y,
                                        BLOCK ? (uint32_t)Lw * row2 : 0u);
            // the lane's channel pair (2 col, 2 col + 1): both valid or neither (Di is even)
            const bool vc = cbase + 2 * col < Di;
            // z first, all at once: the y stores below may alias it as far as the
            // compiler can tell, so a load placed between them would wait out a
            // full round trip per element
            uint32_t zb[16];
            if (BLOCK) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t vo = vc ? (uint32_t)((4 * hh + r) * Di + 2 * col) * 2 : kOOB;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        zb[4 * q + r] =
                            __builtin_amdgcn_raw_buffer_load_b32(rz, vo, (uint32_t)(8 * q) * row2, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bf16x8 xh, xl;
                split8(xs[j], xh, xl);
                Y[j] = mfma(Csc, xh, Y[j]);
                Y[j] = mfma(Csc, xl, Y[j]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t vo = vc ? (uint32_t)((4 * hh + r) * Di + 2 * col) * 2 : kOOB;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = 4 * q + r;
                    const uint32_t so = (uint32_t)(8 * q) * row2;
                    f32x2 yv = {Pv[0][i] * Y[0][i], Pv[1][i] * Y[1][i]};
                    if (BLOCK) {
                        const float z0 = __uint_as_float(zb[i] << 16);
                        const float z1 = __uint_as_float(zb[i] & 0xffff0000u);
                        yv[0] *= z0 * sigm(z0);
                        yv[1] *= z1 * sigm(z1);
                    }
                    const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(yv, bf16x2));
                    __builtin_amdgcn_raw_buffer_store_b32(pk, ry, vo, so, 0);
                }
            }
        }
        cur = nxt;
    }
    // the last workgroup out advances the epoch (every workgroup has read it)
    if (threadIdx.x == 0) {
        const uint32_t old = add_agent(&hdr->done, 1u);
        if (old == gridDim.x - 1) {
            st_agent(&hdr->done, 0u);
            st_agent(&hdr->epoch, ep);
        }
    }
}

int device_cu_count()
{
    static int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        return v;
    }();
    return n;
}

hipError_t launch_fwd_mfma(const FwdArgs &g, hipStream_t stream)
{
    const FwdPlan pl = fwd_plan(g.Bt, g.L, g.Di, g.N, kMfmaW);
    WsHeader *hdr = (WsHeader *)g.ws;
    uint64_t *agg = (uint64_t *)((char *)g.ws + pl.off_agg);
    uint64_t *incl = (uint64_t *)((char *)g.ws + pl.off_incl);
    const int64_t slots = 2 * (int64_t)device_cu_count();  // two workgroups per CU
    const int64_t grid = pl.n_wg < slots ? pl.n_wg : slots;
    // lazy aggregates when a round of `grid` tickets spans at most ~4 chunks of a row
    const int lazy = (int64_t)g.Bt * pl.n_tiles * 4 >= grid ? 1 : 0;
    if (g.block)
        hipLaunchKernelGGL(fwd_mfma_kernel<true>, dim3(grid), dim3(64 * kMfmaW), 0, stream, g.Bt,
                           g.L, g.Di, pl.n_tiles, pl.n_chunks, g.scale, (const bf16 *)g.hu,
                           (const bf16 *)g.a, (const bf16 *)g.b, (const bf16 *)g.B,
                           (const bf16 *)g.C, g.D, g.x0, (const bf16 *)g.z, g.conv_w,
                           (const bf16 *)g.conv_state, (bf16 *)g.y, g.x_final,
                           (bf16 *)g.conv_state_out, g.ckpt, hdr, agg, incl, lazy);
    else
        hipLaunchKernelGGL(fwd_mfma_kernel<false>, dim3(grid), dim3(64 * kMfmaW), 0, stream,
                           g.Bt, g.L, g.Di, pl.n_tiles, pl.n_chunks, g.scale, (const bf16 *)g.hu,
                           (const bf16 *)g.a, (const bf16 *)g.b, (const bf16 *)g.B,
                           (const bf16 *)g.C, g.D, g.x0, (const bf16 *)g.z, g.conv_w,
                           (const bf16 *)g.conv_state, (bf16 *)g.y, g.x_final,
                           (bf16 *)g.conv_state_out, g.ckpt, hdr, agg, incl, lazy);
    return hipGetLastError();
}

}  // namespace naju

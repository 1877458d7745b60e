// naju_fwd.hip -- forward kernel of the Naju selective scan (scan and block).
//
// Recurrence and readout: "Core equations" of the Naju reproduction README
// (arXiv 2607.21000); block front end / output modulation: that page's block
// flowchart.  The sequence is cut into chunks; a chunk's effect on the state
// is the affine map x -> P x + S (P = prod f, S = state reached from zero),
// and composing these maps in order is exactly the sequential recurrence (the
// page's "Scope" section calls the sequential loop mathematically equivalent
// to the affine scan).
//
// Work decomposition (one launch):
//   workgroup = W waves; one wave = CPW channels x T consecutive tokens; the W
//   waves of a workgroup take W consecutive token chunks of the same channels.
//   Lanes: LPC = N/16 lanes per channel, each holding 16 fp32 states in VGPRs.
//   1. every wave runs the recurrence from a zero state over its T tokens,
//      keeping the local readout ys_loc[j] and the running product P_j;
//   2. the waves' (P, S) pairs are composed through LDS;
//   3. wave 0 publishes the workgroup aggregate, then obtains the state
//      entering the workgroup by decoupled look-back over its predecessors'
//      published aggregates / inclusive states (tickets are taken in launch
//      order, so every predecessor is already running and never waits on a
//      successor);
//   4. every wave adds the contribution of its entering state,
//        y_j = ys_loc[j] + P_j (x_in . C_j) / sqrt(N),
//      applies SiLU(z) for the block, and stores y.
#include <stdlib.h>

#include "naju_device.h"
#include "naju_launch.h"
#include "naju_mfma.h"

namespace naju {

// STG (bf16, d_state 64, d_inner % 8 == 0): each wave first copies its own
// 32 tokens of h|u, a, b (and z), B and C into a private LDS region with a few
// 16-byte-per-lane copies and one wait, instead of two dependent round trips
// to memory per token (the per-token loads of a lane are a handful of bytes).
template <typename IO, int N, bool BLOCK, int T, int W, bool STG = false>
__global__ __launch_bounds__(64 * W) void fwd_kernel(
    const int64_t Bt, const int64_t L, const int64_t Di, const int n_tiles, const int n_chunks,
    const float scale, const IO *__restrict__ hu, const IO *__restrict__ a,
    const IO *__restrict__ bg, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ x0, const IO *__restrict__ z,
    const float *__restrict__ conv_w, const IO *__restrict__ conv_state, IO *__restrict__ y,
    float *__restrict__ x_final, IO *__restrict__ conv_state_out, float *__restrict__ ckpt,
    WsHeader *hdr, uint32_t *flags, float *agg, float *incl)
{
    constexpr int LPC = N / 16;   // lanes per channel
    constexpr int CPW = 64 / LPC; // channels per wave
    const int lane = threadIdx.x & 63;
    // wave-uniform (readfirstlane keeps what derives from it, such as the staging
    // copies' buffer descriptors, in scalar registers)
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // per-wave staging (STG): [tok][16 ch] for h|u, a, b, z, then [tok][N] for B and C
    constexpr int kCh = 64 / LPC;
    constexpr int kStg = STG ? (4 * T * kCh + 2 * T * N) : 8;
    __shared__ __attribute__((aligned(16))) IO sStg[STG ? W : 1][kStg];
    // SBC (d_state 16 without STG): each wave's B and C rows, [tok][N] each, staged
    // once, so that the sequential token loop reads them from LDS instead of making
    // one round trip to memory per token
    constexpr bool SBC = !STG && N == 16;
    constexpr int kBC = SBC ? 2 * T * N : 1;
    __shared__ __attribute__((aligned(16))) IO sBCs[SBC ? W : 1][kBC];
    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ float sP[W][64];
    __shared__ float sS[W][16][64];
    __shared__ float sX[16][64];

    if (threadIdx.x == 0) {
        s_ticket = add_agent(&hdr->ticket, 1u);
        s_epoch = (ld_agent(&hdr->epoch) + 1u) & 0x3FFFFFFFu;
    }
    __syncthreads();
    const uint32_t ticket = s_ticket;
    const uint32_t ep = s_epoch;
    const uint32_t per_chunk = (uint32_t)(Bt * n_tiles);
    const int chunk = (int)(ticket / per_chunk);
    const int rem = (int)(ticket % per_chunk);
    const int bi = rem / n_tiles;
    const int tile = rem % n_tiles;

    const int sg = lane % LPC;
    const int64_t c = (int64_t)tile * CPW + lane / LPC;
    const bool valid = c < Di;
    const int64_t n0 = (int64_t)chunk * (W * T) + (int64_t)wv * T;
    const float Dc = valid ? D[c] : 0.f;
    IO *stg = sStg[STG ? wv : 0];
    if constexpr (STG) {
        static_assert(sizeof(IO) == 2 && N == 64 && T == 32, "staging layout");
        // [tok][16 ch] blocks: lane = (row lane/2, 8-channel half lane%2); the range
        // ends with the wave's last valid token (rows past it read 0)
        const int rows = n0 < L ? (int)(L - n0 < T ? L - n0 : T) : 0;
        const int64_t eb = ((int64_t)bi * L + (n0 < L ? n0 : 0)) * Di + (int64_t)tile * kCh;
        const uint32_t rng = (uint32_t)rows * (uint32_t)Di * 2 - (uint32_t)tile * kCh * 2;
        const uint32_t vo = ((uint32_t)(lane >> 1) * (uint32_t)Di + 8 * (lane & 1)) * 2;
        dma16b(make_rsrc(hu + eb, rows ? rng : 0u), vo, 0u, stg);
        dma16b(make_rsrc(a + eb, rows ? rng : 0u), vo, 0u, stg + T * kCh);
        dma16b(make_rsrc(bg + eb, rows ? rng : 0u), vo, 0u, stg + 2 * T * kCh);
        if (BLOCK) dma16b(make_rsrc(z + eb, rows ? rng : 0u), vo, 0u, stg + 3 * T * kCh);
        // B, C rows: [tok][N], 8 rows per copy (lane = row lane/8, chunk lane%8)
        const int64_t tb = ((int64_t)bi * L + (n0 < L ? n0 : 0)) * N;
        const uint32_t vb = ((uint32_t)(lane >> 3) * N + 8 * (lane & 7)) * 2;
        const rsrc_t rB = make_rsrc(Bm + tb, (uint32_t)rows * N * 2);
        const rsrc_t rC = make_rsrc(Cm + tb, (uint32_t)rows * N * 2);
#pragma unroll
        for (int k = 0; k < T / 8; ++k) {
            dma16b(rB, vb, (uint32_t)(8 * k * N * 2), stg + 4 * T * kCh + 8 * k * N);
            dma16b(rC, vb, (uint32_t)(8 * k * N * 2), stg + 4 * T * kCh + T * N + 8 * k * N);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (SBC) {
        // 16 bytes per lane and instruction through a buffer whose range ends with the
        // wave's last valid token (rows past it read 0)
        static_assert(T * N * sizeof(IO) % 1024 == 0, "staging layout");
        constexpr int kPer = T * N * (int)sizeof(IO) / 1024;
        const int rows = n0 < L ? (int)(L - n0 < T ? L - n0 : T) : 0;
        const int64_t tb = ((int64_t)bi * L + (n0 < L ? n0 : 0)) * N;
        const uint32_t bytes = (uint32_t)rows * N * (uint32_t)sizeof(IO);
        const rsrc_t rB = make_rsrc(Bm + tb, bytes), rC = make_rsrc(Cm + tb, bytes);
        uint4 vb[kPer], vc[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            vb[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rB, (uint32_t)(16 * lane + 1024 * k), 0, 0));
            vc[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rC, (uint32_t)(16 * lane + 1024 * k), 0, 0));
        }
        uint4 *dst = (uint4 *)&sBCs[wv][0];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            dst[lane + 64 * k] = vb[k];
            dst[T * N * (int)sizeof(IO) / 16 + lane + 64 * k] = vc[k];
        }
        __syncthreads();
    }
    const int cl = lane / LPC;  // this lane's channel inside the tile

    // ---------------------------------------------------------- block front end
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, um1 = 0.f, um2 = 0.f, um3 = 0.f;
    if constexpr (BLOCK) {
        if (valid) {
            w0 = conv_w[c * 4 + 0];
            w1 = conv_w[c * 4 + 1];
            w2 = conv_w[c * 4 + 2];
            w3 = conv_w[c * 4 + 3];
            float halo[3];
#pragma unroll
            for (int k = 1; k <= 3; ++k) {
                const int64_t m = n0 - k;
                float v = 0.f;
                if (m >= 0 && m < L)
                    v = to_f(hu[((int64_t)bi * L + m) * Di + c]);
                else if (m < 0 && conv_state)
                    v = to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
                halo[k - 1] = v;
            }
            um1 = halo[0];
            um2 = halo[1];
            um3 = halo[2];
        }
    }

    // ------------------------------------------------------ 1. local recurrence
    float x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = 0.f;
    float P = 1.f;
    float ysl[T], Pn[T];
    // Without staging, the per-token activations of each group of 8 tokens are
    // loaded together: one round trip per group instead of one per token.  The
    // loads are unconditional (rows past L and lanes past Di read element 0 and
    // the value is dropped), so none waits inside a branch of its own.
    constexpr int G = 8;
    float ga[G], gb[G], gh[G];
#pragma unroll
    for (int j = 0; j < T; ++j) {
        const int64_t n = n0 + j;
        if (!STG && j % G == 0) {
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const int64_t nk = n0 + j + k;
                const bool ok = valid && nk < L;
                const int64_t tk = ok ? ((int64_t)bi * L + nk) * Di + c : 0;
                const float va = to_f(a[tk]), vb = to_f(bg[tk]), vh = to_f(hu[tk]);
                ga[k] = ok ? va : 0.f;
                gb[k] = ok ? vb : 0.f;
                gh[k] = ok ? vh : 0.f;
            }
        }
        ysl[j] = 0.f;
        Pn[j] = P;
        if (n < L) {
            float av = 0.f, bv = 0.f, hv = 0.f;
            if (valid) {
                av = STG ? to_f(stg[T * kCh + j * kCh + cl]) : ga[j % G];
                bv = STG ? to_f(stg[2 * T * kCh + j * kCh + cl]) : gb[j % G];
                if constexpr (BLOCK) {
                    const float uv = STG ? to_f(stg[j * kCh + cl]) : gh[j % G];
                    const float pre = w0 * um3 + w1 * um2 + w2 * um1 + w3 * uv;
                    um3 = um2;
                    um2 = um1;
                    um1 = uv;
                    hv = pre * sigm(pre);
                } else {
                    hv = STG ? to_f(stg[j * kCh + cl]) : gh[j % G];
                }
            }
            const float f = sigm(av);
            const float wr = sigm(bv) * hv;
            const IO *Bn = STG   ? stg + 4 * T * kCh + j * N + sg * 16
                           : SBC ? &sBCs[wv][j * N]
                                 : Bm + ((int64_t)bi * L + n) * N + sg * 16;
            const IO *Cn = STG   ? stg + 4 * T * kCh + T * N + j * N + sg * 16
                           : SBC ? &sBCs[wv][T * N + j * N]
                                 : Cm + ((int64_t)bi * L + n) * N + sg * 16;
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                x[s] = fmaf(f, x[s], wr * to_f(Bn[s]));
                acc = fmaf(x[s], to_f(Cn[s]), acc);
            }
            if constexpr (LPC > 1) acc = quad_sum(acc);  // the channel's 4 lanes
            P *= f;
            ysl[j] = fmaf(scale, acc, Dc * hv);
            Pn[j] = P;
        }
    }

    // ------------------------------------------ 2. compose the waves' pairs
    sP[wv][lane] = P;
#pragma unroll
    for (int s = 0; s < 16; ++s) sS[wv][s][lane] = x[s];
    __syncthreads();

    // exclusive prefix of this wave inside the workgroup: x_w = Pe x_wg + Se
    float Pe = 1.f, Se[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) Se[s] = 0.f;
    for (int w = 0; w < wv; ++w) {
        const float pw = sP[w][lane];
#pragma unroll
        for (int s = 0; s < 16; ++s) Se[s] = fmaf(pw, Se[s], sS[w][s][lane]);
        Pe *= pw;
    }

    // ------------------------------------- 3. look-back for the entering state
    if (wv == 0) {
        // workgroup aggregate (all W waves)
        float Pt = 1.f, St[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) St[s] = 0.f;
        for (int w = 0; w < W; ++w) {
            const float pw = sP[w][lane];
#pragma unroll
            for (int s = 0; s < 16; ++s) St[s] = fmaf(pw, St[s], sS[w][s][lane]);
            Pt *= pw;
        }
        const size_t me = ((size_t)bi * n_tiles + tile) * n_chunks + chunk;
        float xin[16];
        if (chunk == 0) {
#pragma unroll
            for (int s = 0; s < 16; ++s)
                xin[s] = (x0 && valid) ? x0[(bi * Di + c) * N + sg * 16 + s] : 0.f;
        } else {
            float *ag = agg + me * (17 * 64);
            st_agent(ag + lane, Pt);
#pragma unroll
            for (int s = 0; s < 16; ++s) st_agent(ag + (1 + s) * 64 + lane, St[s]);
            wait_mem();
            if (lane == 0) st_agent(&flags[me], make_flag(ep, kFlagAgg));
            float accP = 1.f, accS[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) accS[s] = 0.f;
            size_t j = me - 1;
            for (;;) {
                const uint32_t st = wait_flag(&flags[j], ep, hdr);
                if (st == kFlagIncl) {
                    const float *in = incl + j * (16 * 64);
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        xin[s] = fmaf(accP, ld_agent(in + s * 64 + lane), accS[s]);
                    break;
                }
                const float *pa = agg + j * (17 * 64);
                const float pj = ld_agent(pa + lane);
#pragma unroll
                for (int s = 0; s < 16; ++s) accS[s] = fmaf(accP, ld_agent(pa + (1 + s) * 64 + lane), accS[s]);
                accP *= pj;
                --j;  // chunk 0 always publishes an inclusive state, so j stays >= first
            }
        }
        float *ic = incl + me * (16 * 64);
        float xo[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            xo[s] = fmaf(Pt, xin[s], St[s]);
            st_agent(ic + s * 64 + lane, xo[s]);
        }
        wait_mem();
        if (lane == 0) st_agent(&flags[me], make_flag(ep, kFlagIncl));
#pragma unroll
        for (int s = 0; s < 16; ++s) sX[s][lane] = xin[s];
        if (valid) {
            if (chunk == n_chunks - 1 && x_final) {
#pragma unroll
                for (int s = 0; s < 16; ++s) x_final[(bi * Di + c) * N + sg * 16 + s] = xo[s];
            }
            if constexpr (BLOCK) {
                if (chunk == n_chunks - 1 && conv_state_out && sg == 0) {
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        const int64_t m = L - 3 + k;
                        IO v = from_f<IO>(0.f);
                        if (m >= 0)
                            v = hu[((int64_t)bi * L + m) * Di + c];
                        else if (conv_state)
                            v = conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c];
                        conv_state_out[((int64_t)bi * 3 + k) * Di + c] = v;
                    }
                }
            }
        }
    }
    __syncthreads();

    // ------------------------------------------ 4. correction, modulation, store
    float xin[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) xin[s] = fmaf(Pe, sX[s][lane], Se[s]);
    // checkpoint: the state entering this wave's T tokens
    if (ckpt && valid && n0 < L) {
        const int64_t wrow = (int64_t)chunk * W + wv;
        const int64_t n_waves = (L + T - 1) / T;
#pragma unroll
        for (int s = 0; s < 16; ++s)
            ckpt[(((int64_t)bi * n_waves + wrow) * N + sg * 16 + s) * Di + c] = xin[s];
    }
    if (y) {
#pragma unroll
        for (int j = 0; j < T; ++j) {
            const int64_t n = n0 + j;
            if (n < L) {
                const IO *Cn = STG   ? stg + 4 * T * kCh + T * N + j * N + sg * 16
                               : SBC ? &sBCs[wv][T * N + j * N]
                                     : Cm + ((int64_t)bi * L + n) * N + sg * 16;
                float dot = 0.f;
#pragma unroll
                for (int s = 0; s < 16; ++s) dot = fmaf(xin[s], to_f(Cn[s]), dot);
                if constexpr (LPC > 1) dot = quad_sum(dot);
                float yv = fmaf(scale * Pn[j], dot, ysl[j]);
                const int64_t t = ((int64_t)bi * L + n) * Di + c;
                if (valid && sg == 0) {
                    if constexpr (BLOCK) {
                        const float zv = to_f(STG ? stg[3 * T * kCh + j * kCh + cl] : z[t]);
                        yv *= zv * sigm(zv);
                    }
                    y[t] = from_f<IO>(yv);
                }
            }
        }
    }

    // ------------------------------------------------ release the workspace
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

// ---------------------------------------------------------------- launcher
template <typename IO, int N, bool BLOCK, bool STG = false>
static hipError_t launch_fwd_t(const FwdArgs &g, hipStream_t stream)
{
    constexpr int T = kFwdT, W = kFwdW;
    const FwdPlan pl = fwd_plan(g.Bt, g.L, g.Di, g.N);
    WsHeader *hdr = (WsHeader *)g.ws;
    uint32_t *flags = (uint32_t *)((char *)g.ws + pl.off_flags);
    float *agg = (float *)((char *)g.ws + pl.off_agg);
    float *incl = (float *)((char *)g.ws + pl.off_incl);
    hipLaunchKernelGGL((fwd_kernel<IO, N, BLOCK, T, W, STG>), dim3(pl.n_wg), dim3(64 * W), 0, stream,
                       g.Bt, g.L, g.Di, pl.n_tiles, pl.n_chunks, g.scale, (const IO *)g.hu,
                       (const IO *)g.a, (const IO *)g.b, (const IO *)g.B, (const IO *)g.C, g.D,
                       g.x0, (const IO *)g.z, g.conv_w, (const IO *)g.conv_state, (IO *)g.y,
                       g.x_final, (IO *)g.conv_state_out, g.ckpt, hdr, flags, agg, incl);
    return hipGetLastError();
}

// The matrix-core variants serve bf16 activations (d_state 16; d_state 64 when
// its rows fill the device) when the operands allow 16-byte loads;
// NAJU_FWD_VARIANT=rr forces the register recurrence.
static bool forced_rr()
{
    static const bool v = [] {
        const char *e = getenv("NAJU_FWD_VARIANT");
        return e && e[0] == 'r' && e[1] == 'r';
    }();
    return v;
}

static bool use_mfma(const FwdArgs &g)
{
    const auto al16 = [](const void *p) { return ((uintptr_t)p % 16) == 0; };
    // (buffer ranges of 32 token rows / 16 checkpoint rows stay below 2^31 bytes)
    const auto al = [](const void *p, unsigned n) { return ((uintptr_t)p % n) == 0; };
    // (y and z are accessed as channel pairs, the checkpoints as float pairs)
    return !forced_rr() && g.io == 1 && g.N == 16 && g.Di % 8 == 0 && g.Di < ((int64_t)1 << 24) &&
           al16(g.B) && al16(g.C) && al16(g.hu) && al16(g.a) && al16(g.b) && al(g.y, 4) &&
           al(g.z, 4) && al(g.ckpt, 8);
}

hipError_t launch_fwd(const FwdArgs &g, hipStream_t stream)
{
    if (use_mfma(g)) return launch_fwd_mfma(g, stream);
    if (g.io == 0) {
        if (g.N == 16) return g.block ? launch_fwd_t<float, 16, true>(g, stream)
                                      : launch_fwd_t<float, 16, false>(g, stream);
        return g.block ? launch_fwd_t<float, 64, true>(g, stream)
                       : launch_fwd_t<float, 64, false>(g, stream);
    }
    if (g.N == 16) return g.block ? launch_fwd_t<bf16, 16, true>(g, stream)
                                  : launch_fwd_t<bf16, 16, false>(g, stream);
    if (!forced_rr() && use_fwd_mfma64(g)) return launch_fwd_mfma64(g, stream);
    const bool stg = g.Di % 8 == 0 && g.Di < ((int64_t)1 << 24) && ((uintptr_t)g.B % 16) == 0 &&
                     ((uintptr_t)g.C % 16) == 0;
    if (stg)
        return g.block ? launch_fwd_t<bf16, 64, true, true>(g, stream)
                       : launch_fwd_t<bf16, 64, false, true>(g, stream);
    return g.block ? launch_fwd_t<bf16, 64, true>(g, stream)
                   : launch_fwd_t<bf16, 64, false>(g, stream);
}

}  // namespace naju

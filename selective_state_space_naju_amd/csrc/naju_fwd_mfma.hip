// naju_fwd_mfma.hip -- matrix-core forward of the Naju selective scan for bf16
// activations and d_state 16 (scan and block).
//
// The recurrence and readout of the "Core equations" section of the Naju
// reproduction README (arXiv 2607.21000): per channel, x_n = f_n x_{n-1} +
// i_n h_n B_n^T with f = sigma(a), i = sigma(b), and y_n = x_n C_n / sqrt(N) +
// D h_n; the block (the README's flowchart) takes h = SiLU(causal depthwise
// conv4(u)) and returns y SiLU(z).  The README's "Scope" section notes that the
// sequential loop is an affine scan; it is computed here as one:
//
//   * inside a wave's 32-token chunk, with the chunk-local running product
//     P_n = prod_{j<=n} f_j, a pivot p (token 16) and the rescaled writes
//     W'_k = w_k P_p / P_k,
//         x_n = (P_n / P_p) (P_p x_in + sum_{k<=n} W'_k B_k)
//         y_n = (P_n / P_p) ( sum_{k<=n} G[n,k] W'_k + C_n P_p x_in / sqrt(N) ) + D h_n
//     with G = tril(C B^T) / sqrt(N) shared by every channel: G @ W', the
//     chunk's state increment B^T W' and C @ x_in run on the matrix cores
//     (v_mfma_f32_32x32x16_bf16, operands split into bf16 hi + lo parts so the
//     products keep close to fp32 accuracy);
//   * the four waves of a workgroup's 128-token chunk are composed as affine
//     pairs (P, S) in LDS, and workgroup chunks by a decoupled look-back over
//     tagged words in the workspace.
//
// Decomposition: a workgroup of four waves owns 128 tokens x 64 channels; wave
// w owns tokens 32 w .. 32 w + 31.  Lane l holds column l % 32 of the two
// 32-wide MFMA column tiles -- the adjacent channels 2 (l % 32) and
// 2 (l % 32) + 1, so a lane's y, z and checkpoint values of a token are one 4-
// or 8-byte access -- and, in its half h = l / 32, the 16 tokens {8q + 4h + r}:
// that set is both its row set in the 32x32 accumulator and (by the K-slot
// order) its K-slots in the operands, so the gates, W', P and the outputs of a
// token stay in the lane that needs them.
//
// Scheduling: persistent workgroups, as many as fit (two per CU), walk tickets
// (chunk-major, so a chunk's look-back predecessors hold smaller tickets),
// knowing each next ticket one ahead so that its tile copy starts during the
// current ticket.  By default workgroup w takes tickets w, w + G, ...: every
// predecessor is then held by a workgroup of the same grid, which the launch
// sizes to what the device holds at once; if some workgroups could not become
// resident (other work occupying the device), a wait would end at its spin
// bound with the workspace's error bit set, never hang.  The alternative
// schedule takes tickets from per-XCD queues in the order workgroups run
// (a predecessor is then always held by a running or finished workgroup, so
// every wait ends by construction), at some cost in speed.  Waves 2 and 3 copy
// the tiles (HBM -> LDS, 16 bytes per lane, no registers involved); waves 0
// and 1 run the look-back, so their polls never queue behind a copy.
//
// Safety: the factorisation needs the decay ratios to stay in range (the Muir
// page warns that unpivoted chunked decay factorisations overflow, and pivots
// at a chunk point): with the pivot in the middle, P_p / P_k and P_n / P_p each
// span at most 16 tokens.  A wave whose half-chunk has prod(1/f) > 2^96 or a
// non-finite or extreme input computes that chunk with the plain register
// recurrence instead (exact for any input).
#include <type_traits>

#include "naju_device.h"
#include "naju_launch.h"
#include "naju_mfma.h"

namespace naju {

namespace {

constexpr int kT = 32;        // tokens per wave
constexpr int kW = 4;         // waves per workgroup chunk
constexpr int kRows = 128;    // tokens per workgroup chunk
constexpr int kHalo = 8;      // rows of u kept before the chunk (block)

// ------------------------------------------------------------------ fallback
// Register recurrence of one wave's chunk in lane = channel layout (64
// channels, 16 states per lane).  The pointers slide one token per step and the
// block's conv window slides in registers.
struct RrCursor {
    const bf16 *h, *a, *b;  // the lane's channel at the current token
    float u1, u2, u3;       // block: u at the three tokens before
    float cw[4];
};

template <bool BLOCK>
__device__ __forceinline__ void rr_start(RrCursor &k, int64_t L, int64_t Di, int bi, int64_t c,
                                         int64_t n0, const bf16 *hu, const bf16 *a,
                                         const bf16 *bg, const float *conv_w,
                                         const bf16 *conv_state)
{
    const int64_t t = ((int64_t)bi * L + n0) * Di + c;
    k.h = hu + t;
    k.a = a + t;
    k.b = bg + t;
    k.u1 = k.u2 = k.u3 = 0.f;
    if (BLOCK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) k.cw[j] = conv_w[c * 4 + j];
        float w[3];
#pragma unroll
        for (int j = 1; j <= 3; ++j) {
            const int64_t m = n0 - j;
            float v = 0.f;
            if (m >= 0)
                v = to_f(k.h[-j * Di]);
            else if (conv_state)
                v = to_f(conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c]);
            w[j - 1] = v;
        }
        k.u1 = w[0], k.u2 = w[1], k.u3 = w[2];
    }
}

// gates and the write of the cursor's token; advances the cursor
template <bool BLOCK>
__device__ __forceinline__ void rr_step(RrCursor &k, int64_t Di, float &f, float &w, float &h)
{
    if (BLOCK) {
        const float uv = to_f(*k.h);
        const float pre = k.cw[0] * k.u3 + k.cw[1] * k.u2 + k.cw[2] * k.u1 + k.cw[3] * uv;
        k.u3 = k.u2;
        k.u2 = k.u1;
        k.u1 = uv;
        h = pre * sigm(pre);
    } else {
        h = to_f(*k.h);
    }
    f = sigm(to_f(*k.a));
    w = sigm(to_f(*k.b)) * h;
    k.h += Di;
    k.a += Di;
    k.b += Di;
}

// aggregate of the chunk from a zero state: x -> P x + S
template <bool BLOCK>
__device__ void rr_aggregate(int64_t L, int64_t Di, int bi, int64_t c, bool valid, int64_t n0,
                             const bf16 *hu, const bf16 *a, const bf16 *bg, const bf16 *Bm,
                             const float *conv_w, const bf16 *conv_state, float &P,
                             float (&S)[16])
{
    P = 1.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) S[s] = 0.f;
    if (!valid) return;  // a channel past Di: P = 1, S = 0
    RrCursor k;
    rr_start<BLOCK>(k, L, Di, bi, c, n0, hu, a, bg, conv_w, conv_state);
    const int64_t n1 = n0 + kT < L ? n0 + kT : L;
    const bf16 *Bn = Bm + ((int64_t)bi * L + n0) * 16;
#pragma unroll 1
    for (int64_t n = n0; n < n1; ++n, Bn += 16) {
        float f, w, h;
        rr_step<BLOCK>(k, Di, f, w, h);
#pragma unroll
        for (int s = 0; s < 16; ++s) S[s] = fmaf(f, S[s], w * to_f(Bn[s]));
        P *= f;
    }
}

// the chunk's outputs from its entering state
template <bool BLOCK>
__device__ void rr_output(int64_t L, int64_t Di, int bi, int64_t c, bool valid, int64_t n0,
                          float scale, const bf16 *hu, const bf16 *a, const bf16 *bg,
                          const bf16 *Bm, const bf16 *Cm, const float *D, const bf16 *z,
                          const float *conv_w, const bf16 *conv_state, const float (&xin)[16],
                          bf16 *y)
{
    if (!valid) return;
    RrCursor k;
    rr_start<BLOCK>(k, L, Di, bi, c, n0, hu, a, bg, conv_w, conv_state);
    const float Dc = D[c];
    float x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = xin[s];
    const int64_t n1 = n0 + kT < L ? n0 + kT : L;
    const int64_t t0 = ((int64_t)bi * L + n0) * Di + c;
    const bf16 *Bn = Bm + ((int64_t)bi * L + n0) * 16;
    const bf16 *Cn = Cm + ((int64_t)bi * L + n0) * 16;
#pragma unroll 1
    for (int64_t n = n0; n < n1; ++n, Bn += 16, Cn += 16) {
        float f, w, hv;
        rr_step<BLOCK>(k, Di, f, w, hv);
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            x[s] = fmaf(f, x[s], w * to_f(Bn[s]));
            acc = fmaf(x[s], to_f(Cn[s]), acc);
        }
        float yv = fmaf(scale, acc, Dc * hv);
        const int64_t t = t0 + (n - n0) * Di;
        if (BLOCK) {
            const float zv = to_f(z[t]);
            yv *= zv * sigm(zv);
        }
        y[t] = from_f<bf16>(yv);
    }
}

// s_waitcnt with a compile-time vector-memory count (the tile copies are issued
// through inline assembly, so the compiler's own counting does not see them)
template <int K> __device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

}  // namespace

// ------------------------------------------------------------------- kernel
template <bool BLOCK>
__global__ __launch_bounds__(64 * kW, 2) void fwd_chunk_kernel(
    const int64_t L, const int64_t Di, const FastDiv fd_chunk, const FastDiv fd_tiles,
    const uint32_t total, const TicketQueues tq, const int n_chunks, const float scale,
    const bf16 *__restrict__ hu,
    const bf16 *__restrict__ a, const bf16 *__restrict__ bg, const bf16 *__restrict__ Bm,
    const bf16 *__restrict__ Cm, const float *__restrict__ D, const float *__restrict__ x0,
    const bf16 *__restrict__ z, const float *__restrict__ conv_w,
    const bf16 *__restrict__ conv_state, bf16 *__restrict__ y, float *__restrict__ x_final,
    bf16 *__restrict__ conv_state_out, float *__restrict__ ckpt, WsHeader *hdr, uint64_t *agg,
    uint64_t *incl, const int lazy_agg, const int dyn)
{
    constexpr int N = 16, T = kT, H = BLOCK ? kHalo : 0;
    // Scan: each wave reads the second column tile's h, a, b into registers
    // (two tokens per register) before the first tile's gates, so the next
    // ticket's copy can start halfway through the gate arithmetic instead of
    // after it.  The block's conv window would need twice the registers, so it
    // releases the tile after its gates.
    constexpr bool EARLY = !BLOCK;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    __shared__ __attribute__((aligned(16))) bf16 sU[H + kRows][64];  // h (scan) or u (block)
    __shared__ __attribute__((aligned(16))) bf16 sAB[2][kRows][64];  // a, b
    __shared__ __attribute__((aligned(16))) bf16 sBC[2][kRows][16];  // B, C rows
    __shared__ __attribute__((aligned(16))) float sD[64];            // D of the tile
    __shared__ __attribute__((aligned(16))) float sCW[BLOCK ? 64 : 1][4];  // conv taps
    __shared__ float sP[kW][64];
    __shared__ float sS[kW][16][64];
    __shared__ float sX[16][64];
    __shared__ uint32_t s_tk[2];
    __shared__ uint32_t s_epoch;

    const uint32_t n_tiles = fd_tiles.d;
    const int64_t n_waves = (L + T - 1) / T;

    // Copy the h|u, a, b tile, the B, C rows, D and the conv taps of ticket tk
    // into LDS (waves 2 and 3: token rows 64 (w-2) .. +63 each; wave 2 also the
    // B rows and the 8 rows of u before the chunk, wave 3 the C rows, D and the
    // taps).  Rows past L read zeros; channels past Di of a row read the next
    // row's first channels, which no output uses.  The tile copies carry the
    // nontemporal hint (every byte is used once); the B, C rows do not (every
    // channel tile of the batch row reads them).
    auto prefetch = [&](uint32_t tk, int lane) {
        const uint32_t chk = fdiv(tk, fd_chunk);
        const uint32_t rm = tk - chk * fd_chunk.d;
        const uint32_t b_ = fdiv(rm, fd_tiles);
        const int64_t cb = (int64_t)(rm - b_ * n_tiles) * 64;
        const int r0 = 64 * (wv - 2);
        const int64_t n_0 = (int64_t)chk * kRows;
        const int rows = (int)(L - n_0 < kRows ? L - n_0 : kRows);
        const uint32_t rowb = (uint32_t)Di * 2;
        const int64_t base = ((int64_t)b_ * L + n_0) * Di + cb;  // the tile's first element
        const uint32_t range = (uint32_t)rows * rowb - (uint32_t)cb * 2;
        const uint32_t vo = ((uint32_t)(r0 + (lane >> 3)) * (uint32_t)Di + 8 * (lane & 7)) * 2;
        const rsrc_t rh = make_rsrc(hu + base, range);
        const rsrc_t ra = make_rsrc(a + base, range);
        const rsrc_t rb = make_rsrc(bg + base, range);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t so = (uint32_t)(8 * k) * rowb;
            dma16b(rh, vo, so, &sU[H + r0 + 8 * k][0]);
            dma16b(ra, vo, so, &sAB[0][r0 + 8 * k][0]);
            dma16b(rb, vo, so, &sAB[1][r0 + 8 * k][0]);
        }
        // B rows (wave 2) or C rows (wave 3): lane = row lane / 2 of a 32-row group
        const uint32_t vb = (uint32_t)((lane >> 1) * N + 8 * (lane & 1)) * 2;
        const rsrc_t rs = make_rsrc((wv == 2 ? Bm : Cm) + ((int64_t)b_ * L + n_0) * N,
                                    (uint32_t)rows * (N * 2));
#pragma unroll
        for (int k = 0; k < 4; ++k)
            dma16b<false>(rs, vb, (uint32_t)(32 * k * N * 2), &sBC[wv - 2][32 * k][0]);
        if (wv == 2) {
            if (BLOCK) {
                // rows n0-8 .. n0-1 of u (the first chunk's come from conv_state later)
                const rsrc_t rp = make_rsrc(hu + (chk > 0 ? base - 8 * Di : base),
                                            chk > 0 ? 8u * rowb - (uint32_t)cb * 2 : 0u);
                const uint32_t vh = ((uint32_t)(lane >> 3) * (uint32_t)Di + 8 * (lane & 7)) * 2;
                dma16b(rp, vh, 0u, &sU[0][0]);
            }
        } else {
            // D of the tile's 64 channels (lanes 0..15) and, for the block, the
            // conv taps (16 bytes: the 4 taps of channel lane)
            const uint32_t dr = (uint32_t)(Di - cb < 64 ? Di - cb : 64);
            if (lane < 16) dma16b<false>(make_rsrc(D + cb, dr * 4), 16u * lane, 0u, &sD[0]);
            if (BLOCK)
                dma16b<false>(make_rsrc(conv_w + cb * 4, dr * 16), 16u * lane, 0u, &sCW[0][0]);
        }
    };

    // Tickets: dyn = 1 takes them from this XCD's queue (workgroups are
    // dispatched round-robin over the 8 XCDs, so blockIdx % 8 names it; the
    // mapping only decides locality, never correctness), one ahead: the next
    // is requested at the start of a ticket and known at its release, when the
    // next tile's copy is issued.  dyn = 2 takes them from one queue in their
    // own order.  dyn = 0 assigns them statically (w, w + G, ...).
    const uint32_t qx = blockIdx.x & 7;
    // the k-th ticket of queue qx (total when the queue is exhausted)
    auto ticket_of = [&](uint32_t k) -> uint32_t {
        if (k >= tq.total[qx]) return total;
        const uint32_t chk = fdiv(k, tq.rows[qx]);
        const uint32_t row = qx + 8 * (k - chk * tq.rows[qx].d);
        return chk * fd_chunk.d + row;
    };
    // dyn = 2: one queue for the whole grid, handing out tickets in their own
    // (chunk-major) order
    uint32_t *const qc = dyn == 2 ? &hdr->queue[0] : &hdr->queue[qx];
    auto tk_of = [&](uint32_t k) -> uint32_t {
        return dyn == 2 ? (k < total ? k : total) : ticket_of(k);
    };
    if (threadIdx.x == 0) {
        s_epoch = (ld_agent(&hdr->epoch) + 1u) & 0x3FFFFFFFu;
        if (dyn) {
            s_tk[0] = tk_of(add_agent(qc, 1u));
        } else {
            s_tk[0] = blockIdx.x;
            s_tk[1] = blockIdx.x + gridDim.x;
        }
    }
    __syncthreads();
    const uint32_t ep = s_epoch;
    uint32_t cur = s_tk[0];
    if (cur < total && wv >= 2) prefetch(cur, threadIdx.x & 63);
    // VMEM operations this wave issued after its last tile copy that are known
    // to be younger than it (the y and checkpoint stores of a matrix-core
    // ticket): waiting until that many are outstanding waits for the copy only
    int after = 0;

    // (dyn) the queue position requested at this ticket's start by the first lane
    // of wave 2, a copy wave
    uint32_t k_req = 0;
    while (cur < total) {
        if (wv >= 2) {
            if (after == 24)
                wait_vm<24>();
            else if (after == 16)
                wait_vm<16>();
            else
                wait_mem();
        }
        // (dyn) the next ticket is requested now and read just before the release
        // barrier, half a ticket later: reading the counter's reply waits for every
        // memory operation the wave issued before it, and by then the previous
        // ticket's output stores have drained (read here, the wait would put their
        // round trip into every ticket)
        if (dyn && threadIdx.x == 128) k_req = add_agent(qc, 1u);
        __syncthreads();  // the tile of `cur` is in LDS
        // Wave priorities (among the waves of the SIMD, i.e. against the other
        // workgroup): 1 from the tile's arrival to its release, so that the next
        // copy starts early; 2 for the look-back walk, which the whole workgroup
        // waits for; 1 for the outputs, which end the ticket; 0 in between (the
        // second column tile's gates and the aggregate, which the other workgroup's
        // critical phases may overtake).
        __builtin_amdgcn_s_setprio(1);

        // lane-dependent values are re-derived every ticket (kept out of
        // loop-invariant code motion, which would pin per-lane addresses in
        // registers across the whole loop)
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int col = lane & 31;
        const int hh = lane >> 5;
        const bool upper = hh != 0;

        const uint32_t chunk = fdiv(cur, fd_chunk);
        const uint32_t rem = cur - chunk * fd_chunk.d;
        const uint32_t bi = fdiv(rem, fd_tiles);
        const uint32_t tile = rem - bi * n_tiles;
        const int64_t cbase = (int64_t)tile * 64;
        const int64_t n0 = (int64_t)chunk * kRows + (int64_t)wv * T;
        const int64_t tokbase = (int64_t)bi * L;
        const bool active = n0 < L;
        const int Lw = active ? (int)(L - n0 < T ? L - n0 : T) : 0;  // valid tokens of the wave
        // the lane's channel pair (2 col, 2 col + 1): both valid or neither (Di is even)
        const bool vc = cbase + 2 * col < Di;
        auto tok = [&](int i) -> int { return 8 * (i >> 2) + 4 * hh + (i & 3); };

        // y / z offsets of slot i: the lane offset of row 4h + r, plus group q's
        // row offset (the buffers' range, Lw rows, drops rows past the wave's last
        // token; kOOB drops channels past Di)
        const int64_t ebase = (tokbase + (active ? n0 : 0)) * Di + cbase;
        const uint32_t row2 = (uint32_t)Di * 2;
        uint32_t vo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) vo[r] = vc ? (uint32_t)((4 * hh + r) * Di + 2 * col) * 2 : kOOB;
        auto eoff = [&](int i) -> uint32_t { return vo[i & 3] + (uint32_t)(8 * (i >> 2)) * row2; };
        // z (block): loaded now and consumed before the next tile copy is issued
        // (a wait for a load issued after the copy would also wait for the copy)
        uint32_t zb[BLOCK ? 16 : 1];
        if (BLOCK && y) {
            const rsrc_t rz = make_rsrc(z + ebase, (uint32_t)Lw * row2);
#pragma unroll
            for (int i = 0; i < 16; ++i) zb[i] = __builtin_amdgcn_raw_buffer_load_b32(rz, eoff(i), 0, 0);
        }
        float Dn[2], cw[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            Dn[j] = sD[2 * col + j];
            if (BLOCK) {
                const float4 w4 = *(const float4 *)&sCW[2 * col + j][0];
                cw[j][0] = w4.x, cw[j][1] = w4.y, cw[j][2] = w4.z, cw[j][3] = w4.w;
            }
        }
        if (BLOCK && chunk == 0) {
            // the conv window before the sequence start: the carried conv state or zeros
            if (threadIdx.x < 3 * 64) {
                const int r = threadIdx.x >> 6, chn = threadIdx.x & 63;
                const int64_t cg = cbase + chn;
                sU[H - 3 + r][chn] = (conv_state && cg < Di)
                                         ? conv_state[((int64_t)bi * 3 + r) * Di + cg]
                                         : (bf16)0;
            }
            __syncthreads();
        }

        // ------------------------------------------------ token-shared operands
        // Bop / Cop: rows (token col of the wave, states 8h .. 8h+7); Bsv: the
        // transposed B (state col, K-slots tok(i)).  Rows past L are zero in LDS
        // (the copy reads zeros there), and B's rows 16..31 of the transposed
        // operand only reach accumulator rows no lane reads, so no masks.
        bf16x8 Bop, Cop, Bsv[2];
        {
            const int rr = 32 * wv + col;
            Bop = __builtin_bit_cast(bf16x8, *(const uint4 *)&sBC[0][rr][8 * hh]);
            Cop = __builtin_bit_cast(bf16x8, *(const uint4 *)&sBC[1][rr][8 * hh]);
#pragma unroll
            for (int i = 0; i < 16; ++i) Bsv[i >> 3][i & 7] = as_bf(sBC[0][32 * wv + tok(i)][col & 15]);
        }

        // ------------------------------------------------------ gates, W', P
        // e_a = e^{-a}, e_b = e^{-b}; invP_n = prod (1 + e_a) = P_p / P_n, the decay
        // between token n and the pivot p (the wave's token 16), so that neither it
        // nor its inverse spans more than 16 tokens.  One reciprocal
        // r = 1 / (invP (1 + e_b)) gives sigma(b) = r invP and P_n / P_p = r (1 + e_b).
        // Tokens past the end of the sequence (only in the last wave of a row) get
        // f = 1 and w = 0.
        uint32_t rw[3][8];  // EARLY: h, a, b of column tile 1, tokens (2p, 2p + 1)
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
        uint32_t nxt = 0;
        auto release = [&]() {  // every wave holds what it needs of the tile
            __builtin_amdgcn_s_setprio(0);
            if (dyn && threadIdx.x == 128) s_tk[1] = tk_of(k_req);
            __syncthreads();
            nxt = s_tk[1];  // (dyn: requested at this ticket's start; else static)
            if (nxt < total && wv >= 2) prefetch(nxt, lane);
        };
        float Pv[2][16];  // P (block: P SiLU(z)), the factor of the token's output
        f32x16 Y[2];      // D h / P, then + G W', then + C x_in
        bf16x8 Whi[2][2], Wlo[2][2];
        float Ptot[2];  // P over tokens 16..31, the second half (the aggregate's scale)
        float rQv[2];   // P over tokens 0..15: P at the pivot
        bool ok = true;
        auto gates = [&](auto tail_c) {
            constexpr bool TL = decltype(tail_c)::value;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (EARLY && j == 1) release();
                const bool rg1 = EARLY && j == 1;  // tile 1 from registers
                const int chn = 2 * col + j;
                float cum[16], tot[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rg = 32 * wv + 8 * q + 4 * hh;  // tile row of the group's first token
                    float run = 1.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 4 * q + r;
                        float ea = ex2((rg1 ? raw(1, i) : to_f(sAB[0][rg + r][chn])) * -kLog2e);
                        if (TL) ea = tok(i) < Lw ? ea : 0.f;
                        run = fmaf(run, ea, run);  // prod (1 + e^{-a})
                        cum[i] = run;
                    }
                    tot[q] = run;
                }
                // The decay is pivoted at token 16 (the chunk's middle): with Q the
                // product over tokens 0..15, invP'_k = invP_k / Q, so W' = w P_p / P_k and
                // the outputs' factor P_n / P_p stay within a 16-token product either side.
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
                // 2^96 bounds for both halves (W' then stays below 2^96 |h| and the
                // G @ W' sums far below fp32's range); false for NaN
                ok = ok && (Q <= 0x1p96f) && (acc <= 0x1p96f);
                const float rQ = rcp(Q);
                E[0] *= rQ;  // tokens before the pivot: P_p / P_k <= 1
                E[1] *= rQ;
                rQv[j] = rQ;
                Ptot[j] = rcp(acc);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    float wp[8];
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq) {
                        const int q = 2 * kb + qq;
                        const int rg = 32 * wv + 8 * q + 4 * hh;
                        float uw[7];
                        if (BLOCK) {
#pragma unroll
                            for (int k = 0; k < 7; ++k) uw[k] = to_f(sU[H + rg - 3 + k][chn]);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = 4 * q + r;
                            float h;
                            if (BLOCK) {
                                const float pre = cw[j][0] * uw[r] + cw[j][1] * uw[r + 1] +
                                                  cw[j][2] * uw[r + 2] + cw[j][3] * uw[r + 3];
                                h = pre * sigm(pre);
                            } else {
                                h = rg1 ? raw(0, i) : to_f(sU[rg + r][chn]);
                            }
                            if (TL) h = tok(i) < Lw ? h : 0.f;
                            const float eb =
                                ex2((rg1 ? raw(2, i) : to_f(sAB[1][rg + r][chn])) * -kLog2e);
                            const float invP = E[q] * cum[i];
                            const float qv = fmaf(invP, eb, invP);  // invP (1 + e^{-b})
                            const float rq = rcp(qv);
                            const float t = h * invP;
                            wp[4 * qq + r] = t * (rq * invP);  // h sigma(b) / P
                            Pv[j][i] = fmaf(rq, eb, rq);       // P
                            Y[j][i] = Dn[j] * t;               // D h / P
                            ok = ok && (__builtin_fabsf(wp[4 * qq + r]) < 0x1p110f) &&
                                 (qv < 1.329228e36f);  // 2^120
                        }
                    }
                    split8(wp, Whi[j][kb], Wlo[j][kb]);
                }
            }
        };
        if (Lw < T)
            gates(std::true_type{});
        else
            gates(std::false_type{});
        const bool wave_ok = __all(ok);
        if (BLOCK && y) {
            // fold SiLU(z) into the output factor
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float z0 = __uint_as_float(zb[i] << 16);
                const float z1 = __uint_as_float(zb[i] & 0xffff0000u);
                Pv[0][i] *= z0 * sigm(z0);
                Pv[1][i] *= z1 * sigm(z1);
            }
        }
        if constexpr (!EARLY) release();

        // --------------------------------- chunk aggregate (P_T, S) -> LDS
        // S = P_T (W'^T B), formed as B^T W' so each lane holds its own channel;
        // then the intra-chunk term G @ W'.  (One branch for both: the fallback
        // redefines what the epilogue reads, so none of the matrix-core path's
        // values stays live across the register recurrence.)
        bf16x8 Csc;  // C / sqrt(N) (1/4 is exact in bf16)
#pragma unroll
        for (int s = 0; s < 8; ++s) Csc[s] = (__bf16)((float)Cop[s] * scale);
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
                // S = P_T sum_k B_k w_k / P_k = (P_T / P_p) B^T W'; the wave's P_T = Q^-1 Ptot
                for (int i = 0; i < 8; ++i) sS[wv][tok(i)][2 * col + j] = sacc[i] * Ptot[j];
                if (!upper) sP[wv][2 * col + j] = Ptot[j] * rQv[j];
            }
            f32x16 g = {};
            g = mfma(Bop, Csc, g);  // g[i] = C_{col} . B_{tok(i)} / sqrt(N) = G[col][tok(i)]
            bf16x8 Ghi[2], Glo[2];
            float gv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) gv[i] = (tok(i) <= col) ? g[i] : 0.f;
            split16(gv, Ghi, Glo);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    Y[j] = mfma(Ghi[kb], Whi[j][kb], Y[j]);
                    Y[j] = mfma(Ghi[kb], Wlo[j][kb], Y[j]);
                    Y[j] = mfma(Glo[kb], Whi[j][kb], Y[j]);
                }
            }
        } else {
            float P, S[16];
            rr_aggregate<BLOCK>(L, Di, bi, cbase + lane, cbase + lane < Di, n0, hu, a, bg, Bm,
                                conv_w, conv_state, P, S);
            sP[wv][lane] = P;
#pragma unroll
            for (int s = 0; s < 16; ++s) sS[wv][s][lane] = S[s];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    Pv[j][i] = 0.f;
                    Y[j][i] = 0.f;
                }
        }
        __syncthreads();  // every wave's aggregate is in LDS

        // -------------------------------- look-back for the entering state
        // Waves 0 and 1 (which issue no tile copies) carry states 8w .. 8w+7 of
        // the 64 channels (lane = channel); each publishes and reads its own
        // slots, so the two look back in parallel.  Every published value is a
        // tagged word (the call's epoch and the kind: aggregate or inclusive
        // state) written by one agent-scope store: a reader takes a
        // predecessor's values once all 64 lanes' words carry the current tag,
        // so publishing needs no separate flag.  The nearest predecessor's
        // inclusive state ends the walk; otherwise its aggregate is folded in
        // and the walk moves one chunk further.
        if (wv < 2) {
            __builtin_amdgcn_s_setprio(2);  // the walk: the other two waves wait for it
            constexpr int SG = 8;
            const int s0 = SG * wv;
            const int64_t c_l = cbase + lane;
            const bool valid_l = c_l < Di;
            float Pt = 1.f, St[SG];
#pragma unroll
            for (int k = 0; k < SG; ++k) St[k] = 0.f;
            for (int w = 0; w < kW; ++w) {
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
                    xin[k] = (x0 && valid_l) ? x0[((int64_t)bi * Di + c_l) * N + s0 + k] : 0.f;
            } else {
                // The aggregate is published before the walk, or (lazy_agg) only
                // once this chunk finds it has to wait: a successor needs it only
                // while this chunk's inclusive state is not out.  Lazy publication
                // pays when the resident workgroups span few chunks of each row;
                // with deep chains every chunk waits, and late publication would
                // delay the walks behind it.
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
                size_t jx = me - 1;     // nearest predecessor not folded in yet
                uint32_t left = chunk;  // predecessors of this row not folded in yet
                uint32_t spins = 0;
                bool failed = false;
                for (;;) {
                    const uint64_t *pi = incl + (jx * 2 + wv) * (SG * 64);
                    uint64_t iv[SG];
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
                    const uint64_t *pa = agg + (jx * 2 + wv) * ((SG + 1) * 64);
                    uint64_t av[SG + 1];
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
                        failed = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (failed) {
#pragma unroll
                    for (int k = 0; k < SG; ++k) xin[k] = 0.f;
                }
            }
            uint64_t *ic = incl + mg * (SG * 64);
#pragma unroll
            for (int k = 0; k < SG; ++k) {
                const float xo = fmaf(Pt, xin[k], St[k]);
                if (chunk < (uint32_t)n_chunks - 1)
                    st_tagged(ic + k * 64 + lane, xo, tagI);
                else if (x_final && valid_l)
                    x_final[((int64_t)bi * Di + c_l) * N + s0 + k] = xo;
                sX[s0 + k][lane] = xin[k];
            }
            if (BLOCK && wv == 0 && conv_state_out && valid_l && chunk == (uint32_t)n_chunks - 1) {
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const int64_t m = L - 3 + k;
                    bf16 v = 0;
                    if (m >= 0)
                        v = hu[(tokbase + m) * Di + c_l];
                    else if (conv_state)
                        v = conv_state[((int64_t)bi * 3 + (m + 3)) * Di + c_l];
                    conv_state_out[((int64_t)bi * 3 + k) * Di + c_l] = v;
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        // static tickets: the next ticket's successor, for the next release
        // (every wave has read s_tk[1] by now: it did so before the two barriers
        // since)
        if (!dyn && threadIdx.x == 0) s_tk[1] = nxt + gridDim.x;
        __syncthreads();  // the workgroup's entering state is in LDS
        __builtin_amdgcn_s_setprio(1);

        after = (!wave_ok || !y) ? 0 : (ckpt && active) ? 24 : 16;
        if (!wave_ok) {
            // the fallback works in lane = channel layout
            float xin[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) xin[s] = sX[s][lane];
            for (int w = 0; w < wv; ++w) {
                const float pw = sP[w][lane];
#pragma unroll
                for (int s = 0; s < 16; ++s) xin[s] = fmaf(pw, xin[s], sS[w][s][lane]);
            }
            if (ckpt && active && cbase + lane < Di) {
                float *cp = ckpt + (((int64_t)bi * n_waves + (int64_t)chunk * kW + wv) * N) * Di +
                            cbase + lane;
#pragma unroll
                for (int s = 0; s < 16; ++s) cp[(int64_t)s * Di] = xin[s];
            }
            if (y)
                rr_output<BLOCK>(L, Di, bi, cbase + lane, cbase + lane < Di, n0, scale, hu, a, bg,
                                 Bm, Cm, D, z, conv_w, conv_state, xin, y);
        } else {
            // this wave's entering state in the B-operand layout (channel 2 col + j,
            // states 8h .. 8h+7): the workgroup's, carried through the waves before it
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
                // the state entering this 32-token wave: [Bt][n_waves][N][Di]
                float *cp = ckpt + (((int64_t)bi * n_waves + (int64_t)chunk * kW + wv) * N) * Di + cbase;
                const rsrc_t rc = make_rsrc(cp, (uint32_t)(N * Di * 4));
                const uint32_t vk = vc ? (uint32_t)((8 * hh) * Di + 2 * col) * 4 : kOOB;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const f32x2 v = {xs[0][k], xs[1][k]};
                    // (nontemporal: read back only by the backward, much later)
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rc,
                                                          vk + (uint32_t)(k * Di) * 4, 0, 2);
                }
            }
            if (y) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // P_n C x = (P_n / P_p) C (P_p x): the state enters scaled by P_p
                    float xp[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) xp[k] = xs[j][k] * rQv[j];
                    bf16x8 xh, xl;
                    split8(xp, xh, xl);
                    Y[j] = mfma(Csc, xh, Y[j]);
                    Y[j] = mfma(Csc, xl, Y[j]);
                }
                const rsrc_t ry = make_rsrc(y + ebase, (uint32_t)Lw * row2);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const f32x2 yv = {Pv[0][i] * Y[0][i], Pv[1][i] * Y[1][i]};
                    const uint32_t pk =
                        __builtin_bit_cast(uint32_t, __builtin_convertvector(yv, bf16x2));
                    // (no nontemporal hint: L2 merges the 64-byte pieces into whole lines)
                    __builtin_amdgcn_raw_buffer_store_b32(pk, ry, eoff(i), 0, 0);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        cur = nxt;
    }
    // the last workgroup out resets the ticket counter and advances the epoch
    // (every workgroup has taken its last ticket and read the epoch)
    if (threadIdx.x == 0) {
        const uint32_t old = add_agent(&hdr->done, 1u);
        if (old == gridDim.x - 1) {
#pragma unroll
            for (int q = 0; q < 8; ++q) st_agent(&hdr->queue[q], 0u);
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
    // as many workgroups as the device holds at once (two per CU)
    static const int per_cu[2] = {
        [] {
            int n = 0;
            return hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &n, (const void *)fwd_chunk_kernel<false>, 64 * kW, 0) == hipSuccess && n > 0
                       ? n : 1;
        }(),
        [] {
            int n = 0;
            return hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &n, (const void *)fwd_chunk_kernel<true>, 64 * kW, 0) == hipSuccess && n > 0
                       ? n : 1;
        }()};
    const int64_t slots = (int64_t)per_cu[g.block ? 1 : 0] * device_cu_count();
    const int64_t grid = pl.n_wg < slots ? pl.n_wg : slots;
    // lazy aggregates when a round of `grid` tickets spans at most ~4 chunks of a row
    const int lazy = (int64_t)g.Bt * pl.n_tiles * 4 >= grid ? 1 : 0;
    const uint32_t per_chunk = (uint32_t)(g.Bt * pl.n_tiles);
    const FastDiv fdc = make_fastdiv(per_chunk), fdt = make_fastdiv((uint32_t)pl.n_tiles);
    const uint32_t total = per_chunk * (uint32_t)pl.n_chunks;
    const TicketQueues tq = make_ticket_queues(per_chunk, (uint32_t)pl.n_chunks);
    // Ticket schedule: one queue handing out tickets in their own order.  Every
    // predecessor is then held by a workgroup that is running or done, so each
    // wait ends whatever share of the device this launch gets; deep chains also
    // advance as workgroups free up instead of in lockstep rounds (1 x 65536 x
    // 2048: 435 -> 394 us against the static assignment, 8 x 2048 x 1536: 2 %
    // slower).  NAJU_FWD_TICKETS=static (w, w + G, ..., which needs every
    // workgroup resident) or dynamic (per-XCD queues), read at every call,
    // overrides it.
    const char *tkenv = getenv("NAJU_FWD_TICKETS");
    const int dyn = (tkenv && tkenv[0] == 'd') ? 1 : (tkenv && tkenv[0] == 's') ? 0 : 2;
    int64_t L = g.L, Di = g.Di;
    int n_chunks = pl.n_chunks;
    float scale = g.scale;
    const bf16 *hu = (const bf16 *)g.hu, *a = (const bf16 *)g.a, *b = (const bf16 *)g.b,
               *B = (const bf16 *)g.B, *C = (const bf16 *)g.C, *z = (const bf16 *)g.z,
               *cs = (const bf16 *)g.conv_state;
    const float *D = g.D, *x0 = g.x0, *cw = g.conv_w;
    bf16 *y = (bf16 *)g.y, *cso = (bf16 *)g.conv_state_out;
    float *xf = g.x_final, *ck = g.ckpt;
    int dy = dyn;
    void *args[] = {&L, &Di, (void *)&fdc, (void *)&fdt, (void *)&total, (void *)&tq, &n_chunks, &scale,
                    &hu, &a, &b, &B, &C, &D, &x0, &z, &cw, &cs, &y, &xf, &cso, &ck, &hdr, &agg,
                    &incl, (void *)&lazy, &dy};
    const void *fn = g.block ? (const void *)fwd_chunk_kernel<true>
                             : (const void *)fwd_chunk_kernel<false>;
    return hipLaunchKernel(fn, dim3(grid), dim3(64 * kW), args, 0, stream);
}

}  // namespace naju

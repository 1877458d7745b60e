// naju_launch.h -- host-side plans (grid shapes, workspace layout) shared by
// the C-ABI layer and the kernel launchers of libnaju.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace naju {

// Forward decomposition: a wave owns kFwdT tokens of 64/LPC channels, a
// workgroup kFwdW consecutive waves along the sequence.
constexpr int kFwdT = 32;
constexpr int kFwdW = 8;
// The matrix-core forward uses 4-wave workgroups (two fit on a CU, so one can
// compute while the other waits in its look-back).
constexpr int kMfmaW = 4;
// Backward: same wave shape (checkpoints are taken per forward wave).
constexpr int kBwdT = 32;
constexpr int kBwdW = 8;
constexpr int kBwdTB = 8;  // tokens recomputed per sub-block

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Unsigned division of n < 2^31 by a fixed d >= 1 without a divide: with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, n / d =
// (mulhi(n, m) + n) >> l (the round-up multiplier method of Granlund and
// Montgomery, in its 32-bit "add" form).  Kernels take the pair from the host,
// so a uniform division is a scalar multiply-high, an add and a shift.
struct FastDiv {
    uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f)
{
    return (__umulhi(n, f.m) + n) >> f.l;
}

// Ticket queues of a persistent kernel, one per XCD: rows r (batch row x
// channel tile) with r % 8 == q form queue q, served chunk-major, so all chunks
// of a row -- a look-back chain -- run on one XCD.  rows[q] is the queue's row
// count (its FastDiv), total[q] its ticket count.
struct TicketQueues {
    FastDiv rows[8];
    uint32_t total[8];
};
inline TicketQueues make_ticket_queues(uint32_t per_chunk, uint32_t n_chunks)
{
    TicketQueues t{};
    for (uint32_t q = 0; q < 8; ++q) {
        const uint32_t r = per_chunk > q ? (per_chunk - q + 7) / 8 : 0;
        t.rows[q] = make_fastdiv(r > 0 ? r : 1);
        t.total[q] = r * n_chunks;
    }
    return t;
}

struct FwdPlan {
    int n_tiles;      // channel tiles of 64/LPC channels
    int n_chunks;     // workgroup chunks of kFwdT*kFwdW tokens
    int64_t n_wg;     // workgroups = tickets
    int64_t n_waves;  // kFwdT-token chunks (checkpoint rows) per batch row
    size_t off_flags, off_agg, off_incl, bytes;
};

inline FwdPlan fwd_plan(int64_t Bt, int64_t L, int64_t Di, int64_t N, int W = kFwdW)
{
    FwdPlan p{};
    const int64_t cpw = 64 / (N / 16);
    p.n_tiles = (int)((Di + cpw - 1) / cpw);
    p.n_chunks = (int)((L + kFwdT * W - 1) / (kFwdT * W));
    p.n_wg = Bt * p.n_tiles * p.n_chunks;
    p.n_waves = (L + kFwdT - 1) / kFwdT;
    // the matrix-core forwards look back in state groups (four of four: four
    // (P, S[4]) aggregates and four x_out[4] per workgroup chunk; or two of
    // eight), each value a tagged 64-bit word; the register forward uses flags
    // and fp32 payloads
    const size_t fl = W == kMfmaW ? 2 : 1, ar = W == kMfmaW ? 20 : 17;
    const size_t vb = W == kMfmaW ? 8 : 4;  // bytes per published value
    p.off_flags = 256;
    p.off_agg = align256(p.off_flags + 4 * fl * (size_t)p.n_wg);
    p.off_incl = align256(p.off_agg + ar * 64 * vb * (size_t)p.n_wg);
    p.bytes = align256(p.off_incl + 16 * 64 * vb * (size_t)p.n_wg);
    return p;
}

// workspace bytes of a forward call, whichever kernel variant serves it
inline size_t fwd_ws_bytes(int64_t Bt, int64_t L, int64_t Di, int64_t N)
{
    const size_t a = fwd_plan(Bt, L, Di, N, kFwdW).bytes;
    const size_t b = N == 16 ? fwd_plan(Bt, L, Di, N, kMfmaW).bytes : 0;
    return a > b ? a : b;
}

// checkpoint: the state entering every kFwdT-token chunk, [Bt][n_waves][N][Di] fp32
inline size_t ckpt_bytes(int64_t Bt, int64_t L, int64_t Di, int64_t N)
{
    return (size_t)Bt * (size_t)((L + kFwdT - 1) / kFwdT) * (size_t)N * (size_t)Di * 4;
}

// Matrix-core backward decomposition: a workgroup owns 128 tokens (four
// 32-token waves) of a super-tile of n_sub consecutive 32-channel tiles, which
// it visits in turn; its reverse look-back runs per (tile, 128-token chunk).
struct MfmaBwdShape {
    int n_tiles;   // 32-channel tiles
    int n_sub;     // tiles per super-tile
    int n_super;   // super-tiles (dB/dC partials per token)
    int n_chunks;  // 128-token chunks
    int64_t n_wg;  // workgroups = tickets
};

inline MfmaBwdShape mfma_bwd_shape(int64_t Bt, int64_t L, int64_t Di)
{
    // workgroups come in pairs sharing 2 n_sub consecutive tiles (alternate
    // tiles each), so n_super is even
    MfmaBwdShape m{};
    m.n_tiles = (int)((Di + 31) / 32);
    const int half = (m.n_tiles + 1) / 2;
    m.n_sub = half < 4 ? (half > 0 ? half : 1) : 4;
    m.n_super = 2 * ((m.n_tiles + 2 * m.n_sub - 1) / (2 * m.n_sub));
    m.n_chunks = (int)((L + 127) / 128);
    m.n_wg = Bt * m.n_super * m.n_chunks;
    return m;
}

constexpr int kDdGroups = 32;  // most row groups of the first dD / dconv_w reduction pass

struct BwdPlan {
    int n_tiles, n_chunks;
    int64_t n_wg, n_waves;
    size_t off_flags, off_agg, off_incl;  // reverse look-back (same shapes as forward)
    size_t off_mflags, off_magg, off_mincl;  // matrix-core look-back, per (tile, chunk)
    size_t off_bc;    // dB/dC partials   [Bt][L][n_parts][2N] fp32 (tiles or super-tiles)
    size_t off_dd;    // dD partials      [Bt][n_waves][Di] fp32
    size_t off_dw;    // dconv_w partials [Bt][n_waves][Di][4] fp32
    size_t off_edge;  // block: per wave boundary  [Bt][n_waves][6][Di] fp32
                      //   rows 0-2: dpre of the wave's first 3 tokens
                      //   rows 3-5: in-wave partial du of its last 3 tokens
    size_t off_ckpt;  // recomputed checkpoints when the caller passes none
    size_t off_fwd;   // workspace of the checkpoint-only forward
    // matrix-core backward: chunks its rescaled form cannot take
    size_t off_fixmask;  // [Bt][n_super][n_waves] u32 tile bits
    size_t off_fixlist;  // [Bt][n_super][n_waves] u32 keys
    size_t off_fixmu;    // [Bt][n_waves][N][Di] fp32 entering adjoints
    size_t off_dd2;      // dD / dconv_w row-group partials [kDdGroups][Di][5] fp32
    size_t bytes;
};

inline BwdPlan bwd_plan(int64_t Bt, int64_t L, int64_t Di, int64_t N, bool block)
{
    BwdPlan p{};
    const FwdPlan f = fwd_plan(Bt, L, Di, N);
    // look-back regions sized for the finer of the two chunkings (128 tokens)
    const FwdPlan f4 = fwd_plan(Bt, L, Di, N, kMfmaW);
    p.n_tiles = f.n_tiles;
    p.n_chunks = f.n_chunks;
    p.n_wg = f.n_wg;
    p.n_waves = f.n_waves;
    p.off_flags = f4.off_flags;
    p.off_agg = f4.off_agg;
    p.off_incl = f4.off_incl;
    const MfmaBwdShape m = mfma_bwd_shape(Bt, L, Di);
    const size_t m_ent = N == 16 ? (size_t)Bt * m.n_tiles * m.n_chunks : 0;
    p.off_mflags = f4.bytes;
    p.off_magg = align256(p.off_mflags + 4 * m_ent);
    p.off_mincl = align256(p.off_magg + 17 * 32 * 4 * m_ent);
    p.off_bc = align256(p.off_mincl + 16 * 32 * 4 * m_ent);
    const int64_t n_parts = (N == 16 && m.n_super > p.n_tiles) ? m.n_super : p.n_tiles;
    p.off_dd = align256(p.off_bc + (size_t)Bt * L * n_parts * 2 * N * 4);
    p.off_dw = align256(p.off_dd + (size_t)Bt * p.n_waves * Di * 4);
    p.off_edge = align256(p.off_dw + (block ? (size_t)Bt * p.n_waves * Di * 4 * 4 : 0));
    p.off_ckpt = align256(p.off_edge + (block ? (size_t)Bt * p.n_waves * 6 * Di * 4 : 0));
    p.off_fwd = align256(p.off_ckpt + ckpt_bytes(Bt, L, Di, N));
    const size_t n_keys = (size_t)Bt * (size_t)m.n_super * (size_t)p.n_waves;
    p.off_fixmask = align256(p.off_fwd + fwd_ws_bytes(Bt, L, Di, N));
    p.off_fixlist = align256(p.off_fixmask + 4 * n_keys);
    p.off_fixmu = align256(p.off_fixlist + 4 * n_keys);
    p.off_dd2 = align256(p.off_fixmu + (N == 16 ? ckpt_bytes(Bt, L, Di, N) : 0));
    p.bytes = align256(p.off_dd2 + (size_t)kDdGroups * Di * 5 * 4);
    return p;
}

struct FwdArgs {
    int io, N;
    bool block;
    int64_t Bt, L, Di;
    float scale;
    const void *hu, *a, *b, *B, *C;
    const float *D, *x0;
    const void *z;
    const float *conv_w;
    const void *conv_state;
    void *y;
    float *x_final;
    void *conv_state_out;
    float *ckpt;
    void *ws;  // forward workspace (fwd_plan layout)
};

struct BwdArgs {
    int io, N;
    bool block;
    int64_t Bt, L, Di;
    float scale;
    const void *hu, *a, *b, *B, *C;
    const float *D, *x0;
    const void *z;
    const float *conv_w;
    const void *conv_state;
    const float *ckpt;  // required here (the API layer recomputes it if absent)
    const void *dy;
    const float *dx_final;
    void *dhu, *da, *db, *dB, *dC, *dz;
    float *dD, *dx0, *dconv_w;
    void *dconv_state;
    void *ws;  // backward workspace (bwd_plan layout)
};

hipError_t launch_fwd(const FwdArgs &g, hipStream_t stream);
hipError_t launch_fwd_mfma(const FwdArgs &g, hipStream_t stream);  // bf16, d_state 16
bool use_fwd_mfma64(const FwdArgs &g);                              // bf16, d_state 64
hipError_t launch_fwd_mfma64(const FwdArgs &g, hipStream_t stream);
int device_cu_count();  // compute units of the current device (cached)

// one-token step with the state (and, for the block, the conv window) in place
struct StepArgs {
    int io, N;
    bool block;
    int64_t Bt, Di;
    float scale;
    const void *hu, *a, *b, *B, *C;  // [Bt][Di] / [Bt][N]
    const float *D;
    const void *z;
    const float *conv_w;
    void *conv_state;  // [Bt][3][Di], shifted by one token
    float *x;          // [Bt][Di][N], updated
    void *y;           // [Bt][Di]
};
hipError_t launch_step(const StepArgs &g, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &g, hipStream_t stream);
hipError_t launch_bwd_mfma(const BwdArgs &g, hipStream_t stream);  // bf16, d_state 16
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);
hipError_t launch_empty_seq(int io, int64_t Bt, int64_t Di, int64_t N, const float *x0,
                            float *x_final, const void *conv_state, void *conv_state_out,
                            hipStream_t stream);

// mixer layer (bf16): projections around the block forward
struct MixerArgs {
    int64_t Bt, L, dm, Di, N;
    float scale;
    const void *xn, *res;            // [Bt][L][dm]; res may be null
    const void *W_u, *W_z;           // [dm][Di]
    const float *conv_w;             // [Di][4]
    const void *conv_state;          // [Bt][3][Di] or null
    const void *W_a, *W_b;           // [Di][Di]
    const float *a_bias, *b_bias;    // [Di]
    const void *W_B, *W_C;           // [Di][N]
    const float *D;                  // [Di]
    const void *W_out;               // [Di][dm]
    void *out;                       // [Bt][L][dm]
    void *ws;                        // mixer_plan layout
};
size_t mixer_ws_bytes(int64_t Bt, int64_t L, int64_t Di, int64_t N);
size_t mixer_bwd_ws_bytes(int64_t Bt, int64_t L, int64_t Di, int64_t N);
struct MixerGrads {
    const void *d_out;               // [Bt][L][dm] bf16
    const void *saved;               // workspace of a naju_mixer_fwd call, or null
    float *dxn;                      // [Bt][L][dm]
    float *dW_u, *dW_z;              // [dm][Di]
    float *dconv_w;                  // [Di][4]
    void *dconv_state;               // [Bt][3][Di] bf16 or null
    float *dW_a, *da_bias, *dW_b, *db_bias;
    float *dW_B, *dW_C;              // [Di][N]
    float *dD;                       // [Di]
    float *dW_out;                   // [Di][dm]
};
const char *mixer_bwd(const MixerArgs &g, const MixerGrads &d, hipStream_t stream);
// enqueues the layer; returns nullptr, or a message on failure
const char *mixer_fwd(const MixerArgs &g, hipStream_t stream);

}  // namespace naju

// naju_mixer.hip -- the mixer layer around the scan (naju_mixer_fwd).
//
// The block flowchart of the Naju reproduction README (arXiv 2607.21000,
// "Background and main changes"): the normalized token goes through the
// input projection; one branch passes a causal depthwise conv + SiLU and feeds
// the forget gate, the write gate and the token-dependent B/C directions, then
// the state scan with its readout and feedthrough; the other branch modulates
// the readout through SiLU; an output projection and the residual close the
// layer.  Per token (row vectors, W stored [in][out]):
//
//     u = xn W_u,  z = xn W_z                      (bf16)
//     h = SiLU(conv(u))                            (bf16, stored for the projections)
//     a = h W_a + a_bias,  b = h W_b + b_bias      (bf16; biases 5 / -2 at the
//     B = h W_B,  C = h W_C                         page's initialisation)
//     y = scan readout (u, z, a, b, B, C, D)       (naju_block_fwd: it recomputes
//                                                   h from u in fp32)
//     out = res + y W_out                          (bf16)
//
// The projections are dense GEMMs on the matrix cores through hipBLASLt (bf16
// operands, fp32 accumulation, bf16 results), with the gate biases and the
// residual in the GEMM epilogue; conv + SiLU is a streaming kernel here; the
// scan is the block forward of this library.
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "../../include/naju.h"
#include "naju_device.h"
#include "naju_launch.h"
#include "naju_mfma.h"

namespace naju {

// ------------------------------------------------------------ conv + SiLU
// Thread = (batch row, 8 channels, 32-token segment): the 4-tap window slides
// in registers, so each u row is read once (plus 3 halo rows per segment);
// a wave covers 64 x 16 consecutive bytes of a row.
constexpr int kSeg = 32;

__global__ __launch_bounds__(256) void conv_silu_kernel(const int64_t L, const int64_t Di,
                                                        const bf16 *__restrict__ u,
                                                        const float *__restrict__ w,
                                                        const bf16 *__restrict__ cs,
                                                        bf16 *__restrict__ h)
{
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (c0 >= Di) return;
    const int64_t n0 = (int64_t)blockIdx.y * kSeg;
    const int64_t bi = blockIdx.z;
    const bf16 *ub = u + bi * L * Di + c0;
    bf16 *hb = h + bi * L * Di + c0;
    float wk[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float4 q = *(const float4 *)(w + (c0 + e) * 4);
        wk[e][0] = q.x;
        wk[e][1] = q.y;
        wk[e][2] = q.z;
        wk[e][3] = q.w;
    }
    auto unpack = [](const uint4 &q, float (&v)[8]) {
        const uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(p[e] << 16);
            v[2 * e + 1] = __uint_as_float(p[e] & 0xffff0000u);
        }
    };
    // window: u at tokens n-3, n-2, n-1 (before the sequence: conv_state or 0)
    float win[3][8];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int64_t m = n0 - 3 + r;
        uint4 q = {0u, 0u, 0u, 0u};
        if (m >= 0)
            q = *(const uint4 *)(ub + m * Di);
        else if (cs)
            q = *(const uint4 *)(cs + (bi * 3 + (m + 3)) * Di + c0);
        unpack(q, win[r]);
    }
    const int64_t n1 = n0 + kSeg < L ? n0 + kSeg : L;
    for (int64_t n = n0; n < n1; ++n) {
        float cur[8];
        unpack(*(const uint4 *)(ub + n * Di), cur);
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            float hv[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int c = e + k;
                const float pre = wk[c][0] * win[0][c] + wk[c][1] * win[1][c] +
                                  wk[c][2] * win[2][c] + wk[c][3] * cur[c];
                hv[k] = pre * sigm(pre);
            }
            o[e / 2] = (uint32_t)from_f<bf16>(hv[0]) | ((uint32_t)from_f<bf16>(hv[1]) << 16);
        }
        *(uint4 *)(hb + n * Di) = uint4{o[0], o[1], o[2], o[3]};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            win[0][c] = win[1][c];
            win[1][c] = win[2][c];
            win[2][c] = cur[c];
        }
    }
}

// ------------------------------------------------------------ GEMMs
// hipBLASLt is column-major: D (m x n) = op(X) (m x k) op(Y) (k x n)
// (+ bias[m]) (+ C, beta 1), with C of D's type.  The row-major products of
// the layer map onto it as follows (T tokens; W stored [in][out]):
//   D[T][n] = A[T][k] W[k][n]    -> D^T = W^T A^T : X = W (n x k, ld n), Y = A (k x T, ld k)
//   D[T][n] = A[T][k] W[n][k]^T  -> D^T = W A^T   : X = W^T stored (k x n, ld k), op T
//   G[k][n] = A[T][k]^T E[T][n]  -> G^T = E^T A   : X = E (n x T, ld n), Y = A^T stored, op T
// Plans (layouts, epilogue, the heuristic's first algorithm) are cached per
// device and shape.
struct GemmPlan {
    hipblasLtMatmulDesc_t md = nullptr;
    hipblasLtMatrixLayout_t lx = nullptr, ly = nullptr, ld = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
    bool ok = false;
};

struct GemmShape {
    int64_t m, n, k, ldx, ldy, ldd;
    bool tx, ty;
    hipDataType td;  // type of D (and C): HIP_R_16BF or HIP_R_32F
    bool bias, beta;
    int batch = 1;                 // strided batch of independent products
    int64_t sx = 0, sy = 0, sd = 0;  // element strides between the batch's operands
};

static std::mutex g_lt_mu;
static std::map<int, hipblasLtHandle_t> g_lt;
static std::map<std::tuple<int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, int>,
                GemmPlan>
    g_plans;

constexpr size_t kGemmWs = (size_t)32 << 20;  // hipBLASLt workspace inside ws

// Enqueues one product.  Returns a message on failure (nullptr on success).
static const char *gemm_cm(hipStream_t st, const GemmShape &g, const void *X, const void *Y,
                           const float *bias, const void *C, void *D, void *gws)
{
    if (g.m == 0 || g.n == 0) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return "hipGetDevice failed";
    std::lock_guard<std::mutex> lk(g_lt_mu);
    hipblasLtHandle_t &hd = g_lt[dev];
    if (!hd && hipblasLtCreate(&hd) != HIPBLAS_STATUS_SUCCESS) {
        hd = nullptr;
        return "hipblasLtCreate failed";
    }
    const int flags = (g.bias ? 1 : 0) | (g.beta ? 2 : 0) | (g.tx ? 4 : 0) | (g.ty ? 8 : 0) |
                      (g.td == HIP_R_32F ? 16 : 0);
    GemmPlan &p = g_plans[std::make_tuple(dev, g.m, g.n, g.k, g.ldx, g.ldy, g.ldd, flags, g.batch)];
    if (!p.ok) {
        const uint64_t xr = g.tx ? g.k : g.m, xc = g.tx ? g.m : g.k;
        const uint64_t yr = g.ty ? g.n : g.k, yc = g.ty ? g.k : g.n;
        if (hipblasLtMatmulDescCreate(&p.md, HIPBLAS_COMPUTE_32F, HIP_R_32F) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&p.lx, HIP_R_16BF, xr, xc, g.ldx) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&p.ly, HIP_R_16BF, yr, yc, g.ldy) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&p.ld, g.td, (uint64_t)g.m, (uint64_t)g.n, g.ldd) !=
                HIPBLAS_STATUS_SUCCESS)
            return "hipBLASLt descriptor creation failed";
        if (g.batch > 1) {
            const int32_t bc = g.batch;
            const int64_t st3[3] = {g.sx, g.sy, g.sd};
            hipblasLtMatrixLayout_t ls[3] = {p.lx, p.ly, p.ld};
            for (int q = 0; q < 3; ++q)
                if (hipblasLtMatrixLayoutSetAttribute(ls[q], HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT,
                                                      &bc, sizeof(bc)) != HIPBLAS_STATUS_SUCCESS ||
                    hipblasLtMatrixLayoutSetAttribute(
                        ls[q], HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &st3[q],
                        sizeof(st3[q])) != HIPBLAS_STATUS_SUCCESS)
                    return "hipBLASLt batch attributes failed";
        }
        const hipblasOperation_t opx = g.tx ? HIPBLAS_OP_T : HIPBLAS_OP_N;
        const hipblasOperation_t opy = g.ty ? HIPBLAS_OP_T : HIPBLAS_OP_N;
        hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSA, &opx, sizeof(opx));
        hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSB, &opy, sizeof(opy));
        if (g.bias) {
            const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
            const hipDataType bt = HIP_R_32F;
            hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi,
                                            sizeof(epi));
            hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt,
                                            sizeof(bt));
            hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias,
                                            sizeof(bias));
        }
        hipblasLtMatmulPreference_t pref = nullptr;
        const uint64_t wsmax = kGemmWs;
        hipblasLtMatmulHeuristicResult_t res[1];
        int got = 0;
        const bool found =
            hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                  &wsmax, sizeof(wsmax)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulAlgoGetHeuristic(hd, p.md, p.lx, p.ly, p.ld, p.ld, pref, 1, res,
                                            &got) == HIPBLAS_STATUS_SUCCESS &&
            got > 0;
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        if (!found) return "hipBLASLt found no algorithm for a product";
        // (the heuristic's first choice: timing its other candidates on the
        // 8 x 2048-token layer made single projections up to 6 % faster, but it
        // synchronises the stream on a shape's first call, and the gain for the
        // whole layer was not established)
        p.algo = res[0].algo;
        p.ws = res[0].workspaceSize;
        p.ok = true;
    }
    if (g.bias)
        hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias,
                                        sizeof(bias));
    const float one = 1.f, zero = 0.f;
    if (hipblasLtMatmul(hd, p.md, &one, X, p.lx, Y, p.ly, g.beta ? &one : &zero,
                        g.beta ? C : D, p.ld, D, p.ld, &p.algo, gws, p.ws, st) !=
        HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatmul failed";
    return nullptr;
}

// D[T][n] = A[T][k] W[k][n] (+ bias[n]) (+ C[T][n]); bf16 D
static const char *gemm(hipStream_t st, int64_t T, int64_t n, int64_t k, const void *A,
                        const void *W, const float *bias, const void *C, void *D, void *gws)
{
    const GemmShape g{n, T, k, n, k, n, false, false, HIP_R_16BF, bias != nullptr, C != nullptr};
    return gemm_cm(st, g, W, A, bias, C, D, gws);
}

// D[T][n] = A[T][k] W[n][k]^T (+ D when acc); D fp32 or bf16
static const char *gemm_nt(hipStream_t st, int64_t T, int64_t n, int64_t k, const void *A,
                           const void *W, bool acc, void *D, hipDataType td, void *gws)
{
    const GemmShape g{n, T, k, k, k, n, true, false, td, false, acc};
    return gemm_cm(st, g, W, A, nullptr, D, D, gws);
}

// out[i] = sum_s part[s][i], s = 0 .. S-1 in order (fp32)
__global__ __launch_bounds__(256) void sum_parts_kernel(const int64_t n, const int S,
                                                        const float *__restrict__ part,
                                                        float *__restrict__ out)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float v = part[i];
        for (int s = 1; s < S; ++s) v += part[(int64_t)s * n + i];
        out[i] = v;
    }
}

// G[k][n] (fp32) = A[T][k]^T E[T][n]: the weight gradient of D = A W.  The output
// is small (k x n) and the contraction long (T tokens), so one product fills few
// of the CUs: with `scratch` (fp32, `scratch_bytes`) the tokens are cut into S
// slices, multiplied as one strided batch into S partial gradients, and summed in
// slice order.
static const char *gemm_wgrad(hipStream_t st, int64_t T, int64_t n, int64_t k, const void *A,
                              const void *E, float *G, void *gws, float *scratch = nullptr,
                              size_t scratch_bytes = 0)
{
    const int64_t tiles = ((n + 127) / 128) * ((k + 127) / 128);
    int S = (int)std::min<int64_t>(8, std::max<int64_t>(1, (512 + tiles - 1) / tiles));
    while (S > 1 && (T % S != 0 || T / S < 512 || (size_t)S * n * k * 4 > scratch_bytes)) --S;
    if (!scratch || S == 1) {
        const GemmShape g{n, k, T, n, k, n, false, true, HIP_R_32F, false, false};
        return gemm_cm(st, g, E, A, nullptr, nullptr, G, gws);
    }
    const int64_t Ts = T / S;
    const GemmShape g{n, k, Ts, n, k, n, false, true, HIP_R_32F, false, false, S, Ts * n, Ts * k,
                      n * k};
    const char *e = gemm_cm(st, g, E, A, nullptr, nullptr, scratch, gws);
    if (e) return e;
    const int64_t cnt = n * k;
    const unsigned blocks = (unsigned)std::min<int64_t>((cnt + 255) / 256, 4096);
    hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks), dim3(256), 0, st, cnt, S,
                       (const float *)scratch, G);
    return hipGetLastError() == hipSuccess ? nullptr : "partial-sum launch failed";
}

// ------------------------------------------------------------ layout of ws
// u, z, h, a, b, y [T][Di] bf16; B, C [T][N] bf16; the GEMM workspace; the
// block forward's own workspace -- each 256-byte aligned.
struct MixerPlan {
    size_t off_u, off_z, off_h, off_a, off_b, off_y, off_B, off_C, off_g, off_f, off_ck, bytes;
};

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

static MixerPlan mixer_plan(int64_t Bt, int64_t L, int64_t Di, int64_t N)
{
    MixerPlan m{};
    const size_t act = up256((size_t)(Bt * L * Di) * 2), tok = up256((size_t)(Bt * L * N) * 2);
    size_t o = 0;
    m.off_u = o;
    o += act;
    m.off_z = o;
    o += act;
    m.off_h = o;
    o += act;
    m.off_a = o;
    o += act;
    m.off_b = o;
    o += act;
    m.off_y = o;
    o += act;
    m.off_B = o;
    o += tok;
    m.off_C = o;
    o += tok;
    m.off_g = o;
    o += kGemmWs;
    m.off_f = o;
    o += up256(fwd_ws_bytes(Bt, L, Di, N));
    m.off_ck = o;  // the scan's checkpoints, kept for a backward that reuses this workspace
    o += up256(ckpt_bytes(Bt, L, Di, N));
    m.bytes = o;
    return m;
}

size_t mixer_ws_bytes(int64_t Bt, int64_t L, int64_t Di, int64_t N)
{
    return mixer_plan(Bt, L, Di, N).bytes;
}

hipError_t launch_conv_silu(int64_t Bt, int64_t L, int64_t Di, const void *u, const float *w,
                            const void *cs, void *h, hipStream_t st)
{
    if (Bt == 0 || L == 0 || Di == 0) return hipSuccess;
    const dim3 grid((unsigned)((Di / 8 + 255) / 256), (unsigned)((L + kSeg - 1) / kSeg),
                    (unsigned)Bt);
    hipLaunchKernelGGL(conv_silu_kernel, grid, dim3(256), 0, st, L, Di, (const bf16 *)u, w,
                       (const bf16 *)cs, (bf16 *)h);
    return hipGetLastError();
}

static const char *mixer_forward_pass(const MixerArgs &g, const MixerPlan &m, float *ckpt,
                                      hipStream_t st);

const char *mixer_fwd(const MixerArgs &g, hipStream_t st)
{
    const MixerPlan m = mixer_plan(g.Bt, g.L, g.Di, g.N);
    const char *e;
    if ((e = mixer_forward_pass(g, m, (float *)((char *)g.ws + m.off_ck), st))) return e;
    const int64_t T = g.Bt * g.L;
    return gemm(st, T, g.dm, g.Di, (char *)g.ws + m.off_y, g.W_out, nullptr, g.res, g.out,
                (char *)g.ws + m.off_g);
}

// ------------------------------------------------------------ backward
// conv + SiLU backward of the projection path: dpre = dh SiLU'(pre) with
// SiLU'(p) = s (1 + p (1 - s)); du = du_scan + conv^T(dpre); per-segment
// partial sums of dconv_w (reduced in a fixed order by mixer_dw_reduce_kernel);
// the first segment also forms d(conv_state).  Thread = (batch row, 8 channels,
// kSegB-token segment); the window of the last four dpre slides in registers.
constexpr int kSegB = 32;

__global__ __launch_bounds__(64) void conv_silu_bwd_kernel(
    const int64_t L, const int64_t Di, const int nseg, const bf16 *__restrict__ u,
    const float *__restrict__ w, const bf16 *__restrict__ cs, const float *__restrict__ dh,
    const bf16 *__restrict__ du_scan, bf16 *__restrict__ du, float *__restrict__ dw_part,
    const bf16 *__restrict__ dcs_scan, bf16 *__restrict__ dcs)
{
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + threadIdx.x) * 8;
    if (c0 >= Di) return;
    const int64_t n0 = (int64_t)blockIdx.y * kSegB;
    const int64_t bi = blockIdx.z;
    const int64_t n1 = n0 + kSegB < L ? n0 + kSegB : L;
    float wk[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float4 v = *(const float4 *)(w + (c0 + e) * 4);
        wk[e][0] = v.x;
        wk[e][1] = v.y;
        wk[e][2] = v.z;
        wk[e][3] = v.w;
    }
    auto ld_u = [&](int64_t m, float (&v)[8]) {  // u_m (conv_state before 0, zeros past L)
        uint4 q = {0u, 0u, 0u, 0u};
        if (m >= 0 && m < L)
            q = *(const uint4 *)(u + (bi * L + m) * Di + c0);
        else if (m < 0 && cs)
            q = *(const uint4 *)(cs + (bi * 3 + (m + 3)) * Di + c0);
        const uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(p[e] << 16);
            v[2 * e + 1] = __uint_as_float(p[e] & 0xffff0000u);
        }
    };
    float uw[4][8];  // u_{t-3} .. u_t
    for (int r = 0; r < 3; ++r) ld_u(n0 - 3 + r, uw[r + 1]);
    float dp[4][8];  // dpre_{t-3} .. dpre_t
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) dp[r][c] = 0.f;
    float dws[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) dws[c][k] = 0.f;
    // dpre for tokens n0 .. n1 + 2 (zero past L); du_m is complete once dpre_{m+3} is known
    for (int64_t t = n0; t < n1 + 3; ++t) {
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                uw[r][c] = uw[r + 1][c];
                dp[r][c] = dp[r + 1][c];
            }
        ld_u(t, uw[3]);
        float g[8];
        if (t < L) {
            const float4 g0 = *(const float4 *)(dh + (bi * L + t) * Di + c0);
            const float4 g1 = *(const float4 *)(dh + (bi * L + t) * Di + c0 + 4);
            g[0] = g0.x, g[1] = g0.y, g[2] = g0.z, g[3] = g0.w;
            g[4] = g1.x, g[5] = g1.y, g[6] = g1.z, g[7] = g1.w;
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) g[c] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float pre = wk[c][0] * uw[0][c] + wk[c][1] * uw[1][c] + wk[c][2] * uw[2][c] +
                              wk[c][3] * uw[3][c];
            const float sg = sigm(pre);
            dp[3][c] = g[c] * sg * (1.f + pre * (1.f - sg));
            if (t < n1) {
#pragma unroll
                for (int k = 0; k < 4; ++k) dws[c][k] += dp[3][c] * uw[k][c];
            }
        }
        const int64_t m = t - 3;  // du_m = sum_k w_k dpre_{m+3-k}
        if (m >= n0 && m < n1) {
            const uint4 q = *(const uint4 *)(du_scan + (bi * L + m) * Di + c0);
            const uint32_t p[4] = {q.x, q.y, q.z, q.w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v2[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int c = 2 * e + h2;
                    const float base = __uint_as_float(h2 ? (p[e] & 0xffff0000u) : (p[e] << 16));
                    v2[h2] = base + wk[c][0] * dp[3][c] + wk[c][1] * dp[2][c] +
                             wk[c][2] * dp[1][c] + wk[c][3] * dp[0][c];
                }
                o[e] = (uint32_t)from_f<bf16>(v2[0]) | ((uint32_t)from_f<bf16>(v2[1]) << 16);
            }
            *(uint4 *)(du + (bi * L + m) * Di + c0) = uint4{o[0], o[1], o[2], o[3]};
        }
        // d(conv_state) row r (token r - 3): sum over k <= r of w_k dpre_{r-k}
        if (n0 == 0 && dcs && t == 2) {
            // dp[3] = dpre_2, dp[2] = dpre_1, dp[1] = dpre_0 (zero when L is shorter)
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                uint32_t o[4];
                const uint4 q = dcs_scan ? *(const uint4 *)(dcs_scan + (bi * 3 + r) * Di + c0)
                                         : uint4{0u, 0u, 0u, 0u};
                const uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v2[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int c = 2 * e + h2;
                        float acc = __uint_as_float(h2 ? (p[e] & 0xffff0000u) : (p[e] << 16));
                        // token r - 3 is tap k of token t' = r - 3 + 3 - k = r - k
#pragma unroll
                        for (int k = 0; k <= r; ++k) acc += wk[c][k] * dp[1 + r - k][c];
                        v2[h2] = acc;
                    }
                    o[e] = (uint32_t)from_f<bf16>(v2[0]) | ((uint32_t)from_f<bf16>(v2[1]) << 16);
                }
                *(uint4 *)(dcs + (bi * 3 + r) * Di + c0) = uint4{o[0], o[1], o[2], o[3]};
            }
        }
    }
    float *pp = dw_part + ((bi * nseg + blockIdx.y) * Di + c0) * 4;
#pragma unroll
    for (int c = 0; c < 8; ++c)
        *(float4 *)(pp + c * 4) = float4{dws[c][0], dws[c][1], dws[c][2], dws[c][3]};
}

// Column sums of a [rows][cols] array (fp32 partials or bf16 values) in a
// fixed order: workgroup (column block of 64, row slice); its 4 waves take
// interleaved rows of the slice, then combine in LDS in wave order.  With
// rows_per == rows a single launch gives the final sums (plus `add`, if any).
template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const int64_t rows, const int64_t cols,
                                                     const int64_t rows_per,
                                                     const T *__restrict__ x,
                                                     const float *__restrict__ add,
                                                     float *__restrict__ out)
{
    __shared__ float part[4][64];
    const int64_t c = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
    const int wv = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per;
    const int64_t r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
    float acc = 0.f;
    if (c < cols)
        for (int64_t r = r0 + wv; r < r1; r += 4) acc += to_f(x[r * cols + c]);
    part[wv][threadIdx.x & 63] = acc;
    __syncthreads();
    if (wv == 0 && c < cols) {
        float t = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] +
                  part[3][threadIdx.x];
        if (add) t += add[c];
        out[(int64_t)blockIdx.y * cols + c] = t;
    }
}

// two fixed-order passes: [rows][cols] -> [slices][cols] -> out (+ add)
template <typename T>
static hipError_t colsum(const T *x, int64_t rows, int64_t cols, const float *add, float *tmp,
                         int64_t slices, float *out, hipStream_t st)
{
    const int64_t per = (rows + slices - 1) / slices;
    const unsigned cb = (unsigned)((cols + 63) / 64);
    hipLaunchKernelGGL(colsum_kernel<T>, dim3(cb, (unsigned)slices), dim3(256), 0, st, rows,
                       cols, per, x, (const float *)nullptr, tmp);
    hipLaunchKernelGGL(colsum_kernel<float>, dim3(cb, 1), dim3(256), 0, st, slices, cols, slices,
                       (const float *)tmp, add, out);
    return hipGetLastError();
}
constexpr int64_t kSlices = 64;  // row slices of the first column-sum pass

// [X | Y] row by row: out[r][0:nx] = x[r], out[r][nx:nx+ny] = y[r] (bf16), or the
// reverse split of fp32 rows (unpack) -- to run the two narrow B and C products
// of the backward as one
__global__ void pack2_kernel(const int64_t rows, const int nx, const bf16 *__restrict__ x,
                             const bf16 *__restrict__ y, bf16 *__restrict__ out)
{
    const int w = 2 * nx;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * w;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / w;
        const int c = (int)(i - r * w);
        out[i] = c < nx ? x[r * nx + c] : y[r * nx + c - nx];
    }
}

__global__ void unpack2_kernel(const int64_t rows, const int nx, const float *__restrict__ in,
                               float *__restrict__ x, float *__restrict__ y)
{
    const int w = 2 * nx;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * w;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / w;
        const int c = (int)(i - r * w);
        (c < nx ? x[r * nx + c] : y[r * nx + c - nx]) = in[i];
    }
}

struct MixerBwdPlan {
    MixerPlan f;
    size_t off_ck, off_dy, off_dub, off_dz, off_da, off_db, off_dB, off_dC, off_dwb, off_dcsb,
        off_dh, off_du, off_ones, off_dwp, off_bws, off_dBC, off_WBC, off_gBC, bytes;
    int nseg;
};

static MixerBwdPlan mixer_bwd_plan(int64_t Bt, int64_t L, int64_t Di, int64_t N)
{
    MixerBwdPlan m{};
    m.f = mixer_plan(Bt, L, Di, N);
    const size_t act = up256((size_t)(Bt * L * Di) * 2), tok = up256((size_t)(Bt * L * N) * 2);
    m.nseg = (int)((L + kSegB - 1) / kSegB);
    size_t o = m.f.bytes;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += up256(bytes);
        return at;
    };
    m.off_dy = take(act);
    m.off_dub = take(act);
    m.off_dz = take(act);
    m.off_da = take(act);
    m.off_db = take(act);
    m.off_dB = take(tok);
    m.off_dC = take(tok);
    m.off_dwb = take((size_t)Di * 16);
    m.off_dcsb = take((size_t)Bt * 3 * Di * 2);
    m.off_dh = take((size_t)(Bt * L * Di) * 4);
    m.off_du = take(act);
    m.off_ones = take((size_t)kSlices * Di * 16);  // column-sum partials (up to Di * 4 columns)
    m.off_dwp = take((size_t)Bt * m.nseg * Di * 16);
    m.off_bws = take(bwd_plan(Bt, L, Di, N, true).bytes);
    m.off_dBC = take((size_t)(Bt * L) * 2 * N * 2);  // [dB | dC] bf16 [T][2N]
    m.off_WBC = take((size_t)Di * 2 * N * 2);         // [W_B | W_C] bf16 [Di][2N]
    m.off_gBC = take((size_t)Di * 2 * N * 4);         // [dW_B | dW_C] fp32 [Di][2N]
    m.bytes = o;
    return m;
}

size_t mixer_bwd_ws_bytes(int64_t Bt, int64_t L, int64_t Di, int64_t N)
{
    return mixer_bwd_plan(Bt, L, Di, N).bytes;
}

// forward part shared by both directions: u, z, h, a, b, B, C, y (+ checkpoints)
static const char *mixer_forward_pass(const MixerArgs &g, const MixerPlan &m, float *ckpt,
                                      hipStream_t st)
{
    char *ws = (char *)g.ws;
    void *u = ws + m.off_u, *z = ws + m.off_z, *h = ws + m.off_h, *a = ws + m.off_a,
         *b = ws + m.off_b, *y = ws + m.off_y, *B = ws + m.off_B, *C = ws + m.off_C;
    void *gws = ws + m.off_g;
    const int64_t T = g.Bt * g.L;
    const char *e;
    if ((e = gemm(st, T, g.Di, g.dm, g.xn, g.W_u, nullptr, nullptr, u, gws))) return e;
    if ((e = gemm(st, T, g.Di, g.dm, g.xn, g.W_z, nullptr, nullptr, z, gws))) return e;
    if (launch_conv_silu(g.Bt, g.L, g.Di, u, g.conv_w, g.conv_state, h, st) != hipSuccess)
        return "conv + SiLU launch failed";
    if ((e = gemm(st, T, g.Di, g.Di, h, g.W_a, g.a_bias, nullptr, a, gws))) return e;
    if ((e = gemm(st, T, g.Di, g.Di, h, g.W_b, g.b_bias, nullptr, b, gws))) return e;
    if ((e = gemm(st, T, g.N, g.Di, h, g.W_B, nullptr, nullptr, B, gws))) return e;
    if ((e = gemm(st, T, g.N, g.Di, h, g.W_C, nullptr, nullptr, C, gws))) return e;
    FwdArgs f{};
    f.io = NAJU_BF16;
    f.N = (int)g.N;
    f.block = true;
    f.Bt = g.Bt;
    f.L = g.L;
    f.Di = g.Di;
    f.scale = g.scale;
    f.hu = u;
    f.a = a;
    f.b = b;
    f.B = B;
    f.C = C;
    f.D = g.D;
    f.z = z;
    f.conv_w = g.conv_w;
    f.conv_state = g.conv_state;
    f.y = y;
    f.ckpt = ckpt;
    f.ws = ws + m.off_f;
    if (launch_fwd(f, st) != hipSuccess) return "block forward launch failed";
    return nullptr;
}

const char *mixer_bwd(const MixerArgs &g, const MixerGrads &d, hipStream_t st)
{
    const MixerBwdPlan m = mixer_bwd_plan(g.Bt, g.L, g.Di, g.N);
    char *ws = (char *)g.ws;
    const MixerPlan &f = m.f;
    // the forward's intermediates: those a naju_mixer_fwd call left in its own
    // workspace (same inputs), else recomputed into this one
    char *fw = d.saved ? (char *)d.saved : ws;
    void *u = fw + f.off_u, *z = fw + f.off_z, *h = fw + f.off_h, *a = fw + f.off_a,
         *b = fw + f.off_b, *y = fw + f.off_y, *B = fw + f.off_B, *C = fw + f.off_C;
    void *gws = ws + f.off_g;
    float *ck = (float *)(fw + f.off_ck);
    void *dy = ws + m.off_dy, *dub = ws + m.off_dub, *dz = ws + m.off_dz, *da = ws + m.off_da,
         *db = ws + m.off_db, *dB = ws + m.off_dB, *dC = ws + m.off_dC;
    float *dwb = (float *)(ws + m.off_dwb), *dh = (float *)(ws + m.off_dh);
    float *dwp = (float *)(ws + m.off_dwp);
    void *dcsb = ws + m.off_dcsb, *du = ws + m.off_du;
    float *csum = (float *)(ws + m.off_ones);
    const int64_t T = g.Bt * g.L;
    const bool want_dcs = g.conv_state && d.dconv_state;
    const char *e;
    if (!d.saved && (e = mixer_forward_pass(g, f, ck, st))) return e;
    // out = y W_out + res
    if ((e = gemm_nt(st, T, g.Di, g.dm, d.d_out, g.W_out, false, dy, HIP_R_16BF, gws))) return e;
    // (dh is free until the dh products below: the weight gradients' partials go there)
    const size_t dh_bytes = (size_t)T * g.Di * 4;
    if ((e = gemm_wgrad(st, T, g.dm, g.Di, y, d.d_out, d.dW_out, gws, dh, dh_bytes))) return e;
    // the block scan
    BwdArgs k{};
    k.io = NAJU_BF16;
    k.N = (int)g.N;
    k.block = true;
    k.Bt = g.Bt;
    k.L = g.L;
    k.Di = g.Di;
    k.scale = g.scale;
    k.hu = u;
    k.a = a;
    k.b = b;
    k.B = B;
    k.C = C;
    k.D = g.D;
    k.z = z;
    k.conv_w = g.conv_w;
    k.conv_state = g.conv_state;
    k.ckpt = ck;
    k.dy = dy;
    k.dhu = dub;
    k.da = da;
    k.db = db;
    k.dB = dB;
    k.dC = dC;
    k.dz = dz;
    k.dD = d.dD;
    k.dconv_w = dwb;
    k.dconv_state = want_dcs ? dcsb : nullptr;
    k.ws = ws + m.off_bws;
    if (launch_bwd(k, st) != hipSuccess) return "block backward launch failed";
    // a = h W_a + a_bias, b = h W_b + b_bias, B = h W_B, C = h W_C
    if ((e = gemm_nt(st, T, g.Di, g.Di, da, g.W_a, false, dh, HIP_R_32F, gws))) return e;
    if ((e = gemm_nt(st, T, g.Di, g.Di, db, g.W_b, true, dh, HIP_R_32F, gws))) return e;
    // the B and C terms as one product over [dB | dC] and [W_B | W_C] (each narrow
    // product would otherwise read and write all of dh, or read all of h)
    bf16 *dBC = (bf16 *)(ws + m.off_dBC), *WBC = (bf16 *)(ws + m.off_WBC);
    float *gBC = (float *)(ws + m.off_gBC);
    hipLaunchKernelGGL(pack2_kernel, dim3(1024), dim3(256), 0, st, T, (int)g.N,
                       (const bf16 *)dB, (const bf16 *)dC, dBC);
    hipLaunchKernelGGL(pack2_kernel, dim3(256), dim3(256), 0, st, g.Di, (int)g.N,
                       (const bf16 *)g.W_B, (const bf16 *)g.W_C, WBC);
    if (hipGetLastError() != hipSuccess) return "pack launch failed";
    if ((e = gemm_nt(st, T, g.Di, 2 * g.N, dBC, WBC, true, dh, HIP_R_32F, gws))) return e;
    // bias gradients: column sums of da and db (two fixed-order passes)
    if (colsum((const bf16 *)da, T, g.Di, nullptr, csum, kSlices, d.da_bias, st) != hipSuccess ||
        colsum((const bf16 *)db, T, g.Di, nullptr, csum, kSlices, d.db_bias, st) != hipSuccess)
        return "bias gradient launch failed";
    // h = SiLU(conv(u)) on the projection path, plus the scan's own du
    {
        const dim3 grid((unsigned)((g.Di / 8 + 63) / 64), (unsigned)m.nseg, (unsigned)g.Bt);
        hipLaunchKernelGGL(conv_silu_bwd_kernel, grid, dim3(64), 0, st, g.L, g.Di, m.nseg,
                           (const bf16 *)u, g.conv_w, (const bf16 *)g.conv_state, dh,
                           (const bf16 *)dub, (bf16 *)du, dwp,
                           want_dcs ? (const bf16 *)dcsb : nullptr,
                           want_dcs ? (bf16 *)d.dconv_state : nullptr);
        if (hipGetLastError() != hipSuccess) return "conv backward launch failed";
        // dconv_w = the scan's + the segments' partials ([segments][Di * 4])
        if (colsum((const float *)dwp, g.Bt * (int64_t)m.nseg, g.Di * 4, dwb, csum, kSlices,
                   d.dconv_w, st) != hipSuccess)
            return "dconv_w reduction launch failed";
    }
    // the gate and B, C projections' weight gradients (dh is free again: its
    // partials scratch)
    if ((e = gemm_wgrad(st, T, g.Di, g.Di, h, da, d.dW_a, gws, dh, dh_bytes))) return e;
    if ((e = gemm_wgrad(st, T, g.Di, g.Di, h, db, d.dW_b, gws, dh, dh_bytes))) return e;
    if ((e = gemm_wgrad(st, T, 2 * g.N, g.Di, h, dBC, gBC, gws, dh, dh_bytes))) return e;
    hipLaunchKernelGGL(unpack2_kernel, dim3(256), dim3(256), 0, st, g.Di, (int)g.N,
                       (const float *)gBC, d.dW_B, d.dW_C);
    if (hipGetLastError() != hipSuccess) return "unpack launch failed";
    // u = xn W_u, z = xn W_z
    if ((e = gemm_nt(st, T, g.dm, g.Di, du, g.W_u, false, d.dxn, HIP_R_32F, gws))) return e;
    if ((e = gemm_nt(st, T, g.dm, g.Di, dz, g.W_z, true, d.dxn, HIP_R_32F, gws))) return e;
    if ((e = gemm_wgrad(st, T, g.Di, g.dm, g.xn, du, d.dW_u, gws, dh, dh_bytes))) return e;
    if ((e = gemm_wgrad(st, T, g.Di, g.dm, g.xn, dz, d.dW_z, gws, dh, dh_bytes))) return e;
    return nullptr;
}

}  // namespace naju

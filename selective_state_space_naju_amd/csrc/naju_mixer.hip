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

#include <map>
#include <mutex>
#include <tuple>

#include "../../include/naju.h"
#include "naju_device.h"
#include "naju_launch.h"
#include "naju_mfma.h"

namespace naju {

// ------------------------------------------------------------ conv + SiLU
// Thread = (batch row, 8 channels, 16-token segment), one wave per workgroup:
// the segment's 16 rows (and the 3 rows before it) are loaded together, 16
// bytes per thread and row, then the 4-tap window slides in registers; a
// wave covers 64 x 16 consecutive bytes of a row.
constexpr int kSeg = 16;

__global__ __launch_bounds__(64) void conv_silu_kernel(const int64_t L, const int64_t Di,
                                                       const bf16 *__restrict__ u,
                                                       const float *__restrict__ w,
                                                       const bf16 *__restrict__ cs,
                                                       bf16 *__restrict__ h)
{
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + threadIdx.x) * 8;
    if (c0 >= Di) return;
    const int64_t n0 = (int64_t)blockIdx.y * kSeg;
    const int64_t bi = blockIdx.z;
    const bf16 *ub = u + bi * L * Di + c0;
    const int rows = (int)(L - n0 < kSeg ? L - n0 : kSeg);
    // h rows of the segment through a buffer whose range ends with the last
    // valid row: stores past the sequence end are dropped, no branch per row
    const rsrc_t rh = make_rsrc(h + (bi * L + n0) * Di, (uint32_t)rows * (uint32_t)Di * 2);
    // u at tokens n0-3 .. n0+kSeg-1, every load unconditional (rows past the end
    // re-read the last row and are never stored; rows before the sequence come
    // from conv_state, or are zero), so they are all in flight together
    uint4 q[kSeg + 3];
#pragma unroll
    for (int r = 0; r < kSeg + 3; ++r) {
        const int64_t m = n0 - 3 + r;
        const bf16 *src;
        if (m >= 0)
            src = ub + (m < L ? m : L - 1) * Di;
        else
            src = cs ? cs + (bi * 3 + (m + 3)) * Di + c0 : ub;
        q[r] = *(const uint4 *)src;
    }
#pragma unroll
    for (int r = 0; r < 3; ++r)
        if (n0 - 3 + r < 0 && !cs) q[r] = uint4{0u, 0u, 0u, 0u};
    float wk[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float4 v = *(const float4 *)(w + (c0 + e) * 4);
        wk[e][0] = v.x;
        wk[e][1] = v.y;
        wk[e][2] = v.z;
        wk[e][3] = v.w;
    }
    auto at = [&](int r, int c) -> float {  // channel c0 + c of row r
        const uint32_t p = c < 2 ? q[r].x : c < 4 ? q[r].y : c < 6 ? q[r].z : q[r].w;
        return __uint_as_float((c & 1) ? (p & 0xffff0000u) : (p << 16));
    };
#pragma unroll
    for (int t = 0; t < kSeg; ++t) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            float hv[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int c = e + k;
                const float pre = wk[c][0] * at(t, c) + wk[c][1] * at(t + 1, c) +
                                  wk[c][2] * at(t + 2, c) + wk[c][3] * at(t + 3, c);
                hv[k] = pre * sigm(pre);
            }
            o[e / 2] = (uint32_t)from_f<bf16>(hv[0]) | ((uint32_t)from_f<bf16>(hv[1]) << 16);
        }
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 ov = {o[0], o[1], o[2], o[3]};
        __builtin_amdgcn_raw_buffer_store_b128(ov, rh, (uint32_t)c0 * 2,
                                               (uint32_t)t * (uint32_t)Di * 2, 0);
    }
}

// ------------------------------------------------------------ GEMMs
// Row-major D[T][n] = A[T][k] W[k][n] (+ bias[n]) (+ C[T][n]) is, in the
// column-major terms of hipBLASLt, D^T (n x T) = W^T (n x k) A^T (k x T): W is
// the first operand with leading dimension n, A the second with leading
// dimension k, and the bias runs along D^T's rows.  Plans (layouts, epilogue,
// the heuristic's algorithm) are cached per device and shape.
struct GemmPlan {
    hipblasLtMatmulDesc_t md = nullptr;
    hipblasLtMatrixLayout_t lw = nullptr, la = nullptr, ld = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
    bool ok = false;
};

static std::mutex g_lt_mu;
static std::map<int, hipblasLtHandle_t> g_lt;
static std::map<std::tuple<int, int64_t, int64_t, int64_t, int>, GemmPlan> g_plans;

constexpr size_t kGemmWs = (size_t)32 << 20;  // hipBLASLt workspace inside ws

// Enqueues one projection.  Returns a message on failure (nullptr on success).
static const char *gemm(hipStream_t st, int64_t T, int64_t n, int64_t k, const void *A,
                        const void *W, const float *bias, const void *C, void *D, void *gws)
{
    if (T == 0 || n == 0) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return "hipGetDevice failed";
    std::lock_guard<std::mutex> lk(g_lt_mu);
    hipblasLtHandle_t &hd = g_lt[dev];
    if (!hd && hipblasLtCreate(&hd) != HIPBLAS_STATUS_SUCCESS) {
        hd = nullptr;
        return "hipblasLtCreate failed";
    }
    const int flags = (bias ? 1 : 0) | (C ? 2 : 0);
    GemmPlan &p = g_plans[std::make_tuple(dev, T, n, k, flags)];
    if (!p.ok) {
        if (hipblasLtMatmulDescCreate(&p.md, HIPBLAS_COMPUTE_32F, HIP_R_32F) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&p.lw, HIP_R_16BF, (uint64_t)n, (uint64_t)k, n) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, (uint64_t)k, (uint64_t)T, k) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&p.ld, HIP_R_16BF, (uint64_t)n, (uint64_t)T, n) !=
                HIPBLAS_STATUS_SUCCESS)
            return "hipBLASLt descriptor creation failed";
        const hipblasOperation_t opn = HIPBLAS_OP_N;
        hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSA, &opn, sizeof(opn));
        hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSB, &opn, sizeof(opn));
        if (bias) {
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
            hipblasLtMatmulAlgoGetHeuristic(hd, p.md, p.lw, p.la, p.ld, p.ld, pref, 1, res,
                                            &got) == HIPBLAS_STATUS_SUCCESS &&
            got > 0;
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        if (!found) return "hipBLASLt found no algorithm for a projection";
        // (the heuristic's first choice: timing its other candidates on the
        // 8 x 2048-token layer made single projections up to 6 % faster, but the
        // block scan after them as much slower, and the whole layer no faster;
        // it would also synchronise the stream on a shape's first call)
        const int best = 0;
        p.algo = res[best].algo;
        p.ws = res[best].workspaceSize;
        p.ok = true;
    }
    if (bias)
        hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias,
                                        sizeof(bias));
    const float one = 1.f, zero = 0.f;
    if (hipblasLtMatmul(hd, p.md, &one, W, p.lw, A, p.la, C ? &one : &zero, C ? C : D, p.ld, D,
                        p.ld, &p.algo, gws, p.ws, st) != HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatmul failed";
    return nullptr;
}

// ------------------------------------------------------------ layout of ws
// u, z, h, a, b, y [T][Di] bf16; B, C [T][N] bf16; the GEMM workspace; the
// block forward's own workspace -- each 256-byte aligned.
struct MixerPlan {
    size_t off_u, off_z, off_h, off_a, off_b, off_y, off_B, off_C, off_g, off_f, bytes;
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
    const dim3 grid((unsigned)((Di / 8 + 63) / 64), (unsigned)((L + kSeg - 1) / kSeg),
                    (unsigned)Bt);
    hipLaunchKernelGGL(conv_silu_kernel, grid, dim3(64), 0, st, L, Di, (const bf16 *)u, w,
                       (const bf16 *)cs, (bf16 *)h);
    return hipGetLastError();
}

const char *mixer_fwd(const MixerArgs &g, hipStream_t st)
{
    const MixerPlan m = mixer_plan(g.Bt, g.L, g.Di, g.N);
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
    f.ws = ws + m.off_f;
    if (launch_fwd(f, st) != hipSuccess) return "block forward launch failed";
    if ((e = gemm(st, T, g.dm, g.Di, y, g.W_out, nullptr, g.res, g.out, gws))) return e;
    return nullptr;
}

}  // namespace naju

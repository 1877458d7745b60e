// naju_api.hip -- the C ABI of libnaju.so (declared in include/naju.h).
//
// Validation happens before anything is enqueued; the kernels live in
// naju_fwd.hip and naju_bwd.hip.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/naju.h"
#include "naju_device.h"
#include "naju_launch.h"

namespace naju {

static thread_local char g_err[512] = "";

static naju_status_t fail(naju_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

static naju_status_t hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return NAJU_OK;
    return fail(NAJU_EHIP, "%s: %s", what, hipGetErrorString(e));
}

__global__ void zero_kernel(uint32_t *p, size_t n_words)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream)
{
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t *)p,
                       words);
    return hipGetLastError();
}

// seqlen == 0: x_final = x0 (or zeros), conv_state_out = conv_state (or zeros)
template <typename IO>
__global__ void empty_seq_kernel(int64_t n_state, int64_t n_conv, const float *x0,
                                 float *x_final, const IO *cs, IO *cso)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x_final && i < n_state) x_final[i] = x0 ? x0[i] : 0.f;
    if (cso && i < n_conv) cso[i] = cs ? cs[i] : from_f<IO>(0.f);
}

hipError_t launch_empty_seq(int io, int64_t Bt, int64_t Di, int64_t N, const float *x0,
                            float *x_final, const void *conv_state, void *conv_state_out,
                            hipStream_t stream)
{
    const int64_t ns = Bt * Di * N, nc = Bt * 3 * Di;
    const int64_t n = ns > nc ? ns : nc;
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (io == NAJU_F32)
        hipLaunchKernelGGL(empty_seq_kernel<float>, dim3(blocks), dim3(256), 0, stream, ns, nc,
                           x0, x_final, (const float *)conv_state, (float *)conv_state_out);
    else
        hipLaunchKernelGGL(empty_seq_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, ns, nc,
                           x0, x_final, (const bf16 *)conv_state, (bf16 *)conv_state_out);
    return hipGetLastError();
}

// --------------------------------------------------------------- validation
static naju_status_t check_dims(const naju_dims_t *d, bool block)
{
    if (!d) return fail(NAJU_EINVAL, "dims is NULL");
    if (d->batch < 0 || d->seqlen < 0 || d->d_inner < 0)
        return fail(NAJU_EINVAL, "negative size (batch=%lld seqlen=%lld d_inner=%lld)",
                    (long long)d->batch, (long long)d->seqlen, (long long)d->d_inner);
    if (d->io != NAJU_F32 && d->io != NAJU_BF16)
        return fail(NAJU_EINVAL, "io dtype %d is neither NAJU_F32 nor NAJU_BF16", (int)d->io);
    if (d->d_state <= 0) return fail(NAJU_EINVAL, "d_state must be positive");
    if (d->d_state != 16 && d->d_state != 64)
        return fail(NAJU_EUNSUPPORTED, "d_state %lld not built (16 and 64 are)",
                    (long long)d->d_state);
    if (block && d->d_conv != 4)
        return fail(d->d_conv <= 0 ? NAJU_EINVAL : NAJU_EUNSUPPORTED,
                    "d_conv %d not built (4 is)", (int)d->d_conv);
    // index arithmetic limits of the kernels
    const double toks = (double)d->batch * (double)d->seqlen * (double)d->d_inner;
    if (toks > 9.0e15) return fail(NAJU_EINVAL, "tensor too large");
    if (d->seqlen > (int64_t)1 << 40) return fail(NAJU_EINVAL, "seqlen too large");
    const FwdPlan p = fwd_plan(d->batch, d->seqlen, d->d_inner, d->d_state, kMfmaW);
    if ((double)p.n_wg >= 4.0e9) return fail(NAJU_EINVAL, "problem needs too many workgroups");
    return NAJU_OK;
}

static bool empty(const naju_dims_t *d) { return d->batch == 0 || d->d_inner == 0; }

static naju_status_t need(const void *p, const char *name, size_t align)
{
    if (!p) return fail(NAJU_EINVAL, "%s is NULL", name);
    if (((uintptr_t)p) % align) return fail(NAJU_EINVAL, "%s is not %zu-byte aligned", name, align);
    return NAJU_OK;
}

static naju_status_t opt(const void *p, const char *name, size_t align)
{
    if (p && ((uintptr_t)p) % align)
        return fail(NAJU_EINVAL, "%s is not %zu-byte aligned", name, align);
    return NAJU_OK;
}

#define TRY(x)                                                                                 \
    do {                                                                                       \
        naju_status_t _s = (x);                                                                \
        if (_s != NAJU_OK) return _s;                                                          \
    } while (0)

static size_t ws_bytes_for(naju_op_t op, const naju_dims_t *d)
{
    const bool block = (op == NAJU_OP_BLOCK_FWD || op == NAJU_OP_BLOCK_BWD);
    if (op == NAJU_OP_SCAN_FWD || op == NAJU_OP_BLOCK_FWD)
        return fwd_ws_bytes(d->batch, d->seqlen, d->d_inner, d->d_state);
    return bwd_plan(d->batch, d->seqlen, d->d_inner, d->d_state, block).bytes;
}

static naju_status_t check_ws(naju_op_t op, const naju_dims_t *d, const void *ws, size_t bytes)
{
    const size_t need_b = ws_bytes_for(op, d);
    if (!ws) return fail(NAJU_EWORKSPACE, "workspace is NULL (needs %zu bytes)", need_b);
    if (((uintptr_t)ws) % 256) return fail(NAJU_EINVAL, "workspace is not 256-byte aligned");
    if (bytes < need_b)
        return fail(NAJU_EWORKSPACE, "workspace has %zu bytes, needs %zu", bytes, need_b);
    return NAJU_OK;
}

// The forward's argument checks other than the workspace's.
static naju_status_t fwd_check(bool block, const naju_dims_t *d, const void *hu, const void *z,
                               const float *conv_w, const void *conv_state, const void *a,
                               const void *b, const void *B, const void *C, const float *D,
                               const float *x0, const void *y, const float *x_final,
                               const void *conv_state_out, const float *ckpt)
{
    TRY(check_dims(d, block));
    const size_t e = d->io == NAJU_F32 ? 4 : 2;
    if (empty(d)) return NAJU_OK;
    if (d->seqlen > 0) {
        TRY(need(hu, block ? "u" : "h", e));
        TRY(need(a, "a", e));
        TRY(need(b, "b", e));
        TRY(need(B, "B", e));
        TRY(need(C, "C", e));
        TRY(need(D, "D", 4));
        TRY(need(y, "y", e));
        if (block) {
            TRY(need(z, "z", e));
            TRY(need(conv_w, "conv_w", 4));
        }
    }
    TRY(opt(x0, "x0", 4));
    TRY(opt(x_final, "x_final", 4));
    TRY(opt(ckpt, "ckpt", 4));
    if (block) {
        TRY(opt(conv_state, "conv_state", e));
        TRY(opt(conv_state_out, "conv_state_out", e));
    }
    return NAJU_OK;
}

static naju_status_t fwd_common(bool block, const naju_dims_t *d, const void *hu, const void *z,
                                const float *conv_w, const void *conv_state, const void *a,
                                const void *b, const void *B, const void *C, const float *D,
                                const float *x0, void *y, float *x_final, void *conv_state_out,
                                float *ckpt, void *ws, size_t ws_bytes, void *stream)
{
    TRY(fwd_check(block, d, hu, z, conv_w, conv_state, a, b, B, C, D, x0, y, x_final,
                  conv_state_out, ckpt));
    if (empty(d)) return NAJU_OK;
    const bool has_tok = d->seqlen > 0;
    if (has_tok) TRY(check_ws(block ? NAJU_OP_BLOCK_FWD : NAJU_OP_SCAN_FWD, d, ws, ws_bytes));
    hipStream_t st = (hipStream_t)stream;
    if (!has_tok)
        return hip_status(launch_empty_seq(d->io, d->batch, d->d_inner, d->d_state, x0, x_final,
                                           block ? conv_state : nullptr,
                                           block ? conv_state_out : nullptr, st),
                          "empty-sequence launch");
    FwdArgs g{};
    g.io = d->io;
    g.N = (int)d->d_state;
    g.block = block;
    g.Bt = d->batch;
    g.L = d->seqlen;
    g.Di = d->d_inner;
    g.scale = (float)(1.0 / sqrt((double)d->d_state));
    g.hu = hu;
    g.a = a;
    g.b = b;
    g.B = B;
    g.C = C;
    g.D = D;
    g.x0 = x0;
    g.z = z;
    g.conv_w = conv_w;
    g.conv_state = conv_state;
    g.y = y;
    g.x_final = x_final;
    g.conv_state_out = conv_state_out;
    g.ckpt = ckpt;
    g.ws = ws;
    return hip_status(launch_fwd(g, st), "forward launch");
}

static naju_status_t bwd_common(bool block, const naju_dims_t *d, const void *hu, const void *z,
                                const float *conv_w, const void *conv_state, const void *a,
                                const void *b, const void *B, const void *C, const float *D,
                                const float *x0, const float *ckpt, const void *dy,
                                const float *dx_final, void *dhu, void *dz, float *dconv_w,
                                void *dconv_state, void *da, void *db, void *dB, void *dC,
                                float *dD, float *dx0, void *ws, size_t ws_bytes, void *stream)
{
    TRY(check_dims(d, block));
    const naju_op_t op = block ? NAJU_OP_BLOCK_BWD : NAJU_OP_SCAN_BWD;
    const size_t e = d->io == NAJU_F32 ? 4 : 2;
    if (empty(d)) return NAJU_OK;
    hipStream_t st = (hipStream_t)stream;
    TRY(need(D, "D", 4));
    TRY(need(dD, "dD", 4));
    if (block) TRY(need(dconv_w, "dconv_w", 4));
    TRY(opt(x0, "x0", 4));
    TRY(opt(dx_final, "dx_final", 4));
    TRY(opt(dx0, "dx0", 4));
    TRY(opt(ckpt, "ckpt", 4));
    if (block) {
        TRY(need(conv_w, "conv_w", 4));
        TRY(opt(conv_state, "conv_state", e));
        TRY(opt(dconv_state, "dconv_state", e));
    }
    if (d->seqlen == 0) {
        // no tokens: dx0 = dx_final, zero parameter gradients, dconv_state = 0
        hipError_t er = launch_zero(dD, (size_t)d->d_inner * 4, st);
        if (er == hipSuccess && block) er = launch_zero(dconv_w, (size_t)d->d_inner * 16, st);
        if (er == hipSuccess && block && dconv_state)
            er = launch_zero(dconv_state, (size_t)d->batch * 3 * d->d_inner * e, st);
        if (er == hipSuccess)
            er = launch_empty_seq(d->io, d->batch, d->d_inner, d->d_state, dx_final, dx0,
                                  nullptr, nullptr, st);
        return hip_status(er, "empty-sequence launch");
    }
    TRY(need(hu, block ? "u" : "h", e));
    TRY(need(a, "a", e));
    TRY(need(b, "b", e));
    TRY(need(B, "B", e));
    TRY(need(C, "C", e));
    TRY(need(dy, "dy", e));
    TRY(need(dhu, block ? "du" : "dh", e));
    TRY(need(da, "da", e));
    TRY(need(db, "db", e));
    TRY(need(dB, "dB", e));
    TRY(need(dC, "dC", e));
    if (block) {
        TRY(need(z, "z", e));
        TRY(need(dz, "dz", e));
    }
    TRY(check_ws(op, d, ws, ws_bytes));

    const BwdPlan pl = bwd_plan(d->batch, d->seqlen, d->d_inner, d->d_state, block);
    const float scale = (float)(1.0 / sqrt((double)d->d_state));
    if (!ckpt) {
        // recompute the checkpoints with a forward pass that writes no output
        FwdArgs f{};
        f.io = d->io;
        f.N = (int)d->d_state;
        f.block = block;
        f.Bt = d->batch;
        f.L = d->seqlen;
        f.Di = d->d_inner;
        f.scale = scale;
        f.hu = hu;
        f.a = a;
        f.b = b;
        f.B = B;
        f.C = C;
        f.D = D;
        f.x0 = x0;
        f.z = z;
        f.conv_w = conv_w;
        f.conv_state = conv_state;
        f.ckpt = (float *)((char *)ws + pl.off_ckpt);
        f.ws = (char *)ws + pl.off_fwd;
        TRY(hip_status(launch_fwd(f, st), "checkpoint forward launch"));
        ckpt = f.ckpt;
    }
    BwdArgs g{};
    g.io = d->io;
    g.N = (int)d->d_state;
    g.block = block;
    g.Bt = d->batch;
    g.L = d->seqlen;
    g.Di = d->d_inner;
    g.scale = scale;
    g.hu = hu;
    g.a = a;
    g.b = b;
    g.B = B;
    g.C = C;
    g.D = D;
    g.x0 = x0;
    g.z = z;
    g.conv_w = conv_w;
    g.conv_state = conv_state;
    g.ckpt = ckpt;
    g.dy = dy;
    g.dx_final = dx_final;
    g.dhu = dhu;
    g.da = da;
    g.db = db;
    g.dB = dB;
    g.dC = dC;
    g.dz = dz;
    g.dD = dD;
    g.dx0 = dx0;
    g.dconv_w = dconv_w;
    g.dconv_state = dconv_state;
    g.ws = ws;
    return hip_status(launch_bwd(g, st), "backward launch");
}

static naju_status_t mixer_common(const naju_dims_t *d, int64_t dm, const void *xn,
                                  const void *res, const void *W_u, const void *W_z,
                                  const float *conv_w, const void *conv_state, const void *W_a,
                                  const float *a_bias, const void *W_b, const float *b_bias,
                                  const void *W_B, const void *W_C, const float *D,
                                  const void *W_out, void *out, const MixerGrads *grads,
                                  void *ws, size_t ws_bytes, void *stream)
{
    TRY(check_dims(d, true));
    if (d->io != NAJU_BF16) return fail(NAJU_EUNSUPPORTED, "the mixer is built for bf16 io only");
    if (dm <= 0 || d->d_inner <= 0)
        return fail(NAJU_EINVAL, "d_model and d_inner must be positive (d_model=%lld d_inner=%lld)",
                    (long long)dm, (long long)d->d_inner);
    if (dm % 8 || d->d_inner % 8)
        return fail(NAJU_EUNSUPPORTED, "d_model and d_inner must be multiples of 8");
    if (dm > ((int64_t)1 << 24) || d->d_inner >= ((int64_t)1 << 24))
        return fail(NAJU_EINVAL, "d_model or d_inner too large");
    if (d->batch > 65535 || (d->seqlen + 15) / 16 > 65535)
        return fail(NAJU_EINVAL, "batch or seqlen too large for the mixer's conv launch");
    if (d->batch == 0 || d->seqlen == 0) return NAJU_OK;
    TRY(need(xn, "xn", 16));
    TRY(opt(res, "res", 16));
    TRY(need(W_u, "W_u", 16));
    TRY(need(W_z, "W_z", 16));
    TRY(need(conv_w, "conv_w", 16));
    TRY(opt(conv_state, "conv_state", 16));
    TRY(need(W_a, "W_a", 16));
    TRY(need(a_bias, "a_bias", 4));
    TRY(need(W_b, "W_b", 16));
    TRY(need(b_bias, "b_bias", 4));
    TRY(need(W_B, "W_B", 16));
    TRY(need(W_C, "W_C", 16));
    TRY(need(D, "D", 4));
    TRY(need(W_out, "W_out", 16));
    const size_t need_b = grads ? mixer_bwd_ws_bytes(d->batch, d->seqlen, d->d_inner, d->d_state)
                                : mixer_ws_bytes(d->batch, d->seqlen, d->d_inner, d->d_state);
    if (!ws) return fail(NAJU_EWORKSPACE, "workspace is NULL (needs %zu bytes)", need_b);
    if (((uintptr_t)ws) % 256) return fail(NAJU_EINVAL, "workspace is not 256-byte aligned");
    if (ws_bytes < need_b)
        return fail(NAJU_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need_b);
    if (grads) {
        const MixerGrads &q = *grads;
        TRY(need(q.d_out, "d_out", 16));
        TRY(need(q.dxn, "dxn", 16));
        TRY(need(q.dW_u, "dW_u", 16));
        TRY(need(q.dW_z, "dW_z", 16));
        TRY(need(q.dconv_w, "dconv_w", 16));
        TRY(opt(q.dconv_state, "dconv_state", 16));
        TRY(need(q.dW_a, "dW_a", 16));
        TRY(need(q.da_bias, "da_bias", 16));
        TRY(need(q.dW_b, "dW_b", 16));
        TRY(need(q.db_bias, "db_bias", 16));
        TRY(need(q.dW_B, "dW_B", 16));
        TRY(need(q.dW_C, "dW_C", 16));
        TRY(need(q.dD, "dD", 4));
        TRY(need(q.dW_out, "dW_out", 16));
    } else {
        TRY(need(out, "out", 16));
    }
    MixerArgs g{};
    g.Bt = d->batch;
    g.L = d->seqlen;
    g.dm = dm;
    g.Di = d->d_inner;
    g.N = d->d_state;
    g.scale = (float)(1.0 / sqrt((double)d->d_state));
    g.xn = xn;
    g.res = res;
    g.W_u = W_u;
    g.W_z = W_z;
    g.conv_w = conv_w;
    g.conv_state = conv_state;
    g.W_a = W_a;
    g.b_bias = b_bias;
    g.a_bias = a_bias;
    g.W_b = W_b;
    g.W_B = W_B;
    g.W_C = W_C;
    g.D = D;
    g.W_out = W_out;
    g.out = out;
    g.ws = ws;
    const char *e = grads ? mixer_bwd(g, *grads, (hipStream_t)stream)
                          : mixer_fwd(g, (hipStream_t)stream);
    if (e) return fail(NAJU_EHIP, "mixer: %s", e);
    return NAJU_OK;
}

// ---------------------------------------------- allocation-free scan forward
// A device-resident scratch array serves as the workspace of
// naju_scan_fwd_noalloc: zero at load (so, like a zero-filled caller workspace,
// it needs no initialisation), epoch-tagged words and self-resetting counters
// keep it reusable across calls of any shape.  Each GPU holds its own copy of
// the array, at its own address, until the process ends.  In host code the
// array's name is not a device address: the kernels take the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

// the error word read back (and cleared) after a call, for the caller
__global__ void scratch_flags_kernel(WsHeader *hdr, uint32_t *flags)
{
    *flags = hdr->error;
    hdr->error = 0u;
}

static naju_status_t scratch_address(void **out)
{
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
    if (dev < 0 || dev >= 64) return fail(NAJU_EUNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        // (once per device, with that device current)
        TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress"));
        if (!p) return fail(NAJU_EHIP, "hipGetSymbolAddress returned NULL");
        addr[dev] = p;
    }
    *out = addr[dev];
    return NAJU_OK;
}

}  // namespace naju

using namespace naju;

extern "C" {

naju_status_t naju_scan_fwd_noalloc(const naju_dims_t *dims, const void *h, const void *a,
                                    const void *b, const void *B, const void *C, const float *D,
                                    const float *x0, void *y, float *x_final, float *ckpt,
                                    uint32_t *flags, void *stream)
{
    TRY(check_dims(dims, false));
    const size_t need_b = ws_bytes_for(NAJU_OP_SCAN_FWD, dims);
    if (need_b > kScratchBytes)
        return fail(NAJU_EWORKSPACE,
                    "naju_scan_fwd_noalloc: this shape needs %zu bytes of scratch, more than "
                    "the library's %zu; use naju_scan_fwd with a workspace",
                    need_b, kScratchBytes);
    TRY(opt(flags, "flags", 4));
    // every argument is checked before the device is queried
    TRY(fwd_check(false, dims, h, nullptr, nullptr, nullptr, a, b, B, C, D, x0, y, x_final,
                  nullptr, ckpt));
    void *ws = nullptr;
    TRY(scratch_address(&ws));
    TRY(fwd_common(false, dims, h, nullptr, nullptr, nullptr, a, b, B, C, D, x0, y, x_final,
                   nullptr, ckpt, ws, kScratchBytes, stream));
    if (flags) {
        hipLaunchKernelGGL(scratch_flags_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream,
                           (WsHeader *)ws, flags);
        TRY(hip_status(hipGetLastError(), "scratch flags launch"));
    }
    return NAJU_OK;
}

size_t naju_workspace_bytes(naju_op_t op, const naju_dims_t *dims)
{
    const bool block = (op == NAJU_OP_BLOCK_FWD || op == NAJU_OP_BLOCK_BWD);
    if (op < NAJU_OP_SCAN_FWD || op > NAJU_OP_BLOCK_BWD) return 0;
    if (check_dims(dims, block) != NAJU_OK) return 0;
    return ws_bytes_for(op, dims);
}

size_t naju_ckpt_bytes(const naju_dims_t *dims)
{
    if (check_dims(dims, false) != NAJU_OK) return 0;
    return ckpt_bytes(dims->batch, dims->seqlen, dims->d_inner, dims->d_state);
}

naju_status_t naju_workspace_init(void *ws, size_t ws_bytes, void *stream)
{
    if (!ws) return fail(NAJU_EWORKSPACE, "workspace is NULL");
    if (((uintptr_t)ws) % 256) return fail(NAJU_EINVAL, "workspace is not 256-byte aligned");
    return hip_status(launch_zero(ws, ws_bytes, (hipStream_t)stream), "workspace zero fill");
}

naju_status_t naju_workspace_check(const void *ws, size_t ws_bytes, void *stream,
                                   uint32_t *flags)
{
    if (!ws || ws_bytes < sizeof(WsHeader)) return fail(NAJU_EWORKSPACE, "workspace too small");
    if (!flags) return fail(NAJU_EINVAL, "flags is NULL");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) {
        WsHeader h;
        e = hipMemcpy(&h, ws, sizeof(h), hipMemcpyDeviceToHost);
        if (e == hipSuccess) *flags = h.error;
    }
    return hip_status(e, "workspace check");
}

// ------------------------------------------------------------ decode step
static naju_status_t step_common(bool block, const naju_dims_t *d, const void *hu, const void *z,
                                 const float *conv_w, void *conv_state, const void *a,
                                 const void *b, const void *B, const void *C, const float *D,
                                 float *x, void *y, void *stream)
{
    TRY(check_dims(d, block));
    if (empty(d)) return NAJU_OK;
    const size_t e = d->io == NAJU_F32 ? 4 : 2;
    TRY(need(hu, block ? "u" : "h", e));
    TRY(need(a, "a", e));
    TRY(need(b, "b", e));
    TRY(need(B, "B", e));
    TRY(need(C, "C", e));
    TRY(need(D, "D", 4));
    TRY(need(x, "x", 16));
    TRY(need(y, "y", e));
    if (block) {
        TRY(need(z, "z", e));
        TRY(need(conv_w, "conv_w", 4));
        TRY(need(conv_state, "conv_state", e));
    }
    if (d->batch > 65535) return fail(NAJU_EINVAL, "batch %lld too large for a step (65535 max)",
                                      (long long)d->batch);
    StepArgs g{};
    g.io = d->io;
    g.N = (int)d->d_state;
    g.block = block;
    g.Bt = d->batch;
    g.Di = d->d_inner;
    g.scale = (float)(1.0 / sqrt((double)d->d_state));
    g.hu = hu;
    g.a = a;
    g.b = b;
    g.B = B;
    g.C = C;
    g.D = D;
    g.z = z;
    g.conv_w = conv_w;
    g.conv_state = conv_state;
    g.x = x;
    g.y = y;
    return hip_status(launch_step(g, (hipStream_t)stream), "step launch");
}

naju_status_t naju_scan_step(const naju_dims_t *dims, const void *h, const void *a, const void *b,
                             const void *B, const void *C, const float *D, float *x, void *y,
                             void *stream)
{
    return step_common(false, dims, h, nullptr, nullptr, nullptr, a, b, B, C, D, x, y, stream);
}

naju_status_t naju_block_step(const naju_dims_t *dims, const void *u, const void *z,
                              const float *conv_w, void *conv_state, const void *a, const void *b,
                              const void *B, const void *C, const float *D, float *x, void *y,
                              void *stream)
{
    return step_common(true, dims, u, z, conv_w, conv_state, a, b, B, C, D, x, y, stream);
}

naju_status_t naju_scan_fwd(const naju_dims_t *dims, const void *h, const void *a,
                            const void *b, const void *B, const void *C, const float *D,
                            const float *x0, void *y, float *x_final, float *ckpt, void *ws,
                            size_t ws_bytes, void *stream)
{
    return fwd_common(false, dims, h, nullptr, nullptr, nullptr, a, b, B, C, D, x0, y, x_final,
                      nullptr, ckpt, ws, ws_bytes, stream);
}

naju_status_t naju_block_fwd(const naju_dims_t *dims, const void *u, const void *z,
                             const float *conv_w, const void *conv_state, const void *a,
                             const void *b, const void *B, const void *C, const float *D,
                             const float *x0, void *y, float *x_final, void *conv_state_out,
                             float *ckpt, void *ws, size_t ws_bytes, void *stream)
{
    return fwd_common(true, dims, u, z, conv_w, conv_state, a, b, B, C, D, x0, y, x_final,
                      conv_state_out, ckpt, ws, ws_bytes, stream);
}

size_t naju_mixer_workspace_bytes(const naju_dims_t *dims, int64_t d_model)
{
    if (check_dims(dims, true) != NAJU_OK || d_model <= 0) return 0;
    return mixer_ws_bytes(dims->batch, dims->seqlen, dims->d_inner, dims->d_state);
}

naju_status_t naju_mixer_fwd(const naju_dims_t *dims, int64_t d_model, const void *xn,
                             const void *res, const void *W_u, const void *W_z,
                             const float *conv_w, const void *conv_state, const void *W_a,
                             const float *a_bias, const void *W_b, const float *b_bias,
                             const void *W_B, const void *W_C, const float *D,
                             const void *W_out, void *out, void *ws, size_t ws_bytes,
                             void *stream)
{
    return mixer_common(dims, d_model, xn, res, W_u, W_z, conv_w, conv_state, W_a, a_bias, W_b,
                        b_bias, W_B, W_C, D, W_out, out, nullptr, ws, ws_bytes, stream);
}

size_t naju_mixer_bwd_workspace_bytes(const naju_dims_t *dims, int64_t d_model)
{
    if (check_dims(dims, true) != NAJU_OK || d_model <= 0) return 0;
    return mixer_bwd_ws_bytes(dims->batch, dims->seqlen, dims->d_inner, dims->d_state);
}

naju_status_t naju_mixer_bwd(const naju_dims_t *dims, int64_t d_model, const void *xn,
                             const void *W_u, const void *W_z, const float *conv_w,
                             const void *conv_state, const void *W_a, const float *a_bias,
                             const void *W_b, const float *b_bias, const void *W_B,
                             const void *W_C, const float *D, const void *W_out,
                             const void *d_out, float *dxn, float *dW_u, float *dW_z,
                             float *dconv_w, void *dconv_state, float *dW_a, float *da_bias,
                             float *dW_b, float *db_bias, float *dW_B, float *dW_C, float *dD,
                             float *dW_out, const void *fwd_ws, size_t fwd_ws_bytes, void *ws,
                             size_t ws_bytes, void *stream)
{
    if (fwd_ws) {
        if (check_dims(dims, true) != NAJU_OK) return check_dims(dims, true);
        const size_t nf = mixer_ws_bytes(dims->batch, dims->seqlen, dims->d_inner, dims->d_state);
        if (((uintptr_t)fwd_ws) % 256) return fail(NAJU_EINVAL, "fwd_ws is not 256-byte aligned");
        if (fwd_ws_bytes < nf)
            return fail(NAJU_EWORKSPACE, "fwd_ws has %zu bytes, a forward workspace needs %zu",
                        fwd_ws_bytes, nf);
    }
    MixerGrads q{};
    q.d_out = d_out;
    q.saved = fwd_ws;
    q.dxn = dxn;
    q.dW_u = dW_u;
    q.dW_z = dW_z;
    q.dconv_w = dconv_w;
    q.dconv_state = dconv_state;
    q.dW_a = dW_a;
    q.da_bias = da_bias;
    q.dW_b = dW_b;
    q.db_bias = db_bias;
    q.dW_B = dW_B;
    q.dW_C = dW_C;
    q.dD = dD;
    q.dW_out = dW_out;
    return mixer_common(dims, d_model, xn, nullptr, W_u, W_z, conv_w, conv_state, W_a, a_bias,
                        W_b, b_bias, W_B, W_C, D, W_out, nullptr, &q, ws, ws_bytes, stream);
}

naju_status_t naju_scan_bwd(const naju_dims_t *dims, const void *h, const void *a,
                            const void *b, const void *B, const void *C, const float *D,
                            const float *x0, const float *ckpt, const void *dy,
                            const float *dx_final, void *dh, void *da, void *db, void *dB,
                            void *dC, float *dD, float *dx0, void *ws, size_t ws_bytes,
                            void *stream)
{
    return bwd_common(false, dims, h, nullptr, nullptr, nullptr, a, b, B, C, D, x0, ckpt, dy,
                      dx_final, dh, nullptr, nullptr, nullptr, da, db, dB, dC, dD, dx0, ws,
                      ws_bytes, stream);
}

naju_status_t naju_block_bwd(const naju_dims_t *dims, const void *u, const void *z,
                             const float *conv_w, const void *conv_state, const void *a,
                             const void *b, const void *B, const void *C, const float *D,
                             const float *x0, const float *ckpt, const void *dy,
                             const float *dx_final, void *du, void *dz, float *dconv_w,
                             void *dconv_state, void *da, void *db, void *dB, void *dC,
                             float *dD, float *dx0, void *ws, size_t ws_bytes, void *stream)
{
    return bwd_common(true, dims, u, z, conv_w, conv_state, a, b, B, C, D, x0, ckpt, dy,
                      dx_final, du, dz, dconv_w, dconv_state, da, db, dB, dC, dD, dx0, ws,
                      ws_bytes, stream);
}

const char *naju_last_error(void) { return g_err; }

const char *naju_version(void) { return "naju-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"

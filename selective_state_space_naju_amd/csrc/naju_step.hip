// naju_step.hip -- one-token (streaming decode) step of the Naju selective scan
// and of its block, with the state carried in place.
//
// Same recurrence and readout as the sequence kernels ("Core equations" of the
// Naju reproduction README, arXiv 2607.21000), for a single token per call:
//     x[c,s] <- sigma(a[c]) x[c,s] + sigma(b[c]) h[c] B[s]
//     y[c]    = (1/sqrt(N)) sum_s x[c,s] C[s] + D[c] h[c]
// and for the block h = SiLU(conv(u)) over the carried conv window, y *= SiLU(z).
//
// A call reads and writes the state once (Bt * Di * N * 8 bytes, 16 bytes per
// lane per access) and touches each activation once: a few microseconds of
// HBM traffic even at large batch, so the kernel is laid out for coalescing
// and a single pass rather than for arithmetic.  One thread per (batch row,
// channel); a workgroup covers 256 channels of one batch row and stages that
// row's B and C in LDS.
#include "naju_device.h"
#include "naju_launch.h"

namespace naju {

template <typename IO, int N, bool BLOCK>
__global__ __launch_bounds__(256) void step_kernel(
    const int64_t Di, const float scale, const IO *__restrict__ hu, const IO *__restrict__ z,
    const float *__restrict__ conv_w, IO *__restrict__ conv_state, const IO *__restrict__ a,
    const IO *__restrict__ bg, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
    const float *__restrict__ D, float *__restrict__ x, IO *__restrict__ y)
{
    __shared__ float sB[N], sC[N];
    const int64_t bi = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (threadIdx.x < N) {
        sB[threadIdx.x] = to_f(Bm[bi * N + threadIdx.x]);
        sC[threadIdx.x] = to_f(Cm[bi * N + threadIdx.x]);
    }
    __syncthreads();
    if (c >= Di) return;
    const int64_t t = bi * Di + c;  // (batch row, channel) of the [Bt][Di] activations
    float h;
    if (BLOCK) {
        // window u_{-3}, u_{-2}, u_{-1} (carried) and u_0; the carried window
        // shifts by one token
        IO *cs = conv_state + bi * 3 * Di + c;
        const float u0 = to_f(hu[t]);
        const float um3 = to_f(cs[0]), um2 = to_f(cs[Di]), um1 = to_f(cs[2 * Di]);
        const float pre = conv_w[c * 4 + 0] * um3 + conv_w[c * 4 + 1] * um2 +
                          conv_w[c * 4 + 2] * um1 + conv_w[c * 4 + 3] * u0;
        h = pre * sigm(pre);
        cs[0] = cs[Di];
        cs[Di] = cs[2 * Di];
        cs[2 * Di] = hu[t];
    } else {
        h = to_f(hu[t]);
    }
    const float f = sigm(to_f(a[t]));
    const float w = sigm(to_f(bg[t])) * h;
    float4 *xs = (float4 *)(x + t * N);
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        float4 v = xs[q];
        v.x = fmaf(f, v.x, w * sB[4 * q + 0]);
        v.y = fmaf(f, v.y, w * sB[4 * q + 1]);
        v.z = fmaf(f, v.z, w * sB[4 * q + 2]);
        v.w = fmaf(f, v.w, w * sB[4 * q + 3]);
        acc = fmaf(v.x, sC[4 * q + 0], acc);
        acc = fmaf(v.y, sC[4 * q + 1], acc);
        acc = fmaf(v.z, sC[4 * q + 2], acc);
        acc = fmaf(v.w, sC[4 * q + 3], acc);
        xs[q] = v;
    }
    float yv = fmaf(scale, acc, D[c] * h);
    if (BLOCK) {
        const float zv = to_f(z[t]);
        yv *= zv * sigm(zv);
    }
    y[t] = from_f<IO>(yv);
}

template <typename IO, int N>
static hipError_t launch_step_t(const StepArgs &g, hipStream_t stream)
{
    const dim3 grid((unsigned)((g.Di + 255) / 256), (unsigned)g.Bt);
    if (g.block)
        hipLaunchKernelGGL((step_kernel<IO, N, true>), grid, dim3(256), 0, stream, g.Di, g.scale,
                           (const IO *)g.hu, (const IO *)g.z, g.conv_w, (IO *)g.conv_state,
                           (const IO *)g.a, (const IO *)g.b, (const IO *)g.B, (const IO *)g.C,
                           g.D, g.x, (IO *)g.y);
    else
        hipLaunchKernelGGL((step_kernel<IO, N, false>), grid, dim3(256), 0, stream, g.Di, g.scale,
                           (const IO *)g.hu, (const IO *)nullptr, (const float *)nullptr,
                           (IO *)nullptr, (const IO *)g.a, (const IO *)g.b, (const IO *)g.B,
                           (const IO *)g.C, g.D, g.x, (IO *)g.y);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &g, hipStream_t stream)
{
    if (g.io == 0) return g.N == 16 ? launch_step_t<float, 16>(g, stream) : launch_step_t<float, 64>(g, stream);
    return g.N == 16 ? launch_step_t<bf16, 16>(g, stream) : launch_step_t<bf16, 64>(g, stream);
}

}  // namespace naju

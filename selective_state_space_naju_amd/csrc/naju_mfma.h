// naju_mfma.h -- matrix-core and buffer helpers shared by the chunk kernels of
// libnaju (gfx950): the 32x32x16 bf16 MFMA, bf16 hi + lo operand splits, raw
// buffer descriptors, the lane-half exchange and the forward's HBM -> LDS copy.
#pragma once

#include "naju_device.h"

namespace naju {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// D (32x32, fp32) += A (32x16, bf16) B (16x32, bf16).  Operand lane l holds
// row / column l%32 and K-slots 8(l/32) .. 8(l/32)+7; accumulator lane l holds
// column l%32 and rows 8q + 4(l/32) + r (q, r = 0..3) in elements 4q + r.
__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 as_bf(bf16 v) { return __builtin_bit_cast(__bf16, v); }

constexpr uint32_t kOOB = 0x80000000u;  // a buffer offset past every range used here

// Raw buffer over [p, p + bytes): loads past the end read 0, stores past the end
// are dropped.  On gfx950 the range check of a stride-0 buffer covers the whole
// offset (voffset + soffset + the immediate offset), dword by dword for wider
// accesses.  The kernels still put every offset that must be range-checked (row
// offsets included) into voffset, and a nonzero soffset carries only offsets
// under which every lane is in range or already out of range by its voffset
// alone.
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// value of lane l ^ 32 (v_permlane32_swap)
__device__ __forceinline__ float xhalf(float v, bool upper)
{
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(upper ? r[0] : r[1]);
}

// Split 8 fp32 values into bf16 hi + lo operands: hi keeps the top 16 bits
// (truncation), lo = v - hi exactly, rounded to bf16; hi + lo is within 2^-16
// of v.
__device__ __forceinline__ void split8(const float *v, bf16x8 &hi, bf16x8 &lo)
{
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float v0 = v[2 * e], v1 = v[2 * e + 1];
        const uint32_t b0 = __float_as_uint(v0), b1 = __float_as_uint(v1);
        h[e] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
        const f32x2 r = {v0 - __uint_as_float(b0 & 0xffff0000u),
                         v1 - __uint_as_float(b1 & 0xffff0000u)};
        l[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
    }
    const uint4 hq = {h[0], h[1], h[2], h[3]}, lq = {l[0], l[1], l[2], l[3]};
    hi = __builtin_bit_cast(bf16x8, hq);
    lo = __builtin_bit_cast(bf16x8, lq);
}

// 16 values (K-slots i = 8kb + e) -> two K-blocks of hi + lo operands
__device__ __forceinline__ void split16(const float (&v)[16], bf16x8 (&hi)[2], bf16x8 (&lo)[2])
{
    split8(&v[0], hi[0], lo[0]);
    split8(&v[8], hi[1], lo[1]);
}

// 16 bytes per lane HBM -> LDS through a buffer descriptor (buffer_load_dwordx4
// ... lds; NT: with the nontemporal hint): lane i copies bytes voff + soff of r
// (zeros past its range) to lds + 16 i.  Issued through inline assembly so that
// the compiler's memory-counter bookkeeping does not see it: it would otherwise
// wait for the copy before LDS reads it cannot prove disjoint from it and
// before later uses of ordinary loads.  The caller waits for the copy
// (vmcnt(0)) before reading it.  M0 holds the LDS address; the kernels using
// this do not use M0 otherwise.
template <bool NT = true>
__device__ __forceinline__ void dma16b(rsrc_t r, uint32_t voff, uint32_t soff, const void *lds)
{
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)lds);
    // (the row offset joins the lane offset: a constant soffset operand would be
    // emitted as a literal, which the instruction does not accept)
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                     :
                     : "v"(voff + soff), "s"(r), "s"(la)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voff + soff), "s"(r), "s"(la)
                     : "memory", "m0");
}

}  // namespace naju

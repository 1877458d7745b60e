// naju_device.h -- device helpers shared by the libnaju kernels (gfx950).
//
// Element access for the two io types, the gate nonlinearity, and the
// agent-coherent loads/stores used for cross-workgroup hand-offs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace naju {

typedef uint16_t bf16;  // bfloat16 bit pattern

// ---------------------------------------------------------------- io types
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> io type; bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950)
template <typename IO> __device__ __forceinline__ IO from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// --------------------------------------------------------------- math
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigma(v) = 1 / (1 + e^{-v}).  sigma(+inf) = 1, sigma(-inf) = 0, NaN propagates.
__device__ __forceinline__ float sigm(float v) { return rcp(1.f + ex2(-v * kLog2e)); }

// sigma(v) and sigma(-v) from one exponential; sigma(-v) is never formed as
// 1 - sigma(v) (that cancels for large v).
__device__ __forceinline__ void sigm2(float v, float &sp, float &sm) {
    const float e = ex2(-v * kLog2e);
    sp = rcp(1.f + e);
    sm = (e < __builtin_huge_valf()) ? e * sp : 1.f;
}

// Sum over the 4 lanes of each aligned quad (lanes 4k..4k+3), in every lane:
// two DPP quad permutes (xor 1, then xor 2), no LDS round trip.
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                            0xF, 0xF, false));  // [1,0,3,2]
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E,
                                                            0xF, 0xF, false));  // [2,3,0,1]
    return v;
}

// ------------------------------------------------- cross-workgroup traffic
// Stores/loads with agent scope bypass the non-coherent caches (sc1 on
// gfx950), so a value published by one workgroup is visible to workgroups on
// other XCDs once the store has completed.
__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A published value as one 64-bit word: the fp32 value in the low half, the
// tag of the call and kind that wrote it (make_flag) in the high half.  One
// agent-scope store writes both, so a reader that sees the current tag sees the
// value stored with it: no separate flag and no wait between value and flag.
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tagged_value(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ uint32_t tagged_tag(uint64_t w) { return (uint32_t)(w >> 32); }

// Waits until every memory operation this wave issued has completed; also a
// compiler barrier for memory accesses.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------- workspace header
// Lives at the start of every workspace.  `epoch` tags the flags of one call
// (a flag is current iff its tag equals epoch+1); the last workgroup of a call
// advances `epoch` and clears `ticket` and `done`, so the workspace is
// reusable without clearing the flags.
struct WsHeader {
    uint32_t epoch;
    uint32_t ticket;
    uint32_t done;
    uint32_t error;   // bit 0: a bounded spin gave up
    uint32_t ticket2; // second ticket counter (multi-kernel calls)
    uint32_t done2;
    uint32_t pad[10];     // pad[0]: count of the backward's fix-up list
    uint32_t queue[8];    // per-XCD ticket counters of the matrix-core forward
    uint32_t pad2[40];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

constexpr uint32_t kSpinLimit = 1u << 22;  // ~0.4 s of s_sleep polling
constexpr uint32_t kFlagAgg = 1, kFlagIncl = 2;

__device__ __forceinline__ uint32_t make_flag(uint32_t ep, uint32_t st) { return (ep << 2) | st; }

// Polls flags[i] until it carries the current epoch with a nonzero state; returns
// the state.  After kSpinLimit polls it records an error and reports kFlagIncl so
// the caller proceeds (with invalid data) instead of hanging.
__device__ __forceinline__ uint32_t wait_flag(const uint32_t *flag, uint32_t ep, WsHeader *hdr) {
    uint32_t spins = 0;
    for (;;) {
        const uint32_t f = __builtin_amdgcn_readfirstlane(ld_agent(flag));
        if ((f >> 2) == ep && (f & 3u)) {
            wait_mem();
            return f & 3u;
        }
        if (++spins > kSpinLimit) {
            __hip_atomic_fetch_or(&hdr->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return kFlagIncl;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

}  // namespace naju

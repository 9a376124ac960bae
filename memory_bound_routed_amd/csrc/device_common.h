// Device helpers shared by the gfx950 kernels of libmoe (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

// bf16 pattern -> fp32 (exact): the pattern is the upper half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight consecutive bf16 values packed in 16 bytes -> fp32.
__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// 16-byte weight load that streams past the caches: every routed weight is
// read exactly once per step, so it should not evict reusable data.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Hides a value from loop-invariant code motion: weights held in registers
// across a loop are unpacked inside the loop (8 fp32 per 16 bytes) instead of
// all at once before it.  Emits no instruction.
__device__ __forceinline__ uint4 opaque(uint4 v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
    return v;
}

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// DPP lane permutations used by wave_sum (gfx9 DPP control encodings).
#define MOE_DPP_QUAD_XOR1 0xB1     // quad_perm [1,0,3,2]
#define MOE_DPP_QUAD_XOR2 0x4E     // quad_perm [2,3,0,1]
#define MOE_DPP_ROW_HALF_MIRROR 0x141
#define MOE_DPP_ROW_MIRROR 0x140

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave, returned wave-uniform.  Inside each row of
// 16 lanes the partners of every step hold the same two values (quad pairs,
// quads, half-row mirror, row mirror), so after four DPP adds every lane of
// a row holds the row sum; the four row sums are then added as
// (r0 + r1) + (r2 + r3).  The order is fixed by the lane pattern alone.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<MOE_DPP_QUAD_XOR1>(v);
    v += dpp<MOE_DPP_QUAD_XOR2>(v);
    v += dpp<MOE_DPP_ROW_HALF_MIRROR>(v);
    v += dpp<MOE_DPP_ROW_MIRROR>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// # set bits of m below this lane.
__device__ __forceinline__ int mbcnt64(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
    return v;
}

// SiLU(g) * u in fp32: g / (1 + exp(-g)) * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

// Accesses that are coherent across the whole device within one launch:
// agent-scope relaxed atomics, which go through to memory past the XCD's L2,
// so small data can be handed to another workgroup without an L2 writeback
// or invalidate (the hand-off is ordered by waiting for the stores to
// complete before an atomic counter is bumped).
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_agent(const int32_t* p) {
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Quotient and remainder by a divisor fixed at launch, by multiply-high
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994): for 1 <= d < 2^31, s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, every 0 <= x < 2^31 has
// x / d = (umulhi(x, m) + x) >> s (the sum stays below 2^32).
struct FastDiv {
    uint32_t d = 1, m = 1, s = 0;
    FastDiv() = default;
    explicit FastDiv(uint32_t div) : d(div) {
        s = 0;
        while ((1u << s) < d) ++s;
        m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1);
    }
    __device__ __forceinline__ int div(int x) const { return (int)((__umulhi((uint32_t)x, m) + (uint32_t)x) >> s); }
    __device__ __forceinline__ int mod(int x) const { return x - div(x) * (int)d; }
};

// Pins a kernel argument in scalar registers from the start of the kernel:
// the value becomes the output of an (empty) asm statement, so the compiler
// cannot re-read it from the kernel-argument segment where it is used late
// (a dependent memory round trip on a serial path); under register pressure
// it is spilled to a VGPR lane instead.
template <typename T>
__device__ __forceinline__ void pin_arg(T& v) {
    asm volatile("" : "+s"(v));
}
// Pointer arguments (all of which point to global memory): after the asm the
// compiler no longer knows the address space and would use FLAT instructions,
// which also count against the LDS wait counter, so that every LDS wait would
// wait for outstanding global stores and atomics too.  The pinned value is
// therefore a global-space pointer.
template <typename T>
__device__ __forceinline__ T* pin_global(T* p) {
    __attribute__((address_space(1))) T* g = (__attribute__((address_space(1))) T*)p;
    asm volatile("" : "+s"(g));
    return (T*)g;
}
template <typename T>
__device__ __forceinline__ void pin_arg(T*& p) {
    p = pin_global(p);
}
template <typename T>
__device__ __forceinline__ void pin_arg(T* __restrict__& p) {
    p = pin_global(p);
}

// Make a value wave-uniform (lets the compiler keep it in a scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Device error flag bits (mirror of the public enum in moe.h).
#define DEVERR_BAD_ROUTE_ID 1
#define DEVERR_BAD_PLAN 2
#define DEVERR_BAD_BLOCK_EXPERT 4
#define DEVERR_BAD_COUNTS 8

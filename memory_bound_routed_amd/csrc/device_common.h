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

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Butterfly sum over the 64 lanes of a wave.  Partners add the same two
// values (commutative), so every lane ends with the same bits, and the order
// is fixed by the lane pattern alone.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
    return v;
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

// Make a value wave-uniform (lets the compiler keep it in a scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Device error flag bits (mirror of the public enum in moe.h).
#define DEVERR_BAD_ROUTE_ID 1
#define DEVERR_BAD_PLAN 2
#define DEVERR_BAD_BLOCK_EXPERT 4
#define DEVERR_BAD_COUNTS 8

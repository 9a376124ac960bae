// The channel-selection reader's per-token rotation and partial scan (page
// "Channel Selection for Mixture-of-Experts Decoding Needs No Calibration
// Data", Stage 1), shared by the router launch (whose spare workgroups do it
// beside the router GEMV) and the reader's own launch.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kReaderBlock = 128;  // rotation block (coordinates)
constexpr int kReaderScan = 80;    // coordinates scanned per block

// One wave: block `hb` (128 fp32 values) of one token is rotated with the
// signs `sg` (+-1): x'' = H_128 diag(sg) h in fp64 by the butterflies of the
// fast Walsh-Hadamard transform in stride order 1, 2, ..., 64 -- lane l holds
// coordinates 2l and 2l+1, so stride 1 is inside the lane and stride 2d pairs
// lane l with lane l ^ d -- which is exact for fp32 input of ordinary range
// and in any case the same operations in the same order as the definition.
// Then the 80 coordinates of largest |x''| (ties to the lower coordinate) are
// kept: sel[0 .. 80) ascending, val = fp32(x'').  `key` is 128 doubles of LDS
// owned by the wave.  Only wave-level barriers: a caller may let other waves
// of its workgroup leave early.
__device__ __forceinline__ void rotate_scan_wave(const float* __restrict__ hb, const int8_t* __restrict__ sg,
                                                 uint8_t* __restrict__ sel, float* __restrict__ val, double* key) {
    const int lane = threadIdx.x % MOE_WAVE;
    const float2 hv = *reinterpret_cast<const float2*>(hb + 2 * lane);
    const int s0 = sg[2 * lane], s1 = sg[2 * lane + 1];
    double a = (double)hv.x * (double)s0;
    double b = (double)hv.y * (double)s1;
    {
        const double x = a + b, y = a - b;  // stride 1
        a = x;
        b = y;
    }
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {  // stride 2d
        const double pa = __shfl_xor(a, d, MOE_WAVE);
        const double pb = __shfl_xor(b, d, MOE_WAVE);
        if (lane & d) {  // the upper element of each pair: lower - upper
            a = pa - a;
            b = pb - b;
        } else {
            a = a + pa;
            b = b + pb;
        }
    }
    // keys: |x''|, NaN below every number, so that the order stays total and
    // exactly 80 coordinates are kept whatever the input
    const double ka = a == a ? fabs(a) : -1.0, kb = b == b ? fabs(b) : -1.0;
    key[2 * lane] = ka;
    key[2 * lane + 1] = kb;
    __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses execute in order
    // rank = # coordinates ahead: larger magnitude, or equal and lower index
    int ra = 0, rb = 0;
    const int ca = 2 * lane, cb = 2 * lane + 1;
    for (int c0 = 0; c0 < kReaderBlock; c0 += 2) {
        const double2 kc = *reinterpret_cast<const double2*>(key + c0);
        ra += (kc.x > ka || (kc.x == ka && c0 < ca)) ? 1 : 0;
        ra += (kc.y > ka || (kc.y == ka && c0 + 1 < ca)) ? 1 : 0;
        rb += (kc.x > kb || (kc.x == kb && c0 < cb)) ? 1 : 0;
        rb += (kc.y > kb || (kc.y == kb && c0 + 1 < cb)) ? 1 : 0;
    }
    const bool sa = ra < kReaderScan, sb = rb < kReaderScan;
    const uint64_t ma = __ballot(sa), mb = __ballot(sb);
    const int pa = mbcnt64(ma) + mbcnt64(mb);  // kept coordinates below 2l
    if (sa) {
        sel[pa] = (uint8_t)ca;
        val[pa] = (float)a;
    }
    if (sb) {
        sel[pa + (sa ? 1 : 0)] = (uint8_t)cb;
        val[pa + (sa ? 1 : 0)] = (float)b;
    }
    __builtin_amdgcn_wave_barrier();
}

}  // namespace moe

// The channel-selection reader's per-token rotation and partial scan (page
// "Channel Selection for Mixture-of-Experts Decoding Needs No Calibration
// Data", Stage 1), shared by the router launch (whose spare workgroups do it
// beside the router GEMV) and the reader's own launch.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kReaderBlock = 128;  // rotation block (coordinates)
constexpr int kReaderScan = 80;    // coordinates scanned per block

// # of the wave's 128 keys (two per lane) at or above c.
__device__ __forceinline__ int count_at_least(uint64_t ka, uint64_t kb, uint64_t c) {
    return __popcll(__ballot(ka >= c)) + __popcll(__ballot(kb >= c));
}

// One wave: block `hb` (128 fp32 values) of one token is rotated with the
// signs `sg` (+-1): x'' = H_128 diag(sg) h in fp64 by the butterflies of the
// fast Walsh-Hadamard transform in stride order 1, 2, ..., 64 -- lane l holds
// coordinates 2l and 2l+1, so stride 1 is inside the lane and stride 2d pairs
// lane l with lane l ^ d -- which is exact for fp32 input of ordinary range
// and in any case the same operations in the same order as the definition.
// Then the 80 coordinates of largest |x''| (ties to the lower coordinate) are
// kept: sel[0 .. 80) ascending, val = fp32(x'').
//
// Selection without memory: the key of a coordinate is the bit pattern of
// |x''| (order-preserving for non-negative doubles; NaN as 0).  The 80th
// largest key is found two bits at a time from the top, counting keys at or
// above each candidate with ballots; it stops as soon as a candidate has
// exactly 80 keys at or above it.  Otherwise the 80th key T is exact and the
// keys equal to T are taken in coordinate order until 80 are kept.
__device__ __forceinline__ void rotate_scan_wave(const float* __restrict__ hb, const int8_t* __restrict__ sg,
                                                 uint8_t* __restrict__ sel, float* __restrict__ val) {
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
    const uint64_t ka = a == a ? (uint64_t)__double_as_longlong(fabs(a)) : 0ull;
    const uint64_t kb = b == b ? (uint64_t)__double_as_longlong(fabs(b)) : 0ull;
    uint64_t pref = 0;
    bool exact = false;
    for (int hi = 62; hi >= 0 && !exact; hi -= 2) {  // wave-uniform
        const int lo = hi > 0 ? hi - 1 : 0;
        const int nd = hi > 0 ? 3 : 1;
        int best = 0;
        for (int d = nd; d >= 1; --d) {
            const uint64_t c = pref | ((uint64_t)d << lo);
            const int cnt = count_at_least(ka, kb, c);
            if (cnt >= kReaderScan) {
                best = d;
                exact = cnt == kReaderScan;
                break;
            }
        }
        pref |= (uint64_t)best << lo;
    }
    bool sa, sb;
    if (exact) {
        sa = ka >= pref;
        sb = kb >= pref;
    } else {  // pref is the 80th largest key: its ties in coordinate order
        const int gt = __popcll(__ballot(ka > pref)) + __popcll(__ballot(kb > pref));
        const int need = kReaderScan - gt;
        const bool ea = ka == pref, eb = kb == pref;
        const uint64_t mea = __ballot(ea), meb = __ballot(eb);
        const int pe = mbcnt64(mea) + mbcnt64(meb);  // equal keys at coordinates below 2l
        sa = ka > pref || (ea && pe < need);
        sb = kb > pref || (eb && pe + (ea ? 1 : 0) < need);
    }
    const uint64_t ma = __ballot(sa), mb = __ballot(sb);
    const int pa = mbcnt64(ma) + mbcnt64(mb);  // kept coordinates below 2l
    if (sa) {
        sel[pa] = (uint8_t)(2 * lane);
        val[pa] = (float)a;
    }
    if (sb) {
        sel[pa + (sa ? 1 : 0)] = (uint8_t)(2 * lane + 1);
        val[pa + (sa ? 1 : 0)] = (float)b;
    }
}

}  // namespace moe

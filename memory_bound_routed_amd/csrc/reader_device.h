// The channel-selection reader's per-token rotation and partial scan (page
// "Channel Selection for Mixture-of-Experts Decoding Needs No Calibration
// Data", Stage 1), shared by the router launch (whose spare workgroups do it
// beside the router GEMV) and the reader's own launch.
#pragma once

#include "device_common.h"
#include "launch.h"
#include "select_device.h"

namespace moe {

constexpr int kReaderBlock = 128;  // rotation block (coordinates)
constexpr int kReaderScan = 80;    // coordinates scanned per block
constexpr int kReaderMaxGroups = 2;  // block groups of the screening (partial estimates per channel)

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

// Per-candidate scores of the reader for one token (thread tid, candidates
// idx = 8 tid .. 8 tid + 7 = s * I + j): g_hat and v_hat as the screening's
// group partials added in order, then the score (w_s * ||d_j||) *
// |SiLU(g_hat) v_hat| in fp32 (NaN and invalid slots score 0, -0 as +0) as
// its bit pattern sb (non-negative: it orders like the value) and the tie
// key tb = e << 19 | j << 5 | s (invalid slots as expert 8191).  Also the
// mask of real candidates and the largest and smallest score bits; est_out
// and score_out (nullable) receive g_hat, v_hat and the score.  se / sw: the
// token's expert ids (-1 when invalid) and affinities, in LDS.
__device__ inline void reader_scores(const ReaderArgs& ra, int t, FastDiv fI, const int* se, const float* sw,
                                     uint32_t (&sb)[kSelPer], uint32_t (&tb)[kSelPer], unsigned& vmask,
                                     uint32_t& smax, uint32_t& smin, float* __restrict__ est_out,
                                     float* __restrict__ score_out) {
    const int tid = threadIdx.x;
    const int I = ra.I, k = ra.k, nbq = ra.nbq;
    const int n = k * I;
    const float* __restrict__ est = ra.est;
    const float* __restrict__ dnorm = ra.dnorm;
    // every load first: the group partials of g and v and the norm of each
    // candidate -- as 16-byte loads when a thread's 8 candidates are 8
    // consecutive channels of one slot (I % 8 == 0), else one by one
    float g[kSelPer], v[kSelPer], dn[kSelPer];
    if (I % kSelPer == 0) {  // uniform
        const int ic = min(kSelPer * tid, n - kSelPer);
        const int s = fI.div(ic), j = ic - s * I;
        // 16-byte buffer loads (plain vector loads here are split into 4-byte
        // ones by the compiler, and the load count is what this phase pays):
        // the token's estimates, and the down norms
        const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(est + (size_t)t * k * 2 * nbq * I), (short)0, k * 2 * nbq * I * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(dnorm), (short)0, ra.E * I * 4, 0x00020000);
        const int eo = (s * 2 * nbq * I + j) * 4;
        auto ld4 = [](const __amdgpu_buffer_rsrc_t& r, int off) {
            const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
            return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                               __uint_as_float(x.w));
        };
        float4 gq[kReaderMaxGroups][2], vq[kReaderMaxGroups][2], dq[2];
#pragma unroll
        for (int q = 0; q < kReaderMaxGroups; ++q) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                gq[q][h2] = ld4(er, eo + (min(q, nbq - 1) * I + 4 * h2) * 4);
                vq[q][h2] = ld4(er, eo + ((nbq + min(q, nbq - 1)) * I + 4 * h2) * 4);
            }
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) dq[h2] = ld4(dr, ((max(se[s], 0) * I + j) + 4 * h2) * 4);
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            const int h2 = u / 4, c4 = u % 4;
            auto comp = [&](const float4& f) { return c4 == 0 ? f.x : (c4 == 1 ? f.y : (c4 == 2 ? f.z : f.w)); };
            g[u] = comp(gq[0][h2]);
            v[u] = comp(vq[0][h2]);
#pragma unroll
            for (int q = 1; q < kReaderMaxGroups; ++q) {
                g[u] += q < nbq ? comp(gq[q][h2]) : 0.f;
                v[u] += q < nbq ? comp(vq[q][h2]) : 0.f;
            }
            dn[u] = comp(dq[h2]);
        }
    } else {
        float gp[kSelPer][kReaderMaxGroups], vp[kSelPer][kReaderMaxGroups];
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            const int ic = min(kSelPer * tid + u, n - 1);
            const int s = fI.div(ic), j = ic - s * I;
            const float* eg = est + (((size_t)t * k + s) * 2 * nbq) * I + j;
#pragma unroll
            for (int q = 0; q < kReaderMaxGroups; ++q) {
                gp[u][q] = eg[(size_t)min(q, nbq - 1) * I];
                vp[u][q] = eg[(size_t)(nbq + min(q, nbq - 1)) * I];
            }
            dn[u] = dnorm[(size_t)max(se[s], 0) * I + j];
        }
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            g[u] = gp[u][0];
            v[u] = vp[u][0];
#pragma unroll
            for (int q = 1; q < kReaderMaxGroups; ++q) {
                g[u] += q < nbq ? gp[u][q] : 0.f;
                v[u] += q < nbq ? vp[u][q] : 0.f;
            }
        }
    }
    vmask = 0;
    smax = 0;
    smin = 0xFFFFFFFFu;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = kSelPer * tid + u;
        const int ic = min(idx, n - 1);
        const int s = fI.div(ic), j = ic - s * I;
        const int e = se[s];
        float sc = (sw[s] * dn[u]) * fabsf(silu_mul(g[u], v[u]));
        if (!(sc >= 0.f) || e < 0) sc = 0.f;  // NaN, invalid slot
        sc += 0.f;                          // -0 as +0
        if (idx < n) {
            if (est_out) {
                est_out[(((size_t)t * k + s) * 2 + 0) * I + j] = g[u];
                est_out[(((size_t)t * k + s) * 2 + 1) * I + j] = v[u];
            }
            if (score_out) score_out[((size_t)t * k + s) * I + j] = sc;
        }
        sb[u] = idx < n ? __float_as_uint(sc) : 0u;
        tb[u] = ((uint32_t)(e < 0 ? 8191 : e) << 19) | ((uint32_t)j << 5) | (uint32_t)s;
        vmask |= idx < n ? (1u << u) : 0u;
        if (idx < n) {
            smax = max(smax, sb[u]);
            smin = min(smin, sb[u]);
        }
    }
}

}  // namespace moe

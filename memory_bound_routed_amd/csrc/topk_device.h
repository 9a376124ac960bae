// Top-k by rank counting under a total order of (logit, expert), shared by
// the router and by the expert kernel that routes its own token (page
// "Route-Block Membership Selects Packed-AWQ Arithmetic", Sec. 2.1: the
// router's M x k expert-id array; ties go to the lower expert id).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

// Total-order key of (logit, expert): a larger key ranks first.  The high
// word maps the fp32 logit monotonically onto uint32 (-0 is first turned into
// +0, so equal logits give equal words), the low word is ~e, so that equal
// logits order by ascending expert id.  Keys are distinct within a token.
__device__ __forceinline__ uint64_t order_key(float l, int e) {
    uint32_t u = __float_as_uint(l + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}

// The logit and the expert a key was made from (-0 comes back as +0).
__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t hi = (uint32_t)(key >> 32);
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }

// c + (kv < o): the borrow out of the 64-bit difference kv - o, taken by a
// chain of 32-bit subtract-with-borrow operations and added as a carry.  The
// compiler turns the plain comparison into 64-bit compares and selects,
// which take several times longer on this path.
__device__ __forceinline__ int add_if_less(int c, uint64_t kv, uint64_t o) {
    uint32_t t;
    asm("v_sub_co_u32 %1, vcc, %2, %4\n\t"
        "v_subb_co_u32 %1, vcc, %3, %5, vcc\n\t"
        "v_addc_co_u32 %0, vcc, 0, %0, vcc"
        : "+v"(c), "=&v"(t)
        : "v"((uint32_t)kv), "v"((uint32_t)(kv >> 32)), "v"((uint32_t)o), "v"((uint32_t)(o >> 32))
        : "vcc");
    return c;
}

// # keys in row[j0 .. j0+n) greater than kv (n and j0 even: 16-byte pairs).
__device__ __forceinline__ int count_greater(const uint64_t* row, int j0, int n, uint64_t kv) {
    const ulonglong2* r2 = reinterpret_cast<const ulonglong2*>(row + j0);
    int c = 0;
    int q = 0;
    for (; q + 8 <= n / 2; q += 8) {  // eight 16-byte reads in flight
        ulonglong2 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = r2[q + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) c = add_if_less(add_if_less(c, kv, o[u].x), kv, o[u].y);
    }
    for (; q < n / 2; ++q) {
        const ulonglong2 o = r2[q];
        c = add_if_less(add_if_less(c, kv, o.x), kv, o.y);
    }
    return c;
}

__device__ __forceinline__ uint64_t minmax64(uint64_t a, uint64_t b, bool take_max) {
    return take_max ? (a > b ? a : b) : (a < b ? a : b);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// One butterfly step over a DPP lane pairing: the larger (take_max) or the
// smaller of a lane's key and its partner's.
template <int CTRL>
__device__ __forceinline__ uint64_t bfly_step(uint64_t v, bool take_max) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return minmax64(v, ((uint64_t)hi << 32) | lo, take_max);
}

// Top-k of one token's E <= 64*G keys (keys[x], x < E, in LDS) by one wave,
// without the other waves.  T = the least of the maxima of k' >= k aligned
// groups of 64/k' lanes (k' the power of two >= k; lane l holds keys
// l + 64 g): at least k keys are >= T, so every key of the top k is >= T (a
// candidate), and a candidate's rank among all keys is its rank among the
// candidates.  With at most 64 candidates they are ranked in the wave's LDS
// list wk/wi (64 entries each; a wave's LDS accesses execute in order), the
// expert and logit of slot s go to sel_e[s] / sel_l[s] (s < k) and the
// function returns true; else it writes nothing and returns false (uniform).
template <int G>
__device__ __forceinline__ bool wave_topk(const uint64_t* keys, int E, int k, int* sel_e, float* sel_l, uint64_t* wk,
                                          int* wi) {
    const int lane = threadIdx.x % MOE_WAVE;
    uint64_t kk[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint64_t kv = keys[min(lane + MOE_WAVE * g, E - 1)];
        kk[g] = lane + MOE_WAVE * g < E ? kv : 0ull;  // 0: no expert
    }
    uint64_t v = kk[0];
#pragma unroll
    for (int g = 1; g < G; ++g) v = v > kk[g] ? v : kk[g];
    const int gb = 6 - (k <= 1 ? 0 : 32 - __builtin_clz((unsigned)(k - 1)));  // steps taking the maximum
    v = bfly_step<MOE_DPP_QUAD_XOR1>(v, 0 < gb);
    v = bfly_step<MOE_DPP_QUAD_XOR2>(v, 1 < gb);
    v = bfly_step<MOE_DPP_ROW_HALF_MIRROR>(v, 2 < gb);
    v = bfly_step<MOE_DPP_ROW_MIRROR>(v, 3 < gb);
    const uint64_t T = minmax64(minmax64(readlane64(v, 0), readlane64(v, 16), 4 < gb),
                                minmax64(readlane64(v, 32), readlane64(v, 48), 4 < gb), 5 < gb);
    uint64_t m[G];
    int C = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = __ballot(lane + MOE_WAVE * g < E && kk[g] >= T);
        C += __popcll(m[g]);
    }
    if (C > MOE_WAVE) return false;
    int base = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if ((m[g] >> lane) & 1ull) {
            const int pos = base + mbcnt64(m[g]);
            wk[pos] = kk[g];
            wi[pos] = lane + MOE_WAVE * g;
        }
        base += __popcll(m[g]);
    }
    if (lane >= C) wk[lane] = 0ull;  // pad: ranks no one
    __builtin_amdgcn_wave_barrier();
    if (lane < C) {
        const uint64_t ck = wk[lane];
        const ulonglong2* w2 = reinterpret_cast<const ulonglong2*>(wk);
        int c = 0;
        for (int j0 = 0; j0 < (C + 1) / 2; j0 += 8) {  // eight pairs in flight; entries past C are 0
            ulonglong2 o[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] = w2[j0 + u];  // j0 + u < 32
#pragma unroll
            for (int u = 0; u < 8; ++u) c = add_if_less(add_if_less(c, ck, o[u].x), ck, o[u].y);
        }
        if (c < k) {
            sel_e[c] = wi[lane];
            sel_l[c] = key_logit(ck);
        }
    }
    __builtin_amdgcn_wave_barrier();
    return true;
}

// Renormalised softmax over the selected logits of one token, on one wave:
// lane s < k holds the logit of slot s (slot 0 the largest); returns
// exp(l_s - l_0) / sum_{s' < k} exp(l_s' - l_0), the denominator added in slot
// order.  Lanes s >= k return an unspecified value.
__device__ __forceinline__ float topk_softmax(float l, int lane, int k) {
    const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 0));
    const float x = lane < k ? expf(l - l0) : 0.f;
    float den = 0.f;
    for (int s = 0; s < k; ++s) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), s));
    return x / den;
}

// LDS of route_token in a workgroup of NT threads.
template <int NT>
struct __align__(16) RouteLds {
    uint64_t skey[NT];
    uint64_t wk[MOE_WAVE];
    int wi[MOE_WAVE];
    int sel_e[32];
    float sel_l[32];
    float sel_w[32];
    int slow;
};

// The router's slice partials of logit tid (< E) of token t, slices 0 .. 7
// (and the bias), loaded into registers: route_token_load issues the loads
// and returns, so that a caller can work while they are in flight;
// route_token_from adds them (and slices past 8) in slice order.
constexpr int kRoutePre = 8;
struct RoutePart {
    float x[kRoutePre];
    float bias;
};
__device__ __forceinline__ void route_token_load(const float* __restrict__ part, const float* __restrict__ bias,
                                                 int nslices, int M, int t, int E, RoutePart& rp) {
    const int tid = threadIdx.x;
    const int ex = min(tid, E - 1);
    if ((tid / MOE_WAVE) * MOE_WAVE < E) {  // uniform: the waves that hold experts
#pragma unroll
        for (int u = 0; u < kRoutePre; ++u) rp.x[u] = part[((size_t)min(u, nslices - 1) * M + t) * E + ex];
        rp.bias = bias ? bias[ex] : 0.f;
    } else {
#pragma unroll
        for (int u = 0; u < kRoutePre; ++u) rp.x[u] = 0.f;
        rp.bias = 0.f;
    }
}

// One token's routing inside a workgroup of NT threads (E <= NT, k <= 32):
// the router's slice partials part[slice][t][e] of M tokens added in slice
// order (+ bias), the top-k by (logit, expert) -- by one wave (wave_topk)
// when E <= 256 and the keys at or above its threshold fit in a wave, else
// by counting every key -- and the renormalised softmax.  The arithmetic is
// the router's, so the ids and weights are its own bit for bit.  Leaves
// L.sel_e, sel_l[0 .. k) readable by every thread, and with `weights` (or in
// the writer) sel_w[0 .. k) too (each path ends with a barrier); the writer
// (uniform) also stores the token's logits (when logits is not null), ids
// and weights.  route_token_from takes the first kRoutePre slices (and the
// bias) from route_token_load.
template <int NT>
__device__ inline void route_token_from(const RoutePart& rp, const float* __restrict__ part,
                                        const float* __restrict__ bias, int nslices, int M, int t, int E, int k,
                                        bool writer, float* __restrict__ logits, int32_t* __restrict__ ids,
                                        float* __restrict__ wts, RouteLds<NT>& L, bool weights = true) {
    const int tid = threadIdx.x;
    if (tid < E) {
        float lg = 0.f;
#pragma unroll
        for (int u = 0; u < kRoutePre; ++u) lg += u < nslices ? rp.x[u] : 0.f;  // slice order
        for (int sl0 = kRoutePre; sl0 < nslices; sl0 += 8) {  // eight slices in flight
            float xs[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) xs[u] = part[((size_t)min(sl0 + u, nslices - 1) * M + t) * E + tid];
#pragma unroll
            for (int u = 0; u < 8; ++u) lg += sl0 + u < nslices ? xs[u] : 0.f;
        }
        if (bias) lg += rp.bias;
        if (logits && writer) logits[(size_t)t * E + tid] = lg;
        L.skey[tid] = order_key((lg != lg) ? -INFINITY : lg, tid);  // NaN ranks as -inf
    }
    if (tid == 0) L.slow = E > 4 * MOE_WAVE;
    __syncthreads();
    if (tid < MOE_WAVE && E <= 4 * MOE_WAVE && !wave_topk<4>(L.skey, E, k, L.sel_e, L.sel_l, L.wk, L.wi)) L.slow = 1;
    __syncthreads();
    if (L.slow) {  // every key counted
        if (tid < E) {
            const int rank = count_greater(L.skey, 0, E, L.skey[tid]);
            if (rank < k) {
                L.sel_e[rank] = tid;
                L.sel_l[rank] = key_logit(L.skey[tid]);
            }
        }
        __syncthreads();
    }
    if (!weights && !writer) return;  // uniform: the selection is readable
    if (tid < MOE_WAVE) {  // lane s: slot s
        const float w = topk_softmax(L.sel_l[min(tid, k - 1)], tid, k);
        if (tid < k) {
            L.sel_w[tid] = w;
            if (writer) {
                ids[(size_t)t * k + tid] = L.sel_e[tid];
                wts[(size_t)t * k + tid] = w;
            }
        }
    }
    __syncthreads();
}

template <int NT>
__device__ inline void route_token(const float* __restrict__ part, const float* __restrict__ bias, int nslices,
                                   int M, int t, int E, int k, bool writer, float* __restrict__ logits,
                                   int32_t* __restrict__ ids, float* __restrict__ wts, RouteLds<NT>& L,
                                   bool weights = true) {
    RoutePart rp;
    route_token_load(part, bias, nslices, M, t, E, rp);
    route_token_from<NT>(rp, part, bias, nslices, M, t, E, k, writer, logits, ids, wts, L, weights);
}

}  // namespace moe

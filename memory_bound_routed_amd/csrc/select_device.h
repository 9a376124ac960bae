// Exact top-K selection of one token's candidates inside one 1024-thread
// workgroup, shared by the channel selections (page "Channel Selection for
// Mixture-of-Experts Decoding Needs No Calibration Data", Stage 2: the K best
// (slot, channel) candidates across all routed experts).
//
// Thread tid owns the candidates idx = 8 tid .. 8 tid + 7.  Each candidate
// has a coarse bin (monotone in the candidates' order: a larger bin means a
// better candidate) and NL 32-bit keys compared one after the other (larger
// is better), the last of which is distinct between candidates.  The K best
// are found as
//   1. a histogram over 2048 bins and a suffix scan: the bin B where the count
//      of candidates in better bins reaches K (bins above B are kept, bins
//      below dropped);
//   2. inside bin B only: when B holds at most 256 candidates, they are
//      listed in LDS and each is kept when fewer than the demand of them
//      rank above it (keys compared in order); else a radix select over each
//      key in turn -- digit passes of up to 11 bits from the highest bit
//      where the candidates' keys differ (a key on which they all tie is
//      skipped) -- narrowing to the candidates that tie on the keys so far
//      until the demand is met exactly.  Both keep the same set: the best
//      `demand` by the keys, the last of which is distinct.
// The bins (linear_bin between the candidates' minimum and maximum) spread
// the candidates so that the histogram's LDS atomics seldom meet on one
// address; the radix passes only see bin B's few candidates.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kSelThreads = 1024;
constexpr int kSelPer = 8;  // candidates per thread (k * I <= 8192)
constexpr int kSelWaves = kSelThreads / MOE_WAVE;
constexpr int kRadixBins = 2048;  // bins of the first pass and of a radix digit pass (11 bits)
constexpr int kRankList = 256;    // threshold-bin candidates ranked directly (at most)

struct __align__(16) RadixLds {
    int hist[kRadixBins];  // also the ranked list: [kRankList] x 4 keys, then [kRankList] flags
    int wsum[kSelWaves];
    uint32_t wmax[kSelWaves], wmin[kSelWaves];
    int digit, above, cnt, total, nlist;
    int slot_off[33];
};
static_assert(kRankList * 5 <= kRadixBins, "the ranked list fits in the histogram");

// After the histogram L.hist[0 .. nb) is complete (and a barrier): the bin
// where the candidates in larger bins first reach `need` -- its index, the
// count in larger bins and its own count, the same in every thread.  nb is a
// power of two, 2 <= nb <= 2048; thread tid owns the bins nb - 1 - per tid -
// i, i < per = max(nb / 1024, 1) (descending).
__device__ __forceinline__ void find_bin(int nb, int need, RadixLds& L, int* digit, int* above, int* cnt) {
    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE, wave = tid / MOE_WAVE;
    const int per = nb > kSelThreads ? nb / kSelThreads : 1;
    const int nbt = nb / per;  // threads with bins
    int hv[kRadixBins / kSelThreads];
    int loc = 0;
#pragma unroll
    for (int i = 0; i < kRadixBins / kSelThreads; ++i) {
        hv[i] = (i < per && tid < nbt) ? L.hist[nb - 1 - per * tid - i] : 0;
        loc += hv[i];
    }
    int incl = loc;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int y = __shfl_up(incl, d, MOE_WAVE);
        if (lane >= d) incl += y;
    }
    if (lane == MOE_WAVE - 1) L.wsum[wave] = incl;
    __syncthreads();
    int before = incl - loc;  // candidates in larger bins
    for (int x = 0; x < wave; ++x) before += L.wsum[x];
    if (tid < nbt && before < need && need <= before + loc) {
#pragma unroll
        for (int i = 0; i < kRadixBins / kSelThreads; ++i) {
            if (i < per && before < need && need <= before + hv[i]) {
                L.digit = nb - 1 - per * tid - i;
                L.above = before;
                L.cnt = hv[i];
            }
            before += hv[i];
        }
    }
    __syncthreads();
    *digit = L.digit;
    *above = L.above;
    *cnt = L.cnt;
    __syncthreads();  // L is reused next
}

// Among the candidates u with (vmask >> u) & 1 (at least `need` of them),
// which all share the key bits above `hibit` (those of `common`), the value
// X such that `need` keys are >= X: returns X and sets *whole when the keys
// >= X are exactly `need` (else the keys equal to X exceed the demand: ties).
// Digit passes of up to 11 bits from bit hibit down, each a histogram of the
// candidates sharing the digits found so far.
__device__ inline uint32_t radix_kth_largest(const uint32_t (&key)[kSelPer], unsigned vmask, int need, RadixLds& L,
                                             bool* whole, int hibit, uint32_t common) {
    const int tid = threadIdx.x;
    uint32_t pmask = ~((2u << hibit) - 1u);  // bits above hibit (none when hibit = 31)
    uint32_t prefix = common & pmask;
    *whole = false;
    for (int top = hibit; top >= 0;) {  // uniform
        const int width = top + 1 < 11 ? top + 1 : 11;
        const int shift = top - width + 1;
        const int nb = 1 << width;
        for (int i = tid; i < nb; i += kSelThreads) L.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kSelPer; ++u)
            if (((vmask >> u) & 1u) && (key[u] & pmask) == prefix) atomicAdd(&L.hist[(key[u] >> shift) & (nb - 1)], 1);
        __syncthreads();
        int dg, ab, ct;
        find_bin(nb, need, L, &dg, &ab, &ct);
        prefix |= (uint32_t)dg << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        need -= ab;
        if (need == ct) {  // the whole bin is kept (uniform)
            *whole = true;
            return prefix;
        }
        top = shift - 1;
    }
    return prefix;  // exact value; its keys exceed the demand
}

// Workgroup sum of one small count per thread (LDS atomic; three barriers).
__device__ __forceinline__ int block_sum(int c, RadixLds& L) {
    if (threadIdx.x == 0) L.total = 0;
    __syncthreads();
    if (c) atomicAdd(&L.total, c);
    __syncthreads();
    const int v = L.total;
    __syncthreads();
    return v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Workgroup maximum and minimum of one value per thread.
__device__ __forceinline__ void block_max_min(uint32_t mx, uint32_t mn, RadixLds& L, uint32_t* omx, uint32_t* omn) {
    mx = max(mx, dpp_u32<MOE_DPP_QUAD_XOR1>(mx));
    mn = min(mn, dpp_u32<MOE_DPP_QUAD_XOR1>(mn));
    mx = max(mx, dpp_u32<MOE_DPP_QUAD_XOR2>(mx));
    mn = min(mn, dpp_u32<MOE_DPP_QUAD_XOR2>(mn));
    mx = max(mx, dpp_u32<MOE_DPP_ROW_HALF_MIRROR>(mx));
    mn = min(mn, dpp_u32<MOE_DPP_ROW_HALF_MIRROR>(mn));
    mx = max(mx, dpp_u32<MOE_DPP_ROW_MIRROR>(mx));
    mn = min(mn, dpp_u32<MOE_DPP_ROW_MIRROR>(mn));
    uint32_t wmx = 0, wmn = 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        wmx = max(wmx, (uint32_t)__builtin_amdgcn_readlane((int)mx, 16 * r));
        wmn = min(wmn, (uint32_t)__builtin_amdgcn_readlane((int)mn, 16 * r));
    }
    const int wave = threadIdx.x / MOE_WAVE;
    if (threadIdx.x % MOE_WAVE == 0) {
        L.wmax[wave] = wmx;
        L.wmin[wave] = wmn;
    }
    __syncthreads();
    uint32_t a = 0, b = 0xFFFFFFFFu;
    for (int x = 0; x < kSelWaves; ++x) {
        a = max(a, L.wmax[x]);
        b = min(b, L.wmin[x]);
    }
    *omx = a;
    *omn = b;
    __syncthreads();  // L is reused next
}

// Order-preserving map of a float to uint32 (larger value -> larger key;
// -0 and +0 share a key).
__device__ __forceinline__ uint32_t float_order_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of_order_key(uint32_t k) {
    return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}

// First-pass bin of a value x >= lo among nbins bins linear between lo and
// hi (scale nbins / (hi - lo), 0 when that is not finite): monotone
// non-decreasing in x.  Linear in the value, the bins follow the candidates'
// actual spread, however narrow (static channel norms of one layer can lie
// within a few percent of each other).
__device__ __forceinline__ int linear_bin(float x, float lo, float scl, int nbins) {
    const float f = (x - lo) * scl;
    return f < (float)(nbins - 1) ? (f > 0.f ? (int)f : 0) : nbins - 1;
}
__device__ __forceinline__ float linear_scale(float lo, float hi, int nbins) {
    const float d = hi - lo;
    const float s = d > 0.f ? (float)nbins / d : 0.f;
    return s < INFINITY ? s : 0.f;
}

// The K best of the candidates with (vmask >> u) & 1 by (bin, key[0], key[1],
// ...), bins in [0, 2048), K <= their number; returns this thread's kept
// mask.
template <int NL>
__device__ unsigned select_top(const int (&bin)[kSelPer], const uint32_t (&key)[NL][kSelPer], unsigned vmask, int K,
                               RadixLds& L) {
    static_assert(NL >= 1 && NL <= 4, "up to four keys per candidate");
    const int tid = threadIdx.x;
    for (int i = tid; i < kRadixBins; i += kSelThreads) L.hist[i] = 0;
    if (tid == 0) L.nlist = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSelPer; ++u)
        if ((vmask >> u) & 1u) atomicAdd(&L.hist[bin[u]], 1);
    __syncthreads();
    int B, ab, ct;
    find_bin(kRadixBins, K, L, &B, &ab, &ct);
    int need = K - ab;
    unsigned kept = 0, cand = 0;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        kept |= (((vmask >> u) & 1u) && bin[u] > B) ? (1u << u) : 0u;
        cand |= (((vmask >> u) & 1u) && bin[u] == B) ? (1u << u) : 0u;
    }
    if (need == ct) return kept | cand;  // the whole bin
    if (ct <= kRankList) {  // uniform
        // list bin B's candidates: slots by a wave scan and one LDS atomic
        // per wave (the order of the list does not matter)
        uint4* lk = reinterpret_cast<uint4*>(L.hist);  // entry i: its keys
        int* flag = L.hist + 4 * kRankList;
        const int lane = tid % MOE_WAVE;
        int slot0 = 0;
        if (__ballot(cand != 0u)) {  // uniform per wave
            const int c = __builtin_popcount(cand);
            int incl = c;
#pragma unroll
            for (int d = 1; d < MOE_WAVE; d <<= 1) {
                const int y = __shfl_up(incl, d, MOE_WAVE);
                if (lane >= d) incl += y;
            }
            int wbase = 0;
            if (lane == MOE_WAVE - 1) wbase = atomicAdd(&L.nlist, incl);
            slot0 = __shfl(wbase, MOE_WAVE - 1, MOE_WAVE) + incl - c;
#pragma unroll
            for (int u = 0, sl = slot0; u < kSelPer; ++u) {
                if (!((cand >> u) & 1u)) continue;
                uint32_t kk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int lv = 0; lv < NL; ++lv) kk[lv] = key[lv][u];
                lk[sl++] = make_uint4(kk[0], kk[1], kk[2], kk[3]);
            }
        }
        __syncthreads();
        if (tid < ct) {  // entry tid: kept when fewer than `need` entries rank above it
            const uint4 me = lk[tid];
            const uint32_t mk[4] = {me.x, me.y, me.z, me.w};
            int rank = 0;
            for (int j = 0; j < ct; ++j) {
                const uint4 o = lk[j];
                const uint32_t ok[4] = {o.x, o.y, o.z, o.w};
                bool gt = false, eq = true;
#pragma unroll
                for (int lv = 0; lv < NL; ++lv) {
                    gt = gt || (eq && ok[lv] > mk[lv]);
                    eq = eq && ok[lv] == mk[lv];
                }
                rank += gt ? 1 : 0;
            }
            flag[tid] = rank < need ? 1 : 0;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0, sl = slot0; u < kSelPer; ++u) {
            if (!((cand >> u) & 1u)) continue;
            kept |= flag[sl++] ? (1u << u) : 0u;
        }
        __syncthreads();  // L is reused next
        return kept;
    }
#pragma unroll
    for (int lv = 0; lv < NL; ++lv) {
        // the candidates' range on this key: equal keys need no pass; else
        // the passes start at the highest bit where they differ
        uint32_t kmx = 0, kmn = 0xFFFFFFFFu;
#pragma unroll
        for (int u = 0; u < kSelPer; ++u)
            if ((cand >> u) & 1u) {
                kmx = max(kmx, key[lv][u]);
                kmn = min(kmn, key[lv][u]);
            }
        block_max_min(kmx, kmn, L, &kmx, &kmn);
        if (kmx == kmn) continue;  // all tie on this key (uniform)
        bool whole;
        const uint32_t X = radix_kth_largest(key[lv], cand, need, L, &whole, 31 - __builtin_clz(kmx ^ kmn), kmn);
        unsigned above = 0, eq = 0;
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            const bool c = (cand >> u) & 1u;
            above |= (c && (whole ? key[lv][u] >= X : key[lv][u] > X)) ? (1u << u) : 0u;
            eq |= (c && key[lv][u] == X) ? (1u << u) : 0u;
        }
        kept |= above;
        if (whole) return kept;
        need -= block_sum(__builtin_popcount(above), L);
        cand = eq;
    }
    return kept | cand;  // unreachable when the last key is distinct
}

// Writes the kept set of one token (kmask per thread, exactly K candidates
// unless all n are kept): per slot the kept channels in ascending order,
// slot_kept[t][s][0 .. c_s) and slot_cnt[t][s] = c_s; optionally the kept
// set as s * I + j ascending, kept_out[t][0 .. K), and a flag per candidate,
// kept_flag[t][s][j].
__device__ inline void emit_kept(unsigned kmask, int t, int k, int I, int K, bool all, FastDiv fI, RadixLds& L,
                                 int32_t* __restrict__ slot_cnt, int32_t* __restrict__ slot_kept,
                                 int32_t* __restrict__ kept_out, uint8_t* __restrict__ kept_flag) {
    const int tid = threadIdx.x;
    const int n = k * I;
    const int cntk = __builtin_popcount(kmask);
    const int lane = tid % MOE_WAVE, wave = tid / MOE_WAVE;
    int incl = cntk;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int y = __shfl_up(incl, d, MOE_WAVE);
        if (lane >= d) incl += y;
    }
    if (lane == MOE_WAVE - 1) L.wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int x = 0; x < wave; ++x) base += L.wsum[x];
    int pos = base + incl - cntk;
    // the first kept position of every slot: the slot's first candidate's owner
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = kSelPer * tid + u;
        if (idx < n && fI.mod(idx) == 0)
            L.slot_off[fI.div(idx)] = pos + __builtin_popcount(kmask & ((1u << u) - 1u));
    }
    if (tid == 0) L.slot_off[k] = all ? n : K;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = kSelPer * tid + u;
        if (idx >= n) continue;
        const int s = fI.div(idx), j = idx - s * I;
        const bool kept = (kmask >> u) & 1u;
        if (kept_flag) kept_flag[((size_t)t * k + s) * I + j] = kept ? 1 : 0;
        if (kept) {
            if (kept_out) kept_out[(size_t)t * K + pos] = idx;
            slot_kept[((size_t)t * k + s) * I + (pos - L.slot_off[s])] = j;
            ++pos;
        }
    }
    if (tid < k) slot_cnt[(size_t)t * k + tid] = L.slot_off[tid + 1] - L.slot_off[tid];
}

}  // namespace moe

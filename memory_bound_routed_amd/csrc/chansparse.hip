// Channel-sparse reads (page "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data", Background: channel j owns gate row j,
// up row j and down column j; Stage 2: top-k across all routed experts,
// exact compute of the kept channels, down stored transposed so that each
// d_j is contiguous).
//
// The score of candidate (slot s, channel j) is a_s * n[e_s][j]: the exact
// fp64 product of two fp32 values, so selection needs no rounding decision.
// With positive affinities the K best form a prefix of each routed expert's
// channels ordered by decreasing norm (an order computed once per layer), so
// each (slot, token) workgroup finds its own prefix length by binary searches
// over the k orders instead of sorting; ties go to the lower expert id, then
// channel, then slot.
#include <algorithm>
#include <climits>

#include "device_common.h"
#include "launch.h"
#include "topk_device.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;

// Order-preserving map of a double score to uint64 (larger score -> larger key).
__device__ __forceinline__ unsigned long long score_key(double x) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Exclusive scan of one int per thread over a workgroup of NT threads;
// returns the exclusive prefix and writes the total to *total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
    constexpr int NWV = NT / MOE_WAVE;
    const int lane = threadIdx.x % MOE_WAVE;
    const int wave = threadIdx.x / MOE_WAVE;
    int x = v;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int y = __shfl_up(x, d, MOE_WAVE);
        if (lane >= d) x += y;
    }
    if (lane == MOE_WAVE - 1) wsum[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const int c = wsum[w];
        base += w < wave ? c : 0;
        all += c;
    }
    __syncthreads();
    *total = all;
    return base + x - v;
}

// Order-preserving map of a float to uint32 (larger value -> larger key;
// -0 and +0 share a key).
__device__ __forceinline__ uint32_t float_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return (u >> 31) ? ~u : (u | 0x80000000u);
}

// Channel top-K of one token by search over k sorted lists.
//
// Candidate (s, j) is ranked by its score (descending), then expert id,
// channel and slot (ascending): a strict total order.  List s holds
// slot s's I candidates in decreasing key order; the kept candidates of a
// slot are then a prefix of its list, and only the k prefix lengths c_s
// (summing to K) have to be found.
//
// Lists.  The load-time ranks (moe_channel_ranks: each channel's position
// when its expert's channels are ordered by decreasing norm, ties to the
// lower channel) place every channel in its list with one scatter through
// LDS.  For a_s > 0 and finite norms that is the list's key order, since the
// product of two fp32 values is exact in fp64 and therefore strictly
// increasing in n.  Every list is checked (a permutation, strictly
// decreasing keys); a list that fails -- a_s = 0 or negative, non-finite
// norms, ranks that do not belong to these norms -- is sorted in LDS by rank
// counting instead, so the result is always the exact top K.  A slot whose
// expert id is invalid contributes candidates of key 0 in channel order,
// after every valid expert's.
//
// Search.  The global rank of list entry (s, r) is r plus, for every other
// list t, the number of t's entries ranked above it (a binary search).  One
// workgroup per (slot s0, token) finds c_s0 alone: a window bracketing it
// starts at [0, I]; each round evaluates the ranks of P evenly spread
// positions of the window (P * k binary searches, one per thread) and
// narrows it to the step where the rank crosses K.  At k = 8, I = 768: P =
// 128, two rounds.  The k workgroups of a token build the same lists, so
// their prefix lengths add up to exactly K without any exchange.
//
// Output: per (token, slot) the kept channels in ascending order,
// slot_kept[t][s][0 .. c_s), and slot_cnt[t][s] = c_s.  The gather turns the
// counts into offsets; in candidate order (s * I + j ascending) the kept set
// is the concatenation of the slots' lists.
//
// LDS (dynamic, n = k * I): the 64-bit score key of each list position
// [n] (computed once; reused for the kept flags), the channel of each list
// position uint16 [n].
constexpr int kSelThreads = 1024;
constexpr int kSelPer = 8;  // candidates per thread (n <= 8192)
constexpr uint16_t kNoChannel = 0xFFFF;

// ROUTE: the workgroup first routes its token from the router's slice
// partials -- the logits added in slice order (+ bias), the top-k (one wave
// from the keys above a threshold, else every key counted) and the
// renormalised softmax, with the router's arithmetic -- and writes the ids
// and affinities (and logits) as the router would.
// Pivots per round (one binary search per thread and list), and the
// divisors of the search (multiply-high division: a divide by a variable
// costs tens of instructions otherwise).
struct SelSearch {
    int P;
    FastDiv fk, fP1;  // by k, P + 1
};
SelSearch sel_search(int k) {
    SelSearch q;
    q.P = std::max(1, kSelThreads / k);  // k <= 32: P * k <= kSelThreads
    q.fk = FastDiv((uint32_t)k);
    q.fP1 = FastDiv((uint32_t)(q.P + 1));
    return q;
}

template <bool ROUTE>
__global__ void __launch_bounds__(kSelThreads)
chan_select_kernel(const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
                   const float* __restrict__ norms, const int32_t* __restrict__ ranks, int k, int I, int E, int K,
                   FastDiv fI, SelSearch srch_div, int32_t* __restrict__ slot_cnt, int32_t* __restrict__ slot_kept,
                   SelRoute route) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int n = k * I;
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(lds);  // [k][I] key at list position
    uint16_t* jsrt = reinterpret_cast<uint16_t*>(lds + 8 * (size_t)n);     // [k][I] channel at list position
    unsigned char* flag = lds;  // [I] kept channels of the own list (over the keys, after the search)
    __shared__ double sa[32];
    __shared__ int se[32];
    __shared__ int seo[32];  // tie order of slot s: its expert id, invalid last
    __shared__ unsigned s_bad;  // bit s: list s fails the order check
    __shared__ int pcnt[2][kSelThreads];  // per round (alternating), per (pivot, list): entries ranked above
    __shared__ int wsum[kSelThreads / MOE_WAVE];
    const int s0 = blockIdx.x;  // own slot
    const int t = blockIdx.y;
    const int tid = threadIdx.x;
    if (tid == 0) s_bad = 0u;

    if constexpr (ROUTE) {
        __shared__ uint64_t skey[kSelThreads];
        __shared__ int sel_e[32];
        __shared__ float sel_l[32];
        __shared__ uint64_t wk[MOE_WAVE];
        __shared__ int wi[MOE_WAVE];
        __shared__ int s_slow;
        float lg = 0.f;
        if (tid < E) {
            const float bv = route.bias ? route.bias[tid] : 0.f;
            for (int sl0 = 0; sl0 < route.nslices; sl0 += 8) {  // eight slices in flight
                float x[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    x[u] = route.part[((size_t)min(sl0 + u, route.nslices - 1) * route.M + t) * E + tid];
#pragma unroll
                for (int u = 0; u < 8; ++u) lg += sl0 + u < route.nslices ? x[u] : 0.f;  // slice order
            }
            if (route.bias) lg += bv;
            if (route.logits && s0 == 0) route.logits[(size_t)t * E + tid] = lg;
            skey[tid] = order_key((lg != lg) ? -INFINITY : lg, tid);  // NaN ranks as -inf
        }
        if (tid == 0) s_slow = E > 4 * MOE_WAVE;
        __syncthreads();
        if (tid < MOE_WAVE && E <= 4 * MOE_WAVE && !wave_topk<4>(skey, E, k, sel_e, sel_l, wk, wi)) s_slow = 1;
        __syncthreads();
        if (s_slow) {  // every key counted (E <= 1024 threads)
            if (tid < E) {
                const int rank = count_greater(skey, 0, E, skey[tid]);
                if (rank < k) {
                    sel_e[rank] = tid;
                    sel_l[rank] = key_logit(skey[tid]);
                }
            }
            __syncthreads();
        }
        if (tid < MOE_WAVE) {  // lane s: slot s
            const float w = topk_softmax(sel_l[min(tid, k - 1)], tid, k);
            if (tid < k) {
                if (s0 == 0) {
                    route.ids[(size_t)t * k + tid] = sel_e[tid];
                    route.wts[(size_t)t * k + tid] = w;
                }
                se[tid] = sel_e[tid];
                sa[tid] = (double)w;
            }
        }
    } else {
        if (tid < k) {
            const int e = topk_ids[(size_t)t * k + tid];
            se[tid] = (e >= 0 && e < E) ? e : -1;
            sa[tid] = (double)topk_w[(size_t)t * k + tid];
        }
    }
    for (int i = tid; i < n; i += kSelThreads) jsrt[i] = kNoChannel;
    __syncthreads();
    if (tid < k) seo[tid] = se[tid] < 0 ? INT_MAX : se[tid];
    // Score key of slot s's channel with norm x (-0 ranks as +0; an invalid
    // slot's candidates all have key 0).
    auto cand_key = [&](int s, float x) -> unsigned long long {
        return se[s] < 0 ? 0ull : score_key(sa[s] * (double)x + 0.0);
    };
    // Norm and list position of each candidate idx = s * I + j, thread tid
    // owning idx = tid + kSelThreads * u (coalesced loads, issued together);
    // the list position of an invalid slot's candidate is its channel.
    float nv[kSelPer];
    int rv[kSelPer];
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = min(tid + kSelThreads * u, n - 1);
        const int sl = fI.div(idx), j = idx - sl * I;
        const int e = se[sl];
        const size_t g = (size_t)(e < 0 ? 0 : e) * I + j;
        nv[u] = norms[g];
        rv[u] = ranks[g];
    }
    unsigned bad = 0u;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = tid + kSelThreads * u;
        if (idx >= n) break;
        const int sl = fI.div(idx), j = idx - sl * I;
        const int r = se[sl] < 0 ? j : rv[u];
        if (r < 0 || r >= I) {
            bad |= 1u << sl;
            continue;
        }
        keys[sl * I + r] = cand_key(sl, nv[u]);
        jsrt[sl * I + r] = (uint16_t)j;
    }
    __syncthreads();
    // Every list position filled and keys strictly decreasing (ties: channel ascending).
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int p = tid + kSelThreads * u;
        if (p >= n) break;
        const int s = fI.div(p), r = p - s * I;
        const int jr = jsrt[p];
        bool ok = jr != kNoChannel;
        if (ok && r + 1 < I) {
            const int jn = jsrt[p + 1];
            const unsigned long long kc = keys[p], kn = keys[p + 1];
            ok = jn == kNoChannel || kc > kn || (kc == kn && jr < jn);  // an empty next slot fails on its own
        }
        if (!ok) bad |= 1u << s;
    }
    if (bad) atomicOr(&s_bad, bad);
    __syncthreads();
    // Lists that fail: channel order first, then each channel moved to its
    // rank under the run-time key (counted over the whole list).
    for (unsigned todo = s_bad; todo; todo &= todo - 1) {  // uniform
        const int s = __builtin_ctz(todo);
        const int e = se[s];  // an invalid slot's list is always in order; guarded anyway
        const int nj = (I + kSelThreads - 1) / kSelThreads;
        for (int j = tid; j < I; j += kSelThreads) {
            keys[s * I + j] = cand_key(s, e < 0 ? 0.f : norms[(size_t)e * I + j]);
            jsrt[s * I + j] = (uint16_t)j;
        }
        __syncthreads();
        int rr[kSelPer];
        unsigned long long kk[kSelPer];
        for (int q = 0; q < nj; ++q) {
            const int j = tid + kSelThreads * q;
            if (j >= I) break;
            const unsigned long long x = keys[s * I + j];
            int c = 0;
            for (int j2 = 0; j2 < I; ++j2) {
                const unsigned long long y = keys[s * I + j2];
                c += (y > x || (y == x && j2 < j)) ? 1 : 0;
            }
            rr[q] = c;
            kk[q] = x;
        }
        __syncthreads();
        for (int q = 0; q < nj; ++q) {
            const int j = tid + kSelThreads * q;
            if (j >= I) break;
            keys[s * I + rr[q]] = kk[q];
            jsrt[s * I + rr[q]] = (uint16_t)j;
        }
        __syncthreads();
    }

    // Own list s0: a window [lo, hi] around c_s0, narrowed by rounds of P
    // pivots (P * k binary searches, one per thread: pivot p = tid / k,
    // list tl = tid % k).  The pivots' ranks increase with their positions,
    // so the pivots kept form a prefix whose length one block-wide count
    // gives.  A pivot's count in list tl lies between the counts of the two
    // pivots of the previous round that bracket the window, [clo, chi], so
    // later searches only cover that range.
    const int P = srch_div.P;
    const FastDiv fk = srch_div.fk, fP1 = srch_div.fP1;
    const int p = fk.div(tid);
    const int tl = tid - p * k;
    const bool act = tid < P * k;
    // ranks summed over the k lanes of a pivot by shuffles when k is a power
    // of two (the lanes are consecutive inside one wave), else through LDS
    const bool pow2 = (k & (k - 1)) == 0;
    int lo = 0, hi = I, clo = 0, chi = I;
    for (int round = 0;; ++round) {
        int* pc = pcnt[round & 1];
        const int r = lo + fP1.div((p + 1) * (hi - lo));  // in [lo, hi) when act; (p + 1) * (hi - lo) < 2^24
        const int rc = min(r, I - 1);
        const unsigned long long kc = keys[s0 * I + rc];
        const int jc = jsrt[s0 * I + rc], ec = seo[s0];
        const bool srch = act && tl != s0;
        int cnt = (act && tl == s0) ? r : clo;  // own list: the entries before r
        int span = chi - clo;
        int step = 1;
        while (step * 2 <= span) step *= 2;
        // entries of list tl ranked above the candidate (a prefix of the list)
        for (; step > 0; step >>= 1) {
            const int np = cnt + step;
            if (srch && np <= chi) {
                const unsigned long long y = keys[tl * I + np - 1];
                bool above = y > kc;
                if (y == kc) {  // equal scores: expert, channel, slot
                    const int jy = jsrt[tl * I + np - 1], ey = seo[tl];
                    above = ey < ec || (ey == ec && (jy < jc || (jy == jc && tl < s0)));
                }
                if (above) cnt = np;
            }
        }
        if (act) pc[tid] = cnt;
        bool kept_pivot = false;
        if (pow2) {
            int rank = act ? cnt : 0;
            for (int m = 1; m < k; m <<= 1) rank += __shfl_xor(rank, m, MOE_WAVE);
            kept_pivot = act && tl == 0 && rank < K;
        } else {
            __syncthreads();
            if (tid < P) {
                int rank = 0;
                for (int x = 0; x < k; ++x) rank += pc[tid * k + x];
                kept_pivot = rank < K;
            }
        }
        const int c = __syncthreads_count(kept_pivot);  // also orders the pc writes before the reads below
        const int nlo = c > 0 ? lo + fP1.div(c * (hi - lo)) + 1 : lo;  // past the last kept pivot
        const int nhi = c < P ? lo + fP1.div((c + 1) * (hi - lo)) : hi;  // the first dropped pivot
        if (tl < k) {
            clo = c > 0 ? pc[(c - 1) * k + tl] : clo;
            chi = c < P ? pc[c * k + tl] : chi;
        }
        lo = nlo;
        hi = nhi;
        if (lo >= hi) break;  // uniform
    }
    // Kept channels of the own list in ascending channel order (flags over
    // the keys, no longer read), then their count.
    const int c = lo;
    for (int i = tid; i < (I + 3) / 4; i += kSelThreads) reinterpret_cast<unsigned*>(flag)[i] = 0u;
    __syncthreads();
    for (int r = tid; r < c; r += kSelThreads) flag[jsrt[s0 * I + r]] = 1;
    __syncthreads();
    const int pj = (I + kSelThreads - 1) / kSelThreads;  // <= kSelPer
    const int j0 = tid * pj;
    unsigned takemask = 0;
    for (int u = 0; u < pj; ++u)
        if (j0 + u < I && flag[j0 + u]) takemask |= 1u << u;
    int total;
    int pos = block_exclusive_scan<kSelThreads>(__builtin_popcount(takemask), wsum, &total);
    int32_t* dst = slot_kept + ((size_t)t * k + s0) * I;
    for (int u = 0; u < pj; ++u)
        if ((takemask >> u) & 1u) dst[pos++] = j0 + u;
    if (tid == 0) slot_cnt[(size_t)t * k + s0] = c;
}

// Gate/up of KC = 4*2 kept channels (two per wave), scaled by the router
// weight, then their down rows summed over all H in kept order:
//   part[t][chunk][col] = sum_{q in chunk} (a_{s_q} * p_q) * d_q[col].
// Kept position q of a token (candidate order) is entry q - C_s of slot s's
// list, C_s = c_0 + ... + c_{s-1} <= q < C_s + c_s; workgroup (chunk, t)
// also writes kept_out[t][q] = s * I + j for its positions when asked.
template <int Q, int CQ>
__global__ void __launch_bounds__(kThreads)
chan_gather_kernel(const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
                   const int32_t* __restrict__ slot_cnt, const int32_t* __restrict__ slot_kept,
                   int32_t* __restrict__ kept_out, int k, int I, int E, int H, int K, const float* __restrict__ h,
                   const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu, const uint16_t* __restrict__ Wd,
                   float* __restrict__ part) {
    constexpr int KC = kWaves * 2;
    __shared__ float cs[KC];
    const int t = blockIdx.y;
    const int chunk = blockIdx.x;
    const int nchunks = gridDim.x;
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int q0 = chunk * KC;

    // h of the token first: it depends on nothing, and a load queued behind
    // the weight stream would wait for all of it
    float4 hq[Q][2];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int col = min((lane + MOE_WAVE * q) * 8, H - 8);
        hq[q][0] = *reinterpret_cast<const float4*>(h + (size_t)t * H + col);
        hq[q][1] = *reinterpret_cast<const float4*>(h + (size_t)t * H + col + 4);
    }
    // Resolve the KC kept channels of the chunk: lane l < k loads slot l's
    // count, expert and affinity (one round of vector loads), lane q finds
    // the slot of position q0 + q from the running counts and loads its
    // channel (a second round), then every lane takes the values by readlane.
    int ce[KC], cj[KC];
    float ca[KC];
    {
        const int sl = min(lane, k - 1);
        const int cnt_l = slot_cnt[(size_t)t * k + sl];
        const int e_l = topk_ids[(size_t)t * k + sl];
        const float a_l = topk_w[(size_t)t * k + sl];
        const int q = lane % KC;
        const int pos = q0 + q;
        int s = -1, off = 0, run = 0;
        for (int x = 0; x < k; ++x) {  // k <= 32
            const int cx = min(max(__builtin_amdgcn_readlane(cnt_l, x), 0), I);
            if (s < 0 && pos < run + cx) {
                s = x;
                off = pos - run;
            }
            run += cx;
        }
        const bool qin = pos < K && s >= 0;
        const int sc = qin ? s : 0;
        const int jv = slot_kept[((size_t)t * k + sc) * I + (qin ? off : 0)];
        const int e = __builtin_amdgcn_ds_bpermute(sc << 2, e_l);
        const float a = __int_as_float(__builtin_amdgcn_ds_bpermute(sc << 2, __float_as_int(a_l)));
        const bool vin = qin && jv >= 0 && jv < I;
        const int ev = (vin && e >= 0 && e < E) ? e : -1;
        if (kept_out && lane < KC && wave == 0 && pos < K) kept_out[(size_t)t * K + pos] = vin ? sc * I + jv : -1;
#pragma unroll
        for (int qq = 0; qq < KC; ++qq) {
            ce[qq] = __builtin_amdgcn_readlane(ev, qq);
            cj[qq] = __builtin_amdgcn_readlane(jv, qq);
            ca[qq] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), qq));
        }
    }
    // issue every load of the chunk: gate/up rows of this wave's two
    // channels, down rows of all KC channels, the token's h
    uint4 wg[2][Q], wu[2][Q], wd[KC][CQ];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int qq = wave * 2 + c;
        const bool ok = ce[qq] >= 0;
        const size_t row = ok ? ((size_t)ce[qq] * I + cj[qq]) * H : 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int col = (lane + MOE_WAVE * q) * 8;
            const bool in = ok && col < H;
            wg[c][q] = in ? load_stream16(Wg + row + col) : make_uint4(0, 0, 0, 0);
            wu[c][q] = in ? load_stream16(Wu + row + col) : make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int qq = 0; qq < KC; ++qq) {
        const bool ok = ce[qq] >= 0;
        const size_t row = ok ? ((size_t)ce[qq] * I + cj[qq]) * H : 0;
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq) {
            const int col = (tid + kThreads * cq) * 8;
            wd[qq][cq] = (ok && col < H) ? load_stream16(Wd + row + col) : make_uint4(0, 0, 0, 0);
        }
    }
    float ag[2] = {0.f, 0.f}, au[2] = {0.f, 0.f};
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int col = (lane + MOE_WAVE * q) * 8;
        if (col >= H) continue;
        const float4 h0 = hq[q][0], h1 = hq[q][1];
        const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float gf[8], uf[8];
            unpack8(wg[c][q], gf);
            unpack8(wu[c][q], uf);
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                ag[c] = fmaf(gf[x], hv[x], ag[c]);
                au[c] = fmaf(uf[x], hv[x], au[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float g = wave_sum(ag[c]);
        const float u = wave_sum(au[c]);
        const int qq = wave * 2 + c;
        if (lane == 0) cs[qq] = ce[qq] >= 0 ? ca[qq] * silu_mul(g, u) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int cq = 0; cq < CQ; ++cq) {
        const int col = (tid + kThreads * cq) * 8;
        if (col >= H) continue;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qq = 0; qq < KC; ++qq) {
            float wf[8];
            unpack8(wd[qq][cq], wf);
            const float cq_ = cs[qq];
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[x] = fmaf(cq_, wf[x], acc[x]);
        }
        float* dst = part + ((size_t)t * nchunks + chunk) * H + col;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

// y[t][col] = sum over the chunks of part[t][chunk][col].  One wave per
// workgroup: lane (row group g, float4 column c4); row group g adds chunks
// g, g + kCombRG, ... in order (a batch of loads issued together), then the
// row groups are combined by a butterfly over the lane bits above the column
// bits (xor 4, 8, 16, 32): a fixed order.
constexpr int kCombCG = 4;
constexpr int kCombRG = MOE_WAVE / kCombCG;
constexpr int kCombBatch = 8;

__global__ void __launch_bounds__(MOE_WAVE)
chan_combine_kernel(int H, int nchunks, const float* __restrict__ part, float* __restrict__ y) {
    const int t = blockIdx.y;
    const int lane = threadIdx.x;
    const int cg = lane % kCombCG;
    const int rg = lane / kCombCG;
    const int col = (blockIdx.x * kCombCG + cg) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* src = part + (size_t)t * nchunks * H + min(col, H - 4);
    for (int c0 = rg; c0 < nchunks; c0 += kCombBatch * kCombRG) {
        float4 v[kCombBatch];
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u)
            v[u] = *reinterpret_cast<const float4*>(src + (size_t)min(c0 + u * kCombRG, nchunks - 1) * H);
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const bool use = c0 + u * kCombRG < nchunks;
            acc.x += use ? v[u].x : 0.f;
            acc.y += use ? v[u].y : 0.f;
            acc.z += use ? v[u].z : 0.f;
            acc.w += use ? v[u].w : 0.f;
        }
    }
#pragma unroll
    for (int m = kCombCG; m < MOE_WAVE; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m, MOE_WAVE);
        acc.y += __shfl_xor(acc.y, m, MOE_WAVE);
        acc.z += __shfl_xor(acc.z, m, MOE_WAVE);
        acc.w += __shfl_xor(acc.w, m, MOE_WAVE);
    }
    if (rg == 0 && col < H) *reinterpret_cast<float4*>(y + (size_t)t * H + col) = acc;
}

// One wave per channel: fp64 sums of squares of the gate row, up row and
// down row, lanes summed by a fixed butterfly, then
// n = fp32( (sqrt(sg) * sqrt(sv)) * sqrt(sd) ).
__global__ void __launch_bounds__(kThreads)
channel_norms_kernel(int EI, int H, const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu,
                     const uint16_t* __restrict__ Wd, float* __restrict__ norms) {
    const int ch = blockIdx.x * kWaves + threadIdx.x / MOE_WAVE;
    const int lane = threadIdx.x % MOE_WAVE;
    if (ch >= EI) return;
    const size_t row = (size_t)ch * H;
    double sg = 0.0, sv = 0.0, sd = 0.0;
    for (int col = lane * 8; col < H; col += MOE_WAVE * 8) {
        float a[8], b[8], c[8];
        unpack8(load16(Wg + row + col), a);
        unpack8(load16(Wu + row + col), b);
        unpack8(load16(Wd + row + col), c);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
            sg += (double)a[x] * (double)a[x];
            sv += (double)b[x] * (double)b[x];
            sd += (double)c[x] * (double)c[x];
        }
    }
    sg = wave_sum_f64(sg);
    sv = wave_sum_f64(sv);
    sd = wave_sum_f64(sd);
    if (lane == 0) norms[ch] = (float)((sqrt(sg) * sqrt(sv)) * sqrt(sd));
}

// Load-time list positions of the channel-sparse selection: ranks[e][j] =
// the number of channels j2 of expert e whose norm is greater (float order)
// or equal with j2 < j, i.e. channel j's position when the expert's channels
// are ordered by decreasing norm, ties to the lower channel.  One workgroup
// per expert, the expert's norms in LDS.
__global__ void __launch_bounds__(kSelThreads)
channel_ranks_kernel(int I, const float* __restrict__ norms, int32_t* __restrict__ ranks) {
    extern __shared__ uint32_t nk[];
    const int e = blockIdx.x;
    for (int j = threadIdx.x; j < I; j += kSelThreads) nk[j] = float_key(norms[(size_t)e * I + j]);
    __syncthreads();
    for (int j = threadIdx.x; j < I; j += kSelThreads) {
        const uint32_t x = nk[j];
        int c = 0;
        for (int j2 = 0; j2 < I; ++j2) {
            const uint32_t y = nk[j2];
            c += (y > x || (y == x && j2 < j)) ? 1 : 0;
        }
        ranks[(size_t)e * I + j] = c;
    }
}

template <int Q>
hipError_t gather_q(const int32_t* topk_ids, const float* topk_w, const int32_t* slot_cnt, const int32_t* slot_kept,
                    int32_t* kept_out, int M, int k, int I, int E, int H, int K, const float* h, const uint16_t* Wg,
                    const uint16_t* Wu, const uint16_t* Wd, float* part, hipStream_t stream) {
    constexpr int KC = kWaves * 2;
    const dim3 grid((K + KC - 1) / KC, M);
    const int CQ = (H + 2047) / 2048;
    if (CQ <= 1)
        MOE_LAUNCH((chan_gather_kernel<Q, 1>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, slot_cnt,
                   slot_kept, kept_out, k, I, E, H, K, h, Wg, Wu, Wd, part);
    else if (CQ <= 2)
        MOE_LAUNCH((chan_gather_kernel<Q, 2>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, slot_cnt,
                   slot_kept, kept_out, k, I, E, H, K, h, Wg, Wu, Wd, part);
    else if (CQ <= 4)
        MOE_LAUNCH((chan_gather_kernel<Q, 4>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, slot_cnt,
                   slot_kept, kept_out, k, I, E, H, K, h, Wg, Wu, Wd, part);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

// list keys uint64 [n] (later the kept flags) + list channels uint16 [n]
size_t chan_select_lds_bytes(int n) { return (size_t)n * (sizeof(unsigned long long) + sizeof(uint16_t)); }

hipError_t launch_chan_select(const int32_t* topk_ids, const float* topk_w, const float* norms, const int32_t* ranks,
                              int M, int k, int I, int E, int K, int32_t* slot_cnt, int32_t* slot_kept,
                              hipStream_t stream) {
    if (k * I > kSelThreads * kSelPer || k > 32) return hipErrorInvalidValue;
    MOE_LAUNCH(chan_select_kernel<false>, dim3(k, M), dim3(kSelThreads), chan_select_lds_bytes(k * I), stream,
               topk_ids, topk_w, norms, ranks, k, I, E, K, FastDiv((uint32_t)I), sel_search(k), slot_cnt, slot_kept,
               SelRoute{});
    return hipGetLastError();
}

hipError_t launch_chan_select_routed(const SelRoute& route, const float* norms, const int32_t* ranks, int M, int k,
                                     int I, int E, int K, int32_t* slot_cnt, int32_t* slot_kept, hipStream_t stream) {
    if (k * I > kSelThreads * kSelPer || E > kSelThreads || k > 32 || route.M != M) return hipErrorInvalidValue;
    MOE_LAUNCH(chan_select_kernel<true>, dim3(k, M), dim3(kSelThreads), chan_select_lds_bytes(k * I), stream, nullptr,
               nullptr, norms, ranks, k, I, E, K, FastDiv((uint32_t)I), sel_search(k), slot_cnt, slot_kept, route);
    return hipGetLastError();
}

hipError_t launch_chan_gather(const int32_t* topk_ids, const float* topk_w, const int32_t* slot_cnt,
                              const int32_t* slot_kept, int32_t* kept_out, int M, int k, int I, int E, int H, int K,
                              int chunk, const float* h, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                              float* part, hipStream_t stream) {
    (void)chunk;
    if (k > MOE_WAVE) return hipErrorInvalidValue;
    const int Q = (H + 511) / 512;
#define MOE_GATHER(QQ) gather_q<QQ>(topk_ids, topk_w, slot_cnt, slot_kept, kept_out, M, k, I, E, H, K, h, Wg, Wu, Wd, \
                                   part, stream)
    if (Q <= 1) return MOE_GATHER(1);
    if (Q <= 2) return MOE_GATHER(2);
    if (Q <= 4) return MOE_GATHER(4);
    if (Q <= 8) return MOE_GATHER(8);
    if (Q <= 16) return MOE_GATHER(16);
#undef MOE_GATHER
    return hipErrorInvalidValue;
}

hipError_t launch_chan_combine(int M, int H, int nchunks, const float* part, float* y, hipStream_t stream) {
    const dim3 grid((H / 4 + kCombCG - 1) / kCombCG, M);
    MOE_LAUNCH(chan_combine_kernel, grid, dim3(MOE_WAVE), 0, stream, H, nchunks, part, y);
    return hipGetLastError();
}

hipError_t launch_channel_ranks(int E, int I, const float* norms, int32_t* ranks, hipStream_t stream) {
    if (I < 1 || I > kSelThreads * kSelPer) return hipErrorInvalidValue;
    hipLaunchKernelGGL(channel_ranks_kernel, dim3(E), dim3(kSelThreads), (size_t)I * sizeof(uint32_t), stream, I,
                       norms, ranks);
    return hipGetLastError();
}

hipError_t launch_channel_norms(int E, int I, int H, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                                float* norms, hipStream_t stream) {
    const int EI = E * I;
    MOE_LAUNCH(channel_norms_kernel, dim3((EI + kWaves - 1) / kWaves), dim3(kThreads), 0, stream, EI, H, Wg,
                       Wu, Wd, norms);
    return hipGetLastError();
}

}  // namespace moe

// Channel-sparse reads (page "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data", Background: channel j owns gate row j,
// up row j and down column j; Stage 2: top-k across all routed experts,
// exact compute of the kept channels, down stored transposed so that each
// d_j is contiguous).
//
// The score of candidate (slot s, channel j) is a_s * n[e_s][j]: the exact
// fp64 product of two fp32 values, so selection needs no rounding decision.
// The K best are found with an MSD radix select on the 64-bit order key of
// the score; ties at the threshold go to the lower expert id, then channel.
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

// Adds one to hist[d] for every lane with act set.  The scores of a token
// often share their leading digits, and LDS atomics of many lanes on one bin
// serialise in the CU's LDS: the lanes holding the digit of each of the
// first kHistLeaders pending lanes are counted with one atomic each, the rest
// (spread digits) add one per lane.
constexpr int kHistLeaders = 2;
__device__ __forceinline__ void wave_hist_add(int* hist, bool act, int d) {
    const int lane = threadIdx.x % MOE_WAVE;
    uint64_t pend = __ballot(act);
#pragma unroll
    for (int it = 0; it < kHistLeaders; ++it) {
        if (!pend) break;
        const int leader = __builtin_ctzll(pend);
        const int dl = __builtin_amdgcn_readlane(d, leader);
        const uint64_t same = __ballot(((pend >> lane) & 1ull) && d == dl);
        if (lane == leader) atomicAdd(&hist[dl], __builtin_popcountll(same));
        pend &= ~same;
    }
    if ((pend >> lane) & 1ull) atomicAdd(&hist[d], 1);
}

// One workgroup of kSelThreads per token; thread t owns the candidates
// idx = t*per .. t*per + per - 1 (per <= 8, idx = s*I + j) and keeps their
// keys in registers.  An MSD radix select over 8-bit digits narrows the
// leading bits of the K-th best key until its bucket holds exactly the
// candidates still needed; candidates above the bucket are kept, the
// bucket's too, and only if whole keys tie at the K-th place are the first
// `need` of them taken in (expert id, channel) order.  The kept list is
// written in candidate order.  LDS: a tie mark per candidate.
constexpr int kSelThreads = 1024;
constexpr int kSelPer = 8;

//
// ROUTE: the workgroup first routes its token from the router's slice
// partials -- the logits added in slice order (+ bias), the top-k (one wave
// from the keys above a threshold, else every key counted) and the
// renormalised softmax, with the router's arithmetic -- and writes the ids
// and affinities (and logits) as the router would.
template <bool ROUTE>
__global__ void __launch_bounds__(kSelThreads)
chan_select_kernel(const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
                   const float* __restrict__ norms, int k, int I, int E, int K, FastDiv fI,
                   int32_t* __restrict__ kept, SelRoute route) {
    extern __shared__ unsigned char lds[];
    const int n = k * I;
    unsigned char* tie = lds;            // [n], indexed in (expert, channel) order
    __shared__ double sa[32];
    __shared__ int se[32];
    __shared__ int spos[32];  // rank of slot s when slots are ordered by expert id
    __shared__ int hist[2][kSelThreads / MOE_WAVE][256];  // per wave, double-buffered
    __shared__ unsigned long long s_wmin[kSelThreads / MOE_WAVE], s_wmax[kSelThreads / MOE_WAVE];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_need;
    __shared__ int s_cnt;
    __shared__ int wsum[kSelThreads / MOE_WAVE];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;
    const int per = (n + kSelThreads - 1) / kSelThreads;  // <= kSelPer (n <= 8192)
    const int i0 = tid * per;

    if constexpr (ROUTE) {
        // keys in the histogram's LDS (not used before the radix passes)
        uint64_t* skey = reinterpret_cast<uint64_t*>(&hist[0][0][0]);
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
            if (route.logits) route.logits[(size_t)t * E + tid] = lg;
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
                route.ids[(size_t)t * k + tid] = sel_e[tid];
                route.wts[(size_t)t * k + tid] = w;
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
    __syncthreads();
    if (tid < k) {  // slots ordered by expert id (ids of one token are distinct; invalid slots last)
        const int e = se[tid];
        int pos = 0;
        for (int s2 = 0; s2 < k; ++s2) {
            const unsigned a = (unsigned)e, b2 = (unsigned)se[s2];  // -1 sorts last
            pos += (b2 < a || (b2 == a && s2 < tid)) ? 1 : 0;
        }
        spos[tid] = pos;
    }
    // keys of the owned candidates (norm loads issued together)
    unsigned long long key[kSelPer];
    int tpos[kSelPer];  // (expert, channel)-order position
    float nv[kSelPer];
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = min(i0 + u, n - 1);
        const int sl = fI.div(idx), j = idx - sl * I;
        const int e = se[sl];
        nv[u] = norms[(size_t)(e < 0 ? 0 : e) * I + j];
    }
    __syncthreads();  // spos ready
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = min(i0 + u, n - 1);
        const int sl = fI.div(idx), j = idx - sl * I;
        key[u] = se[sl] < 0 ? 0ull : score_key(sa[sl] * (double)nv[u]);
        tpos[u] = spos[sl] * I + j;
    }

    // Leading digits shared by every candidate's key cannot split them: the
    // passes start below them (min and max over all candidates, the zero keys
    // of invalid slots included, which then share no digit with valid ones).
    unsigned long long kmin = ~0ull, kmax = 0ull;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const bool v = u < per && i0 + u < n;
        kmin = v && key[u] < kmin ? key[u] : kmin;
        kmax = v && key[u] > kmax ? key[u] : kmax;
    }
#pragma unroll
    for (int m = 1; m < MOE_WAVE; m <<= 1) {
        const unsigned long long a = __shfl_xor(kmin, m, MOE_WAVE), c = __shfl_xor(kmax, m, MOE_WAVE);
        kmin = a < kmin ? a : kmin;
        kmax = c > kmax ? c : kmax;
    }
    if (lane == 0) {
        s_wmin[tid / MOE_WAVE] = kmin;
        s_wmax[tid / MOE_WAVE] = kmax;
    }
    for (int i = tid; i < 2 * (kSelThreads / MOE_WAVE) * 256; i += kSelThreads) (&hist[0][0][0])[i] = 0;
    __syncthreads();
    kmin = ~0ull;
    kmax = 0ull;
#pragma unroll
    for (int w = 0; w < kSelThreads / MOE_WAVE; ++w) {
        kmin = s_wmin[w] < kmin ? s_wmin[w] : kmin;
        kmax = s_wmax[w] > kmax ? s_wmax[w] : kmax;
    }
    const int p0 = __builtin_clzll((kmin ^ kmax) | 1ull) / 8;  // whole shared digits (<= 7)

    // MSD passes until the bucket holding the K-th key contains exactly the
    // candidates still needed (all of them kept), or the key is exhausted.
    // Each wave counts into its own histogram (LDS atomics of one wave on one
    // bin serialise, so concentrated digits would otherwise serialise all 16
    // waves); the scanning wave adds the 16 counts of a digit in wave order.
    // The histograms are double-buffered: the scan clears the next pass's.
    unsigned long long prefix = p0 > 0 ? kmax >> (64 - 8 * p0) : 0ull;
    int need = K, shift = 64 - 8 * p0, cnt = 0;
    for (int pass = p0; pass < 8; ++pass) {
        const int sh = 56 - 8 * pass;
        const int cur = pass & 1;
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            const bool act = u < per && i0 + u < n && (pass == 0 || (key[u] >> (sh + 8)) == prefix);
            wave_hist_add(hist[cur][tid / MOE_WAVE], act, (int)((key[u] >> sh) & 255ull));
        }
        __syncthreads();
        if (tid < MOE_WAVE) {
            // lane covers digits 255-4l .. 252-4l (descending)
            int c[4], tot = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                c[x] = 0;
#pragma unroll
                for (int w = 0; w < kSelThreads / MOE_WAVE; ++w) c[x] += hist[cur][w][255 - 4 * lane - x];
                tot += c[x];
            }
            int incl = tot;
#pragma unroll
            for (int d = 1; d < MOE_WAVE; d <<= 1) {
                const int y = __shfl_up(incl, d, MOE_WAVE);
                if (lane >= d) incl += y;
            }
            int before = incl - tot;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if (before < need && before + c[x] >= need) {
                    s_prefix = (prefix << 8) | (unsigned long long)(255 - 4 * lane - x);
                    s_need = need - before;
                    s_cnt = c[x];
                }
                before += c[x];
            }
        } else {
            for (int i = tid - MOE_WAVE; i < (kSelThreads / MOE_WAVE) * 256; i += kSelThreads - MOE_WAVE)
                (&hist[cur ^ 1][0][0])[i] = 0;
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
        cnt = s_cnt;
        shift = sh;
        if (cnt == need) break;  // uniform: every candidate of the bucket is kept
    }
    // kept: keys whose leading (64 - shift) bits exceed the bucket's, and of
    // the bucket either all (cnt == need) or, for whole-key ties, the first
    // `need` in (expert, channel) order
    const bool ties = cnt > need;  // only after the last pass: equal full keys
    if (ties) {
        for (int i = tid; i < n; i += kSelThreads) tie[i] = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kSelPer; ++u)
            if (u < per && i0 + u < n && (key[u] >> shift) == prefix) tie[tpos[u]] = 1;
        __syncthreads();
        int c = 0;
        for (int u = 0; u < per; ++u) c += i0 + u < n ? tie[i0 + u] : 0;
        int total;
        int rank = block_exclusive_scan<kSelThreads>(c, wsum, &total);
        for (int u = 0; u < per; ++u) {
            if (i0 + u >= n) break;
            const int is_tie = tie[i0 + u];
            if (is_tie && rank < need) tie[i0 + u] = 2;
            rank += is_tie;
        }
        __syncthreads();
    }
    // compaction of the kept candidates in candidate order
    unsigned takemask = 0;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        if (!(u < per && i0 + u < n)) continue;
        const unsigned long long top = key[u] >> shift;
        if (top > prefix || (top == prefix && (!ties || tie[tpos[u]] == 2))) takemask |= 1u << u;
    }
    int total;
    int pos = block_exclusive_scan<kSelThreads>(__builtin_popcount(takemask), wsum, &total);
#pragma unroll
    for (int u = 0; u < kSelPer; ++u)
        if ((takemask >> u) & 1u) {
            if (pos < K) kept[(size_t)t * K + pos] = i0 + u;  // exactly K are taken; never write past K
            ++pos;
        }
    (void)lane;
}

// Gate/up of KC = 4*2 kept channels (two per wave), scaled by the router
// weight, then their down rows summed over all H in kept order:
//   part[t][chunk][col] = sum_{q in chunk} (a_{s_q} * p_q) * d_q[col].
template <int Q, int CQ>
__global__ void __launch_bounds__(kThreads)
chan_gather_kernel(const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
                   const int32_t* __restrict__ kept, int k, int I, int E, int H, int K, const float* __restrict__ h,
                   const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu, const uint16_t* __restrict__ Wd,
                   float* __restrict__ part, FastDiv fI) {
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
    // Resolve the KC kept channels of the chunk: lane q of every wave takes
    // channel q0 + q (two rounds of vector loads at clamped addresses, then
    // broadcast), instead of a chain of dependent scalar loads.
    int ce[KC], cj[KC];
    float ca[KC];
    {
        const int q = lane % KC;
        const bool qin = q0 + q < K;
        const int v = kept[(size_t)t * K + min(q0 + q, K - 1)];
        const bool vin = qin && v >= 0 && v < k * I;
        const int vc = vin ? v : 0;
        const int s = fI.div(vc), j = vc - s * (int)fI.d;
        const int e = topk_ids[(size_t)t * k + s];
        const float a = topk_w[(size_t)t * k + s];
        const int ev = (vin && e >= 0 && e < E) ? e : -1;
#pragma unroll
        for (int qq = 0; qq < KC; ++qq) {
            ce[qq] = __builtin_amdgcn_readlane(ev, qq);
            cj[qq] = __builtin_amdgcn_readlane(j, qq);
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

template <int Q>
hipError_t gather_q(const int32_t* topk_ids, const float* topk_w, const int32_t* kept, int M, int k, int I, int E,
                    int H, int K, const float* h, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                    float* part, hipStream_t stream) {
    constexpr int KC = kWaves * 2;
    const dim3 grid((K + KC - 1) / KC, M);
    const int CQ = (H + 2047) / 2048;
    if (CQ <= 1)
        MOE_LAUNCH((chan_gather_kernel<Q, 1>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, kept, k, I,
                           E, H, K, h, Wg, Wu, Wd, part, FastDiv((uint32_t)I));
    else if (CQ <= 2)
        MOE_LAUNCH((chan_gather_kernel<Q, 2>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, kept, k, I,
                           E, H, K, h, Wg, Wu, Wd, part, FastDiv((uint32_t)I));
    else if (CQ <= 4)
        MOE_LAUNCH((chan_gather_kernel<Q, 4>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, kept, k, I,
                           E, H, K, h, Wg, Wu, Wd, part, FastDiv((uint32_t)I));
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

size_t chan_select_lds_bytes(int n) { return (size_t)n; }

hipError_t launch_chan_select(const int32_t* topk_ids, const float* topk_w, const float* norms, int M, int k, int I,
                              int E, int K, int32_t* kept, hipStream_t stream) {
    if (k * I > kSelThreads * kSelPer) return hipErrorInvalidValue;
    MOE_LAUNCH(chan_select_kernel<false>, dim3(M), dim3(kSelThreads), chan_select_lds_bytes(k * I), stream, topk_ids,
               topk_w, norms, k, I, E, K, FastDiv((uint32_t)I), kept, SelRoute{});
    return hipGetLastError();
}

hipError_t launch_chan_select_routed(const SelRoute& route, const float* norms, int M, int k, int I, int E, int K,
                                     int32_t* kept, hipStream_t stream) {
    if (k * I > kSelThreads * kSelPer || E > kSelThreads || k > 32 || route.M != M) return hipErrorInvalidValue;
    MOE_LAUNCH(chan_select_kernel<true>, dim3(M), dim3(kSelThreads), chan_select_lds_bytes(k * I), stream, nullptr,
               nullptr, norms, k, I, E, K, FastDiv((uint32_t)I), kept, route);
    return hipGetLastError();
}

hipError_t launch_chan_gather(const int32_t* topk_ids, const float* topk_w, const int32_t* kept, int M, int k, int I,
                              int E, int H, int K, int chunk, const float* h, const uint16_t* Wg, const uint16_t* Wu,
                              const uint16_t* Wd, float* part, hipStream_t stream) {
    (void)chunk;
    const int Q = (H + 511) / 512;
    if (Q <= 1) return gather_q<1>(topk_ids, topk_w, kept, M, k, I, E, H, K, h, Wg, Wu, Wd, part, stream);
    if (Q <= 2) return gather_q<2>(topk_ids, topk_w, kept, M, k, I, E, H, K, h, Wg, Wu, Wd, part, stream);
    if (Q <= 4) return gather_q<4>(topk_ids, topk_w, kept, M, k, I, E, H, K, h, Wg, Wu, Wd, part, stream);
    if (Q <= 8) return gather_q<8>(topk_ids, topk_w, kept, M, k, I, E, H, K, h, Wg, Wu, Wd, part, stream);
    if (Q <= 16) return gather_q<16>(topk_ids, topk_w, kept, M, k, I, E, H, K, h, Wg, Wu, Wd, part, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_chan_combine(int M, int H, int nchunks, const float* part, float* y, hipStream_t stream) {
    const dim3 grid((H / 4 + kCombCG - 1) / kCombCG, M);
    MOE_LAUNCH(chan_combine_kernel, grid, dim3(MOE_WAVE), 0, stream, H, nchunks, part, y);
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

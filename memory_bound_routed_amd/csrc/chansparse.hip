// Channel-sparse reads (page "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data", Background: channel j owns gate row j,
// up row j and down column j; Stage 2: top-k across all routed experts,
// exact compute of the kept channels, down stored transposed so that each
// d_j is contiguous).
//
// Two scores.  Static mode: candidate (slot s, channel j) scores a_s *
// n[e_s][j], the exact fp64 product of two fp32 values, so selection needs no
// rounding decision.  Reader mode (Stage 2): the output-level score
// w_s * ||d_j|| * |SiLU(g_hat_j) * v_hat_j| of the sketch estimates, in fp32
// (reader_device.h).  Every gather workgroup of a token takes the K best
// exactly (select_device.h), ties to the lower expert id, then channel, then
// slot, computes its share of the kept channels exactly and writes a chunk
// partial that the combine adds in order.
#include <algorithm>
#include <climits>

#include "device_common.h"
#include "launch.h"
#include "reader_device.h"
#include "select_device.h"
#include "topk_device.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kBufferFlags = 0x00020000;  // fourth word of a raw gfx9 buffer descriptor (32-bit data)

// Order-preserving map of a double score to uint64 (larger score -> larger key).
__device__ __forceinline__ unsigned long long score_key(double x) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Selection and gather in one launch.  Grid (ceil(K / 8) chunks, M tokens),
// 1024 threads.  Every workgroup of a token takes the token's K best
// candidates (slot s, channel j) exactly -- the same arithmetic in each, so
// the same set -- then computes the kept candidates at positions 8 c ..
// 8 c + 7 of the candidate order (s * I + j ascending):
//   part[t][c][col] = sum over those (s, j), in position order, of
//                     (a_s * SiLU(g_j . h_t) * (v_j . h_t)) * d_j[col].
// The selection's latency is paid once per workgroup, in parallel, instead of
// in a launch of its own followed by list reads.
//
// MODE 0: candidate (s, j) scores a_s * n[e_s][j], the exact fp64 product of
// two fp32 values; ranked by that score (descending), then expert id,
// channel and slot (ascending); a slot whose expert id is invalid contributes
// candidates below every valid one, in channel order.  select_top takes the
// K best by bins linear in the score (as fp32) between the token's minimum
// and maximum -- invalid slots in a bin of their own below them -- and,
// inside the threshold bin, the 64-bit order key of the fp64 score (high and
// low words) and the complement of the tie key e << 19 | j << 5 | s.
// ROUTE (MODE 0): each workgroup first routes its token from the router's
// slice partials -- the logits added in slice order (+ bias), the top-k (one
// wave from the keys above a threshold, else every key counted) and the
// renormalised softmax, with the router's arithmetic; workgroup 0 writes the
// ids and affinities (and logits) as the router would.
// MODE 1: the reader's scores (reader_scores: the sketch estimates and
// (w_s ||d_j||) |SiLU(g_hat) v_hat|), bins linear in the score, then the
// score bits and the tie key.
//
// Gather: wave w computes projection w % 2 (gate, up) of the chunk's kept
// channel w / 2 -- lane l over hidden columns 8 (l + 64 q), h staged in LDS,
// the lanes added by wave_sum; threads 0..255 then add the 8 down rows
// scaled by a_s * SiLU(g) * u, in position order, at columns 8 (tid + 256 cq).
// Workgroup (0, t) also writes the kept flags (kept_flag[t][s][j], when
// asked) and every workgroup its positions of kept_out.
constexpr int kGatherKC = 8;  // kept channels per workgroup (two waves each)

struct SparseArgs {
    int32_t* topk_ids;        // [M][k] in (out with ROUTE)
    float* topk_w;            // [M][k] in (out with ROUTE)
    const float* norms;       // MODE 0: fp32 [E][I]
    ReaderArgs ra;            // MODE 1
    SelRoute route;           // ROUTE
    int k, I, E, H, K;
    const float* h;
    const uint16_t* Wg;
    const uint16_t* Wu;
    const uint16_t* Wd;
    float* part;              // fp32 [M][nchunks][H]
    int32_t* kept_out;        // int32 [M][K] or null
    uint8_t* kept_flag;       // u8 [M][k][I] or null
};

template <int MODE, bool ROUTE, int Q, int CQ>
__global__ void __launch_bounds__(kSelThreads)
chan_topk_gather_kernel(SparseArgs A, FastDiv fI) {
    constexpr int KC = kGatherKC;
    __shared__ int se[32];
    __shared__ float sa[32];
    __shared__ RadixLds rl;
    __shared__ float4 hs[Q * MOE_WAVE * 2];  // h of the token (8 floats per lane and q)
    __shared__ int ce[KC], cj[KC];
    __shared__ float ca[KC];
    __shared__ float gu[KC][2];
    __shared__ float cs[KC];
    const int t = blockIdx.y;
    const int chunk = blockIdx.x;
    const int nchunks = gridDim.x;
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE, lane = tid % MOE_WAVE;
    const int k = A.k, I = A.I, E = A.E, H = A.H, K = A.K;
    const int n = k * I;
    const int q0 = chunk * KC;

    // h first: it depends on nothing (staged in LDS once the selection's own
    // loads are in flight)
    constexpr int HF4 = Q * MOE_WAVE * 2;  // float4 of h (padded)
    constexpr int HPT = (HF4 + kSelThreads - 1) / kSelThreads;
    float4 hreg[HPT];
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
        const int f = min(tid + kSelThreads * u, HF4 - 1);
        hreg[u] = *reinterpret_cast<const float4*>(A.h + (size_t)t * H + min(4 * f, H - 4));
    }

    unsigned kmask = 0;
    bool all = K >= n;
    if constexpr (MODE == 0) {
        if constexpr (ROUTE) {
            // the token's routing (the router's arithmetic); chunk 0 stores
            // the ids, weights and logits
            const SelRoute& route = A.route;
            __shared__ RouteLds<kSelThreads> rlt;
            route_token<kSelThreads>(route.part, route.bias, route.nslices, route.M, t, E, k, chunk == 0,
                                     route.logits, A.topk_ids, A.topk_w, rlt);
            if (tid < k) {
                se[tid] = rlt.sel_e[tid];
                sa[tid] = rlt.sel_w[tid];
            }
        } else {
            if (tid < k) {
                const int e = A.topk_ids[(size_t)t * k + tid];
                se[tid] = (e >= 0 && e < E) ? e : -1;
                sa[tid] = A.topk_w[(size_t)t * k + tid];
            }
        }
        __syncthreads();
        // the norms of the thread's candidates: 16-byte loads when they are 8
        // consecutive channels of one slot (I % 8 == 0), else one by one
        float nv[kSelPer];
        if (I % kSelPer == 0) {  // uniform
            const int ic = min(kSelPer * tid, n - kSelPer);
            const int s = fI.div(ic), j = ic - s * I;
            // two 16-byte buffer loads (plain vector loads here are split
            // into eight 4-byte loads by the compiler; the load count, not
            // the bytes, is what this latency-bound phase pays for)
            const __amdgpu_buffer_rsrc_t nr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(A.norms), (short)0, E * I * 4, kBufferFlags);
            const int off = (max(se[s], 0) * I + j) * 4;
            const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(nr, off, 0, 0);
            const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(nr, off + 16, 0, 0);
            nv[0] = __uint_as_float(a.x); nv[1] = __uint_as_float(a.y);
            nv[2] = __uint_as_float(a.z); nv[3] = __uint_as_float(a.w);
            nv[4] = __uint_as_float(b.x); nv[5] = __uint_as_float(b.y);
            nv[6] = __uint_as_float(b.z); nv[7] = __uint_as_float(b.w);
        } else {
#pragma unroll
            for (int u = 0; u < kSelPer; ++u) {
                const int ic = min(kSelPer * tid + u, n - 1);
                const int s = fI.div(ic), j = ic - s * I;
                nv[u] = A.norms[(size_t)max(se[s], 0) * I + j];
            }
        }
#pragma unroll
        for (int u = 0; u < HPT; ++u)
            if (tid + kSelThreads * u < HF4) hs[tid + kSelThreads * u] = hreg[u];
        double sc[kSelPer];
        uint32_t key[3][kSelPer];
        unsigned vmask = 0, bmask = 0;  // candidates; candidates of valid slots
        uint32_t fmax = 0, fmin = 0xFFFFFFFFu;
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            const int idx = kSelPer * tid + u;
            const int ic = min(idx, n - 1);
            const int s = fI.div(ic), j = ic - s * I;
            const int e = se[s];
            sc[u] = (double)sa[s] * (double)nv[u] + 0.0;  // exact; -0 as +0
            const unsigned long long kk = e < 0 ? 0ull : score_key(sc[u]);
            key[0][u] = (uint32_t)(kk >> 32);
            key[1][u] = (uint32_t)kk;
            key[2][u] = ~(((uint32_t)(e < 0 ? 8191 : e) << 19) | ((uint32_t)j << 5) | (uint32_t)s);
            vmask |= idx < n ? (1u << u) : 0u;
            if (idx < n && e >= 0) {
                bmask |= 1u << u;
                const uint32_t fk = float_order_key((float)sc[u]);
                fmax = max(fmax, fk);
                fmin = min(fmin, fk);
            }
        }
        kmask = vmask;
        if (!all) {
            // bins linear in the score (as fp32) between the token's minimum
            // and maximum; invalid slots in bin 0, below every valid candidate
            uint32_t mx, mn;
            block_max_min(fmax, fmin, rl, &mx, &mn);
            const float lo = float_of_order_key(mn);
            const float scl = linear_scale(lo, float_of_order_key(mx), kRadixBins - 1);
            int bin[kSelPer];
#pragma unroll
            for (int u = 0; u < kSelPer; ++u)
                bin[u] = ((bmask >> u) & 1u) ? 1 + linear_bin((float)sc[u], lo, scl, kRadixBins - 1) : 0;
            kmask = select_top<3>(bin, key, vmask, K, rl);
        }
    } else {
        if (tid < k) {
            const int e = A.topk_ids[(size_t)t * k + tid];
            se[tid] = (e >= 0 && e < E) ? e : -1;
            sa[tid] = A.topk_w[(size_t)t * k + tid];
        }
        __syncthreads();
        uint32_t sb[kSelPer], tb[kSelPer], smax, smin;
        unsigned vmask;
        reader_scores(A.ra, t, fI, se, sa, sb, tb, vmask, smax, smin, nullptr, nullptr);
#pragma unroll
        for (int u = 0; u < HPT; ++u)
            if (tid + kSelThreads * u < HF4) hs[tid + kSelThreads * u] = hreg[u];
        kmask = vmask;
        if (!all) {
            uint32_t mx, mn;
            block_max_min(smax, smin, rl, &mx, &mn);  // non-negative scores: bits order like values
            const float lo = __uint_as_float(mn);
            const float scl = linear_scale(lo, __uint_as_float(mx), kRadixBins);
            int bin[kSelPer];
            uint32_t key[2][kSelPer];
#pragma unroll
            for (int u = 0; u < kSelPer; ++u) {
                bin[u] = linear_bin(__uint_as_float(sb[u]), lo, scl, kRadixBins);
                key[0][u] = sb[u];
                key[1][u] = ~tb[u];
            }
            kmask = select_top<2>(bin, key, vmask, K, rl);
        }
    }

    // positions of the kept candidates in candidate order; the chunk's own
    if (tid < KC) ce[tid] = -1;
    const int cntk = __builtin_popcount(kmask);
    int incl = cntk;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int y = __shfl_up(incl, d, MOE_WAVE);
        if (lane >= d) incl += y;
    }
    if (lane == MOE_WAVE - 1) rl.wsum[wave] = incl;
    __syncthreads();
    int pos = incl - cntk;
    for (int x = 0; x < wave; ++x) pos += rl.wsum[x];
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int idx = kSelPer * tid + u;
        if (idx >= n) continue;
        const bool kept = (kmask >> u) & 1u;
        const int s = fI.div(idx), j = idx - s * I;
        if (A.kept_flag && chunk == 0) A.kept_flag[((size_t)t * k + s) * I + j] = kept ? 1 : 0;
        if (!kept) continue;
        if (pos >= q0 && pos < q0 + KC) {
            ce[pos - q0] = se[s];
            cj[pos - q0] = j;
            ca[pos - q0] = sa[s];
            if (A.kept_out) A.kept_out[(size_t)t * K + pos] = idx;
        }
        ++pos;
    }
    __syncthreads();

    // gather: every load of the chunk first (gate or up row of one channel
    // per wave, the down rows of all of them in threads 0..255)
    const int qc = wave >> 1, P = wave & 1;
    const int ec = ce[qc];
    const bool okc = ec >= 0;
    const size_t rowc = okc ? ((size_t)ec * I + cj[qc]) * H : 0;
    const uint16_t* W = P ? A.Wu : A.Wg;
    uint4 wv[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int col = (lane + MOE_WAVE * q) * 8;
        wv[q] = (okc && col < H) ? load_stream16(W + rowc + col) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint4 wd[KC];
    auto load_down = [&](int cq) {
#pragma unroll
        for (int qq = 0; qq < KC; ++qq) {
            const bool ok = ce[qq] >= 0;
            const size_t row = ok ? ((size_t)ce[qq] * I + cj[qq]) * H : 0;
            const int col = (tid + kThreads * cq) * 8;
            wd[qq] = (ok && col < H && tid < kThreads) ? load_stream16(A.Wd + row + col) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    load_down(0);
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int col = (lane + MOE_WAVE * q) * 8;
        if (col >= H) continue;
        const float4 h0 = hs[2 * (lane + MOE_WAVE * q)], h1 = hs[2 * (lane + MOE_WAVE * q) + 1];
        const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        float f[8];
        unpack8(wv[q], f);
#pragma unroll
        for (int x = 0; x < 8; ++x) acc = fmaf(f[x], hv[x], acc);
    }
    const float dot = wave_sum(acc);
    if (lane == 0) gu[qc][P] = dot;
    __syncthreads();
    if (tid < KC) cs[tid] = ce[tid] >= 0 ? ca[tid] * silu_mul(gu[tid][0], gu[tid][1]) : 0.f;
    __syncthreads();
    if (tid < kThreads) {
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq) {
            if (cq > 0) load_down(cq);
            const int col = (tid + kThreads * cq) * 8;
            if (col >= H) continue;
            float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qq = 0; qq < KC; ++qq) {
                float wf[8];
                unpack8(wd[qq], wf);
                const float c = cs[qq];
#pragma unroll
                for (int x = 0; x < 8; ++x) o[x] = fmaf(c, wf[x], o[x]);
            }
            float* dst = A.part + ((size_t)t * nchunks + chunk) * H + col;
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
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

}  // namespace

template <int MODE, bool ROUTE>
hipError_t topk_gather(const SparseArgs& a, int M, hipStream_t stream) {
    const int Q = (a.H + 511) / 512;
    const dim3 grid((a.K + kGatherKC - 1) / kGatherKC, M);
    const FastDiv fI((uint32_t)a.I);
#define MOE_TG(QQ, CQQ) MOE_LAUNCH((chan_topk_gather_kernel<MODE, ROUTE, QQ, CQQ>), grid, dim3(kSelThreads), 0, stream, \
                                   a, fI)
    if (Q <= 4) MOE_TG(4, 1);
    else if (Q <= 8) MOE_TG(8, 2);
    else if (Q <= 16) MOE_TG(16, 4);
    else return hipErrorInvalidValue;
#undef MOE_TG
    return hipGetLastError();
}

hipError_t launch_chan_topk_gather(int mode, const SelRoute* route, int32_t* topk_ids, float* topk_w,
                                   const float* norms, const ReaderArgs* ra, int M, int k, int I, int E, int H, int K,
                                   const float* h, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                                   float* part, int32_t* kept_out, uint8_t* kept_flag, hipStream_t stream) {
    if (k * I > kSelThreads * kSelPer || k > 32 || E > 8192 || I > 16384 || K < 1 || K > k * I || M < 1 ||
        H % 8 || H > 8192)
        return hipErrorInvalidValue;
    SparseArgs a{};
    a.topk_ids = topk_ids;
    a.topk_w = topk_w;
    a.norms = norms;
    if (ra) a.ra = *ra;
    a.k = k;
    a.I = I;
    a.E = E;
    a.H = H;
    a.K = K;
    a.h = h;
    a.Wg = Wg;
    a.Wu = Wu;
    a.Wd = Wd;
    a.part = part;
    a.kept_out = kept_out;
    a.kept_flag = kept_flag;
    if (mode == 1) {
        if (!ra || route || ra->nbq < 1 || ra->nbq > kReaderMaxGroups || ra->I != I || ra->k != k) return hipErrorInvalidValue;
        return topk_gather<1, false>(a, M, stream);
    }
    if (route) {
        if (E > kSelThreads || route->M != M) return hipErrorInvalidValue;
        a.route = *route;
        return topk_gather<0, true>(a, M, stream);
    }
    return topk_gather<0, false>(a, M, stream);
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

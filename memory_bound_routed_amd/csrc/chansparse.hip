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

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;

// Order-preserving map of a double to uint64 (larger double -> larger key).
__device__ __forceinline__ unsigned long long order_key(double x) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Exclusive scan of one int per thread over the workgroup; returns the
// exclusive prefix and writes the total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
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
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) base += wsum[w];
        all += wsum[w];
    }
    __syncthreads();
    *total = all;
    return base + x - v;
}

// One workgroup per token.  LDS: the token's candidate norms (fp32 [n]), a
// tie flag and a take flag per candidate.
__global__ void __launch_bounds__(kThreads)
chan_select_kernel(const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
                   const float* __restrict__ norms, int k, int I, int E, int K, int32_t* __restrict__ kept) {
    extern __shared__ unsigned char lds[];
    const int n = k * I;
    float* sn = reinterpret_cast<float*>(lds);                // [n]
    unsigned char* tie = lds + (size_t)n * sizeof(float);     // [n], indexed in (expert, channel) order
    unsigned char* take = tie + n;                            // [n], natural (slot, channel) order
    __shared__ double sa[32];
    __shared__ int se[32];
    __shared__ int spos[32];  // rank of slot s when slots are ordered by expert id
    __shared__ int hist[256];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_need;
    __shared__ int wsum[kWaves];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;

    if (tid < k) {
        const int e = topk_ids[(size_t)t * k + tid];
        se[tid] = (e >= 0 && e < E) ? e : -1;
        sa[tid] = (double)topk_w[(size_t)t * k + tid];
    }
    __syncthreads();
    if (tid < k) {  // slots ordered by expert id (ids of one token are distinct; invalid slots last)
        const int e = se[tid];
        int pos = 0;
        for (int s2 = 0; s2 < k; ++s2) {
            const int e2 = se[s2];
            const unsigned a = (unsigned)e, b2 = (unsigned)e2;  // -1 sorts last
            pos += (b2 < a || (b2 == a && s2 < tid)) ? 1 : 0;
        }
        spos[tid] = pos;
    }
    for (int idx = tid; idx < n; idx += kThreads) {
        const int s = idx / I, j = idx % I;
        const int e = se[s];
        sn[idx] = e >= 0 ? norms[(size_t)e * I + j] : 0.f;
    }
    __syncthreads();

    auto key_of = [&](int idx) -> unsigned long long {
        const int s = idx / I;
        if (se[s] < 0) return 0ull;
        return order_key(sa[s] * (double)sn[idx]);
    };

    unsigned long long prefix = 0;
    int need = K;
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int idx = tid; idx < n; idx += kThreads) {
            const unsigned long long key = key_of(idx);
            if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&hist[(key >> shift) & 255ull], 1);
        }
        __syncthreads();
        if (tid < MOE_WAVE) {
            // lane covers digits 255-4l .. 252-4l (descending)
            int c[4], tot = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) { c[x] = hist[255 - 4 * lane - x]; tot += c[x]; }
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
                }
                before += c[x];
            }
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
        __syncthreads();
    }
    const unsigned long long T = prefix;  // key of the K-th best candidate

    // take: above the threshold, or one of the first `need` ties in (expert, channel) order
    for (int idx = tid; idx < n; idx += kThreads) {
        const unsigned long long key = key_of(idx);
        const int s = idx / I, j = idx % I;
        take[idx] = key > T ? 1 : 0;
        tie[spos[s] * I + j] = key == T ? 1 : 0;
    }
    __syncthreads();
    const int per = (n + kThreads - 1) / kThreads;
    {
        const int u0 = tid * per, u1 = min(n, u0 + per);
        int c = 0;
        for (int u = u0; u < u1; ++u) c += tie[u];
        int total;
        int rank = block_exclusive_scan(c, wsum, &total);
        for (int u = u0; u < u1; ++u) {
            const int is_tie = tie[u];
            tie[u] = (is_tie && rank < need) ? 2 : is_tie;
            rank += is_tie;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < n; idx += kThreads) {
        const int s = idx / I, j = idx % I;
        if (tie[spos[s] * I + j] == 2) take[idx] = 1;
    }
    __syncthreads();
    {
        const int i0 = tid * per, i1 = min(n, i0 + per);
        int c = 0;
        for (int i = i0; i < i1; ++i) c += take[i];
        int total;
        int pos = block_exclusive_scan(c, wsum, &total);
        for (int i = i0; i < i1; ++i)
            if (take[i]) {
                if (pos < K) kept[(size_t)t * K + pos] = i;  // exactly K are taken; never write past K
                ++pos;
            }
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

    // resolve all KC kept channels of the chunk (uniform per workgroup)
    int ce[KC], cj[KC];
    float ca[KC];
#pragma unroll
    for (int qq = 0; qq < KC; ++qq) {
        ce[qq] = -1; cj[qq] = 0; ca[qq] = 0.f;
        if (q0 + qq < K) {
            const int v = kept[(size_t)t * K + q0 + qq];
            const int s = v / I;
            if (v >= 0 && s < k) {
                const int e = topk_ids[(size_t)t * k + s];
                if (e >= 0 && e < E) { ce[qq] = e; cj[qq] = v % I; ca[qq] = topk_w[(size_t)t * k + s]; }
            }
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
        const float4 h0 = *reinterpret_cast<const float4*>(h + (size_t)t * H + col);
        const float4 h1 = *reinterpret_cast<const float4*>(h + (size_t)t * H + col + 4);
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

// y[t][col] = sum over chunks (ascending) of part[t][chunk][col].
__global__ void __launch_bounds__(kThreads)
chan_combine_kernel(int H, int nchunks, const float* __restrict__ part, float* __restrict__ y) {
    const int t = blockIdx.y;
    const int col = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (col >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* src = part + (size_t)t * nchunks * H + col;
    for (int c = 0; c < nchunks; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(src + (size_t)c * H);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(y + (size_t)t * H + col) = acc;
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
                           E, H, K, h, Wg, Wu, Wd, part);
    else if (CQ <= 2)
        MOE_LAUNCH((chan_gather_kernel<Q, 2>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, kept, k, I,
                           E, H, K, h, Wg, Wu, Wd, part);
    else if (CQ <= 4)
        MOE_LAUNCH((chan_gather_kernel<Q, 4>), grid, dim3(kThreads), 0, stream, topk_ids, topk_w, kept, k, I,
                           E, H, K, h, Wg, Wu, Wd, part);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

size_t chan_select_lds_bytes(int n) { return (size_t)n * (sizeof(float) + 2); }

hipError_t launch_chan_select(const int32_t* topk_ids, const float* topk_w, const float* norms, int M, int k, int I,
                              int E, int K, int32_t* kept, hipStream_t stream) {
    MOE_LAUNCH(chan_select_kernel, dim3(M), dim3(kThreads), chan_select_lds_bytes(k * I), stream, topk_ids,
                       topk_w, norms, k, I, E, K, kept);
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
    const dim3 grid((H / 4 + kThreads - 1) / kThreads, M);
    MOE_LAUNCH(chan_combine_kernel, grid, dim3(kThreads), 0, stream, H, nchunks, part, y);
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

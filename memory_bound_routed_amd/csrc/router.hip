// Router: skinny bf16 GEMV partials and the wavefront top-k with the
// renormalised softmax (page "A Multi-Engine Dataflow for MoE Decoding on
// Scratchpad-Based Tensor Accelerators", MoE-block background; page
// "Route-Block Membership Selects Packed-AWQ Arithmetic", Sec. 2.1).
//
// The GEMV kernel also serves the routing-independent shared projection
// z = D^T h of the VQ + low-rank format (same shape: h [M][H] times a bf16
// [H][N] matrix), so both can share one launch.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kGemvThreads = 256;
constexpr int kTokTile = 4;
constexpr int kMaxJobs = 3;

struct GemvJobs {
    GemvJob job[kMaxJobs];
};

// One workgroup per (row slice, matrix).  Thread layout: N/8 threads cover a
// row with one 16-byte load each, 256/(N/8) rows are in flight per pass.
// Per-thread partial sums run over the slice's rows in ascending order, the
// row groups are then added pairwise in LDS (a fixed tree), and the result is
// the slice partial.  The total summation depth of a logit is therefore at
// most ceil(slice_rows/rpp) + ceil(log2 rpp) + nslices (+1 for a bias).
__global__ void __launch_bounds__(kGemvThreads)
gemv_partials_kernel(const float* __restrict__ h, int M, int H, int slice_rows, GemvJobs jobs) {
    extern __shared__ float red[];  // [rpp][kTokTile][N]
    const GemvJob& jb = jobs.job[blockIdx.y];
    const int N = jb.N;
    const uint16_t* __restrict__ W = jb.W;
    const int tpr = N >> 3;
    const int rpp = kGemvThreads / tpr;
    const int tid = threadIdx.x;
    const int col8 = tid % tpr;
    const int rg = tid / tpr;
    const bool active = rg < rpp;
    const int r0 = blockIdx.x * slice_rows;
    const int r1 = min(H, r0 + slice_rows);

    for (int t0 = 0; t0 < M; t0 += kTokTile) {
        const int nt = min(kTokTile, M - t0);
        if (active) {
            float acc[kTokTile][8];
#pragma unroll
            for (int t = 0; t < kTokTile; ++t)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[t][c] = 0.f;
            for (int i = r0 + rg; i < r1; i += rpp) {
                float wf[8];
                unpack8(load16(W + (size_t)i * N + col8 * 8), wf);
#pragma unroll
                for (int t = 0; t < kTokTile; ++t) {
                    if (t < nt) {
                        const float hv = h[(size_t)(t0 + t) * H + i];
#pragma unroll
                        for (int c = 0; c < 8; ++c) acc[t][c] = fmaf(hv, wf[c], acc[t][c]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < kTokTile; ++t)
#pragma unroll
                for (int c = 0; c < 8; ++c) red[(rg * kTokTile + t) * N + col8 * 8 + c] = acc[t][c];
        }
        __syncthreads();
        // pairwise tree over the rpp row groups: cnt -> ceil(cnt/2)
        for (int cnt = rpp; cnt > 1;) {
            const int half = (cnt + 1) >> 1;
            const int pairs = cnt - half;
            for (int idx = tid; idx < pairs * kTokTile * N; idx += kGemvThreads) {
                const int g = idx / (kTokTile * N);
                const int rest = idx % (kTokTile * N);
                red[g * kTokTile * N + rest] += red[(g + half) * kTokTile * N + rest];
            }
            cnt = half;
            __syncthreads();
        }
        for (int idx = tid; idx < nt * N; idx += kGemvThreads) {
            const int t = idx / N, n = idx % N;
            jb.part[((size_t)blockIdx.x * M + t0 + t) * N + n] = red[t * N + n];
        }
        __syncthreads();
    }
}

constexpr int kMaxExpertsPerLane = 16;  // E <= 1024

// One wave per token.  Lane l holds the logits of experts l, l+64, ...; the
// slice partials are added in slice order, then the bias.  Each of the k
// rounds takes the largest remaining logit with a wave-wide reduction under
// the total order (logit descending, expert id ascending), so the winner does
// not depend on the reduction tree.  NaN logits rank below every number.
__global__ void __launch_bounds__(MOE_WAVE)
router_topk_kernel(const float* __restrict__ part, int nslices, int M, int E, int k,
                   const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ wts,
                   float* __restrict__ logits_out) {
    const int t = blockIdx.x;
    const int lane = threadIdx.x;
    float v[kMaxExpertsPerLane];
#pragma unroll
    for (int q = 0; q < kMaxExpertsPerLane; ++q) {
        const int e = lane + MOE_WAVE * q;
        float s = -INFINITY;
        if (e < E) {
            s = 0.f;
            for (int sl = 0; sl < nslices; ++sl) s += part[((size_t)sl * M + t) * E + e];
            if (bias) s += bias[e];
            if (logits_out) logits_out[(size_t)t * E + e] = s;
            if (s != s) s = -INFINITY;
        }
        v[q] = s;
    }
    uint32_t taken = 0;
    float my_l = -INFINITY;  // lane s keeps slot s
    int my_e = 0;
    for (int s = 0; s < k; ++s) {
        float bv = -INFINITY;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < kMaxExpertsPerLane; ++q) {
            const int e = lane + MOE_WAVE * q;
            if (e < E && !((taken >> q) & 1u)) {
                if (v[q] > bv || (v[q] == bv && e < be)) { bv = v[q]; be = e; }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, MOE_WAVE);
            const int oe = __shfl_xor(be, off, MOE_WAVE);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        if ((be & (MOE_WAVE - 1)) == lane) taken |= 1u << (be / MOE_WAVE);
        if (lane == s) { my_l = bv; my_e = be; }
    }
    // softmax over the selected logits, shifted by the largest one; the
    // denominator adds the slots in slot order
    const float l0 = __shfl(my_l, 0, MOE_WAVE);
    const float x = (lane < k) ? expf(my_l - l0) : 0.f;
    float den = 0.f;
    for (int s = 0; s < k; ++s) den += __shfl(x, s, MOE_WAVE);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        wts[(size_t)t * k + lane] = x / den;
    }
}

}  // namespace

hipError_t launch_gemv_partials(const float* h, int M, int H, int slice_rows, const GemvJob* jobs, int njobs,
                                hipStream_t stream) {
    if (njobs < 1 || njobs > kMaxJobs) return hipErrorInvalidValue;
    GemvJobs js{};
    int maxN = 0;
    for (int i = 0; i < njobs; ++i) {
        js.job[i] = jobs[i];
        maxN = jobs[i].N > maxN ? jobs[i].N : maxN;
    }
    // LDS: rpp * kTokTile * N floats; rpp * N <= 256 * 8 for every N
    size_t lds = 0;
    for (int i = 0; i < njobs; ++i) {
        const int tpr = jobs[i].N / 8;
        const size_t b = (size_t)(kGemvThreads / tpr) * kTokTile * jobs[i].N * sizeof(float);
        lds = b > lds ? b : lds;
    }
    const int nslices = (H + slice_rows - 1) / slice_rows;
    hipLaunchKernelGGL(gemv_partials_kernel, dim3(nslices, njobs), dim3(kGemvThreads), lds, stream, h, M, H,
                       slice_rows, js);
    return hipGetLastError();
}

hipError_t launch_router_topk(const float* part, int nslices, int M, int E, int k, const float* bias,
                              int32_t* ids, float* wts, float* logits_out, hipStream_t stream) {
    hipLaunchKernelGGL(router_topk_kernel, dim3(M), dim3(MOE_WAVE), 0, stream, part, nslices, M, E, k, bias, ids,
                       wts, logits_out);
    return hipGetLastError();
}

}  // namespace moe

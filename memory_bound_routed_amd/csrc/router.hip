// Router: bf16 GEMV over row slices, then -- in the last workgroup to finish
// -- the fixed-order sum of the slices, the wavefront top-k and the
// renormalised softmax, all in one launch (page "A Multi-Engine Dataflow for
// MoE Decoding on Scratchpad-Based Tensor Accelerators", MoE-block
// background; page "Route-Block Membership Selects Packed-AWQ Arithmetic",
// Sec. 2.1: the router's M x k expert-id array).
//
// The same row-slice GEMV (without the top-k) computes the
// routing-independent shared projection z = D^T h of the VQ + low-rank
// format.
#include "align_device.h"
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kTokTile = 4;
constexpr int kRowsPerThread = 4;
constexpr int kMaxJobs = 3;
constexpr int kMaxExpertsPerLane = 16;  // E <= 1024

struct GemvJobs {
    GemvJob job[kMaxJobs];
};

// Slice partial of one matrix: part[slice][t][n] = sum_{i in slice} h[t][i] W[i][n].
// N/8 threads cover a row with one 16-byte load each; rpp = 256/(N/8) row
// groups; each thread handles kRowsPerThread rows of the slice (all loads
// issued together), the row groups are added pairwise in LDS.  Summation
// depth per partial: kRowsPerThread + ceil(log2 rpp).
template <int TT>
__device__ __forceinline__ void slice_partial(const float* __restrict__ h, int M, int H,
                                              const uint16_t* __restrict__ W, int N, int slice, float* __restrict__ part,
                                              float* red) {
    const int tpr = N >> 3;
    const int rpp = kThreads / tpr;
    const int tid = threadIdx.x;
    const int col8 = tid % tpr;
    const int rg = tid / tpr;
    const bool active = rg < rpp;
    const int slice_rows = rpp * kRowsPerThread;
    const int r0 = slice * slice_rows;

    for (int t0 = 0; t0 < M; t0 += TT) {
        const int nt = min(TT, M - t0);
        if (active) {
            float wf[kRowsPerThread][8];
            float hv[kRowsPerThread][TT];
#pragma unroll
            for (int u = 0; u < kRowsPerThread; ++u) {
                const int i = r0 + rg + u * rpp;
                if (i < H) {
                    unpack8(load_stream16(W + (size_t)i * N + col8 * 8), wf[u]);
#pragma unroll
                    for (int t = 0; t < TT; ++t) hv[u][t] = t < nt ? h[(size_t)(t0 + t) * H + i] : 0.f;
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) wf[u][c] = 0.f;
#pragma unroll
                    for (int t = 0; t < TT; ++t) hv[u][t] = 0.f;
                }
            }
            float acc[TT][8];
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[t][c] = 0.f;
#pragma unroll
            for (int u = 0; u < kRowsPerThread; ++u)
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[t][c] = fmaf(hv[u][t], wf[u][c], acc[t][c]);
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int c = 0; c < 8; ++c) red[(rg * TT + t) * N + col8 * 8 + c] = acc[t][c];
        }
        __syncthreads();
        for (int cnt = rpp; cnt > 1;) {
            const int half = (cnt + 1) >> 1;
            const int pairs = cnt - half;
            for (int idx = tid; idx < pairs * TT * N; idx += kThreads) {
                const int g = idx / (TT * N);
                const int rest = idx % (TT * N);
                red[g * TT * N + rest] += red[(g + half) * TT * N + rest];
            }
            cnt = half;
            __syncthreads();
        }
        for (int idx = tid; idx < nt * N; idx += kThreads) {
            const int t = idx / N, n = idx % N;
            part[((size_t)slice * M + t0 + t) * N + n] = red[t * N + n];
        }
        __syncthreads();
    }
}

__global__ void __launch_bounds__(kThreads)
gemv_partials_kernel(const float* __restrict__ h, int M, int H, GemvJobs jobs) {
    extern __shared__ float red[];
    const GemvJob& jb = jobs.job[blockIdx.y];
    const int rpp = kThreads / (jb.N >> 3);
    const int nslices = (H + rpp * kRowsPerThread - 1) / (rpp * kRowsPerThread);
    if ((int)blockIdx.x >= nslices) return;
    if (M == 1)
        slice_partial<1>(h, M, H, jb.W, jb.N, blockIdx.x, jb.part, red);
    else
        slice_partial<kTokTile>(h, M, H, jb.W, jb.N, blockIdx.x, jb.part, red);
}

// Router: slices as above; the last workgroup to finish (integer ticket)
// adds the slices in slice order (+ bias) for up to four tokens at a time --
// every partial load of a pass is issued before the first add.  The top-k is
// taken by rank counting under the total order (logit desc, expert id asc):
// rank(e) = #{e' : l[e'] > l[e] or (l[e'] == l[e] and e' < e)}, and the
// expert of rank s < k goes to slot s.  The ranks are exact, so the result
// does not depend on how the work is split.  NaN logits count as -inf.  The
// softmax over the selected logits adds the denominator in slot order.
constexpr int kSliceBatch = 32;

// Returns true in the last workgroup (which has written ids and weights).
template <int TT>
__device__ __forceinline__ bool router_body(const float* __restrict__ h, int M, int H, const uint16_t* __restrict__ Wr,
                                            int E, const float* __restrict__ bias, int k, float* __restrict__ part,
                                            unsigned* __restrict__ ticket, int32_t* __restrict__ ids,
                                            float* __restrict__ wts, float* __restrict__ logits_out, float* red) {
    __shared__ int s_last;
    __shared__ int sel_e[kTokTile][32];
    __shared__ float sel_l[kTokTile][32];
    const int nslices = gridDim.x;
    slice_partial<TT>(h, M, H, Wr, E, blockIdx.x, part, red);

    __threadfence();  // publish this workgroup's partials device-wide
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(ticket, 1u) == (unsigned)(nslices - 1);
    __syncthreads();
    if (!s_last) return false;
    __threadfence();  // observe every other workgroup's partials

    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    float* slog = red;  // [kTokTile][E] logits of the pass (red holds >= kTokTile * E floats)
    for (int t0 = 0; t0 < M; t0 += TT) {
        const int nt = min(TT, M - t0);
        for (int pr = tid; pr < nt * E; pr += kThreads) {
            const int t = t0 + pr / E, e = pr % E;
            float s = 0.f;
            for (int sl0 = 0; sl0 < nslices; sl0 += kSliceBatch) {
                float x[kSliceBatch];
#pragma unroll
                for (int u = 0; u < kSliceBatch; ++u)
                    x[u] = sl0 + u < nslices ? part[((size_t)(sl0 + u) * M + t) * E + e] : 0.f;
#pragma unroll
                for (int u = 0; u < kSliceBatch; ++u) s += x[u];  // slice order
            }
            if (bias) s += bias[e];
            if (logits_out) logits_out[(size_t)t * E + e] = s;
            slog[pr] = (s != s) ? -INFINITY : s;
        }
        __syncthreads();
        for (int pr = tid; pr < nt * E; pr += kThreads) {
            const int tl = pr / E, e = pr % E;
            const float v = slog[pr];
            const float* row = slog + tl * E;
            int rank = 0;
            for (int e2 = 0; e2 < E; e2 += 4) {  // E % 8 == 0
                const float4 o = *reinterpret_cast<const float4*>(row + e2);
                rank += (o.x > v || (o.x == v && e2 < e)) ? 1 : 0;
                rank += (o.y > v || (o.y == v && e2 + 1 < e)) ? 1 : 0;
                rank += (o.z > v || (o.z == v && e2 + 2 < e)) ? 1 : 0;
                rank += (o.w > v || (o.w == v && e2 + 3 < e)) ? 1 : 0;
            }
            if (rank < k) {
                sel_e[tl][rank] = e;
                sel_l[tl][rank] = v;
            }
        }
        __syncthreads();
        if (wave < nt && lane < k) {
            const int t = t0 + wave;
            const float l = sel_l[wave][lane];
            const float x = expf(l - sel_l[wave][0]);
            float den = 0.f;
            for (int s = 0; s < k; ++s) den += expf(sel_l[wave][s] - sel_l[wave][0]);
            ids[(size_t)t * k + lane] = sel_e[wave][lane];
            wts[(size_t)t * k + lane] = x / den;
        }
        __syncthreads();
    }
    if (tid == 0) atomicExch(ticket, 0u);  // ready for the next call on this context
    return true;
}

__global__ void __launch_bounds__(kThreads)
router_kernel(const float* __restrict__ h, int M, int H, const uint16_t* __restrict__ Wr, int E,
              const float* __restrict__ bias, int k, float* __restrict__ part, unsigned* __restrict__ ticket,
              int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits_out) {
    extern __shared__ float red[];
    if (M == 1)
        router_body<1>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red);
    else
        router_body<kTokTile>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red);
}

// Router, then the canonical alignment of the ids in the last workgroup
// (which wrote them; the workgroup barrier makes them visible to it).
__global__ void __launch_bounds__(kThreads)
router_align_kernel(const float* __restrict__ h, int M, int H, const uint16_t* __restrict__ Wr, int E,
                    const float* __restrict__ bias, int k, float* __restrict__ part, unsigned* __restrict__ ticket,
                    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits_out, int b,
                    int32_t* __restrict__ sorted_routes, int32_t* __restrict__ block_expert,
                    int32_t* __restrict__ counts, int32_t* __restrict__ err) {
    extern __shared__ float red[];
    const bool last = M == 1 ? router_body<1>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red)
                             : router_body<kTokTile>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red);
    if (!last) return;
    __syncthreads();
    align_workgroup(ids, M * k, E, b, sorted_routes, block_expert, counts, err, reinterpret_cast<int*>(red));
}

size_t lds_bytes(int N) { return (size_t)(kThreads / (N / 8)) * kTokTile * N * sizeof(float); }

}  // namespace

int gemv_slices(int H, int N) {
    const int rpp = kThreads / (N / 8);
    return (H + rpp * kRowsPerThread - 1) / (rpp * kRowsPerThread);
}

hipError_t launch_gemv_partials(const float* h, int M, int H, const GemvJob* jobs, int njobs, hipStream_t stream) {
    if (njobs < 1 || njobs > kMaxJobs) return hipErrorInvalidValue;
    GemvJobs js{};
    size_t lds = 0;
    int grid = 0;
    for (int i = 0; i < njobs; ++i) {
        js.job[i] = jobs[i];
        lds = lds_bytes(jobs[i].N) > lds ? lds_bytes(jobs[i].N) : lds;
        grid = gemv_slices(H, jobs[i].N) > grid ? gemv_slices(H, jobs[i].N) : grid;
    }
    MOE_LAUNCH(gemv_partials_kernel, dim3(grid, njobs), dim3(kThreads), lds, stream, h, M, H, js);
    return hipGetLastError();
}

hipError_t launch_router_align(const float* h, int M, int H, const uint16_t* Wr, int E, const float* bias, int k,
                               float* part, unsigned* ticket, int32_t* ids, float* wts, float* logits_out, int b,
                               int32_t* sorted_routes, int32_t* block_expert, int32_t* counts, int32_t* err,
                               hipStream_t stream) {
    const size_t la = align_lds_bytes(M * k, E);
    const size_t lds = lds_bytes(E) > la ? lds_bytes(E) : la;
    MOE_LAUNCH(router_align_kernel, dim3(gemv_slices(H, E)), dim3(kThreads), lds, stream, h, M, H, Wr, E, bias,
                       k, part, ticket, ids, wts, logits_out, b, sorted_routes, block_expert, counts, err);
    return hipGetLastError();
}

hipError_t launch_router(const float* h, int M, int H, const uint16_t* Wr, int E, const float* bias, int k,
                         float* part, unsigned* ticket, int32_t* ids, float* wts, float* logits_out,
                         hipStream_t stream) {
    MOE_LAUNCH(router_kernel, dim3(gemv_slices(H, E)), dim3(kThreads), lds_bytes(E), stream, h, M, H, Wr, E,
                       bias, k, part, ticket, ids, wts, logits_out);
    return hipGetLastError();
}

}  // namespace moe

// Dense bf16 experts: fused gate/up GEMV with SiLU(gate)*up kept in
// registers, down GEMV row-chunk partials, and the fixed-order weighted
// combine (page "A Multi-Engine Dataflow for MoE Decoding on Scratchpad-Based
// Tensor Accelerators", MoE-block background and Sec. 4.3; page "Channel
// Selection for Mixture-of-Experts Decoding Needs No Calibration Data",
// Background: the channel view of the same computation).
//
// Work is expert-major: the workgroups of an alignment block that starts an
// expert's run of blocks walk every block of that run, so each routed
// expert's weights are streamed from HBM once per step whatever its number of
// routes.  The weights of a workgroup's channel chunk are loaded into
// registers first (all loads in flight at once) and reused for every route.
// The arithmetic of one route never depends on its position in the plan or on
// the grid: per lane the hidden dimension is walked in ascending order, lanes
// are summed by a fixed butterfly, and results are stored by route id.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;

// Resolve the workgroup's expert.  Returns -1 when the workgroup has nothing
// to do (beyond num_blocks, or not the first block of its expert's run).
__device__ __forceinline__ int run_expert(const PlanArgs& plan, int blk, int* nb_out, int32_t* err) {
    int nb = plan.counts[0];
    if (nb < 0 || nb > plan.max_blocks) {
        if (blk == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(err, DEVERR_BAD_COUNTS);
        nb = nb < 0 ? 0 : plan.max_blocks;
    }
    *nb_out = nb;
    if (blk >= nb) return -1;
    const int e = plan.block_expert[blk];
    if (e < 0 || e >= plan.E) {
        if (blockIdx.y == 0 && threadIdx.x == 0) atomicOr(err, DEVERR_BAD_BLOCK_EXPERT);
        return -1;
    }
    if (blk > 0 && plan.block_expert[blk - 1] == e) return -1;
    return e;
}

// Row q of block bb: the route id if it is a valid route of expert e, else -1.
// Values other than the pad sentinel that are not such a route flag the plan.
__device__ __forceinline__ int plan_route(const PlanArgs& plan, int bb, int q, int e, int32_t* err) {
    if (q >= plan.b) return -1;
    const int r = plan.sorted_routes[(size_t)bb * plan.b + q];
    if (r == plan.R) return -1;
    if (r < 0 || r > plan.R || plan.topk_ids[r] != e) {
        if (threadIdx.x == 0) atomicOr(err, DEVERR_BAD_PLAN);
        return -1;
    }
    return r;
}

// Gate/up + SiLU.  Grid (plan blocks, ceil(I / (4*CPW))); wave w of
// workgroup (blk, cy) owns channels (cy*4 + w)*CPW + c.  Lane l covers hidden
// columns 8*(l + 64*q), q < Q (one 16-byte load per row and q).
template <int Q, int CPW, int RT>
__global__ void __launch_bounds__(kThreads)
gateup_dense_kernel(PlanArgs plan, const float* __restrict__ h, int H, int I, const uint16_t* __restrict__ Wg,
                    const uint16_t* __restrict__ Wu, float* __restrict__ p, int32_t* __restrict__ err) {
    const int blk = blockIdx.x;
    int nb;
    const int e = run_expert(plan, blk, &nb, err);
    if (e < 0) return;
    const int wave = threadIdx.x / MOE_WAVE;
    const int lane = threadIdx.x % MOE_WAVE;
    const int j0 = (blockIdx.y * kWaves + wave) * CPW;
    if (j0 >= I) return;  // no barriers below: a wave may leave on its own

    uint4 wg[CPW][Q], wu[CPW][Q];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int j = min(j0 + c, I - 1);  // clamped rows are computed and discarded
        const uint16_t* rg = Wg + ((size_t)e * I + j) * H;
        const uint16_t* ru = Wu + ((size_t)e * I + j) * H;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int col = (lane + MOE_WAVE * q) * 8;
            if (col < H) {
                wg[c][q] = load_stream16(rg + col);
                wu[c][q] = load_stream16(ru + col);
            } else {
                wg[c][q] = make_uint4(0, 0, 0, 0);
                wu[c][q] = make_uint4(0, 0, 0, 0);
            }
        }
    }

    for (int bb = blk; bb < nb; ++bb) {
        if (bb > blk && plan.block_expert[bb] != e) break;
        for (int q0 = 0; q0 < plan.b; q0 += RT) {
            int rt[RT];
            bool any = false;
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                rt[i] = plan_route(plan, bb, q0 + i, e, err);
                any |= rt[i] >= 0;
            }
            if (!any) continue;
            float ag[CPW][RT], au[CPW][RT];
#pragma unroll
            for (int c = 0; c < CPW; ++c)
#pragma unroll
                for (int i = 0; i < RT; ++i) ag[c][i] = au[c][i] = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int col = (lane + MOE_WAVE * q) * 8;
                if (col >= H) continue;
                float gf[CPW][8], uf[CPW][8];
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    unpack8(wg[c][q], gf[c]);
                    unpack8(wu[c][q], uf[c]);
                }
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    if (rt[i] < 0) continue;
                    const float* hr = h + (size_t)(rt[i] / plan.k) * H + col;
                    const float4 h0 = *reinterpret_cast<const float4*>(hr);
                    const float4 h1 = *reinterpret_cast<const float4*>(hr + 4);
                    const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                    for (int c = 0; c < CPW; ++c)
#pragma unroll
                        for (int x = 0; x < 8; ++x) {
                            ag[c][i] = fmaf(gf[c][x], hv[x], ag[c][i]);
                            au[c][i] = fmaf(uf[c][x], hv[x], au[c][i]);
                        }
                }
            }
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                if (rt[i] < 0) continue;
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    const float g = wave_sum(ag[c][i]);
                    const float u = wave_sum(au[c][i]);
                    if (lane == 0 && j0 + c < I) p[(size_t)rt[i] * I + j0 + c] = silu_mul(g, u);
                }
            }
        }
    }
}

// Down GEMV partials.  Grid (plan blocks, ceil(I / RC)); workgroup (blk, rc)
// multiplies rows rc*RC .. rc*RC+RC-1 of W_down,e by the matching p values of
// each route of the run; thread t covers hidden columns 8*(t + 256*cq).  The
// RC rows are added in ascending order into
// part[route][rc][col] = sum_{j in chunk} p[route][j] * Wd[e][j][col].
template <int CQ, int RC, int RT>
__global__ void __launch_bounds__(kThreads)
down_kernel(PlanArgs plan, int H, int I, int nrc, const uint16_t* __restrict__ Wd, const float* __restrict__ p,
            float* __restrict__ part, int32_t* __restrict__ err) {
    const int blk = blockIdx.x;
    const int rc = blockIdx.y;
    int nb;
    const int e = run_expert(plan, blk, &nb, err);
    if (e < 0) return;
    const int tid = threadIdx.x;
    const int j0 = rc * RC;

    uint4 w[RC][CQ];
#pragma unroll
    for (int jr = 0; jr < RC; ++jr) {
        const int j = min(j0 + jr, I - 1);
        const uint16_t* row = Wd + ((size_t)e * I + j) * H;
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq) {
            const int col = (tid + kThreads * cq) * 8;
            w[jr][cq] = (col < H && j0 + jr < I) ? load_stream16(row + col) : make_uint4(0, 0, 0, 0);
        }
    }

    for (int bb = blk; bb < nb; ++bb) {
        if (bb > blk && plan.block_expert[bb] != e) break;
        for (int q0 = 0; q0 < plan.b; q0 += RT) {
            int rt[RT];
            bool any = false;
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                rt[i] = plan_route(plan, bb, q0 + i, e, err);
                any |= rt[i] >= 0;
            }
            if (!any) continue;
            float pv[RT][RC];
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int jr = 0; jr < RC; ++jr)
                    pv[i][jr] = (rt[i] >= 0 && j0 + jr < I) ? p[(size_t)rt[i] * I + j0 + jr] : 0.f;
#pragma unroll
            for (int cq = 0; cq < CQ; ++cq) {
                const int col = (tid + kThreads * cq) * 8;
                if (col >= H) continue;
                float acc[RT][8];
#pragma unroll
                for (int i = 0; i < RT; ++i)
#pragma unroll
                    for (int x = 0; x < 8; ++x) acc[i][x] = 0.f;
#pragma unroll
                for (int jr = 0; jr < RC; ++jr) {
                    float wf[8];
                    unpack8(w[jr][cq], wf);
#pragma unroll
                    for (int i = 0; i < RT; ++i)
#pragma unroll
                        for (int x = 0; x < 8; ++x) acc[i][x] = fmaf(pv[i][jr], wf[x], acc[i][x]);
                }
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    if (rt[i] < 0) continue;
                    float* dst = part + ((size_t)rt[i] * nrc + rc) * H + col;
                    *reinterpret_cast<float4*>(dst) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                    *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
                }
            }
        }
    }
}

// y[t][col] = sum_{s=0..k-1} w[t][s] * (sum_{c=0..nchunks-1} part[t*k+s][c][col]),
// slots in order, chunks in order; routes with an id outside [0, E) add nothing.
__global__ void __launch_bounds__(kThreads)
combine_kernel(const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w, int M, int k, int E, int H,
               int nchunks, const float* __restrict__ part, float* __restrict__ y) {
    const int t = blockIdx.y;
    const int col = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (col >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < k; ++s) {
        const int r = t * k + s;
        const int e = topk_ids[r];
        if (e < 0 || e >= E) continue;
        const float w = topk_w[r];
        float4 ys = make_float4(0.f, 0.f, 0.f, 0.f);
        const float* src = part + (size_t)r * nchunks * H + col;
        for (int c = 0; c < nchunks; ++c) {
            const float4 v = *reinterpret_cast<const float4*>(src + (size_t)c * H);
            ys.x += v.x; ys.y += v.y; ys.z += v.z; ys.w += v.w;
        }
        acc.x = fmaf(w, ys.x, acc.x);
        acc.y = fmaf(w, ys.y, acc.y);
        acc.z = fmaf(w, ys.z, acc.z);
        acc.w = fmaf(w, ys.w, acc.w);
    }
    *reinterpret_cast<float4*>(y + (size_t)t * H + col) = acc;
}

template <int Q, int CPW>
hipError_t gateup_q(const PlanArgs& plan, int RT, const float* h, int H, int I, const uint16_t* Wg,
                    const uint16_t* Wu, float* p, int32_t* err, hipStream_t stream) {
    const dim3 grid(plan.max_blocks, (I + kWaves * CPW - 1) / (kWaves * CPW));
    if (RT == 1)
        hipLaunchKernelGGL((gateup_dense_kernel<Q, CPW, 1>), grid, dim3(kThreads), 0, stream, plan, h, H, I, Wg, Wu,
                           p, err);
    else if (RT == 4)
        hipLaunchKernelGGL((gateup_dense_kernel<Q, CPW, 4>), grid, dim3(kThreads), 0, stream, plan, h, H, I, Wg, Wu,
                           p, err);
    else
        hipLaunchKernelGGL((gateup_dense_kernel<Q, CPW, 8>), grid, dim3(kThreads), 0, stream, plan, h, H, I, Wg, Wu,
                           p, err);
    return hipGetLastError();
}

template <int CQ>
hipError_t down_cq(const PlanArgs& plan, int RT, int H, int I, int RC, const uint16_t* Wd, const float* p,
                   float* part, int32_t* err, hipStream_t stream) {
    const int nrc = (I + RC - 1) / RC;
    const dim3 grid(plan.max_blocks, nrc);
    if (RT == 1 && RC == 16)
        hipLaunchKernelGGL((down_kernel<CQ, 16, 1>), grid, dim3(kThreads), 0, stream, plan, H, I, nrc, Wd, p, part,
                           err);
    else if (RT == 1 && RC == 32)
        hipLaunchKernelGGL((down_kernel<CQ, 32, 1>), grid, dim3(kThreads), 0, stream, plan, H, I, nrc, Wd, p, part,
                           err);
    else if (RT == 4 && RC == 8)
        hipLaunchKernelGGL((down_kernel<CQ, 8, 4>), grid, dim3(kThreads), 0, stream, plan, H, I, nrc, Wd, p, part,
                           err);
    else if (RT == 8 && RC == 8)
        hipLaunchKernelGGL((down_kernel<CQ, 8, 8>), grid, dim3(kThreads), 0, stream, plan, H, I, nrc, Wd, p, part,
                           err);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

// Register tile of routes for a plan with M tokens: one route per block at
// M == 1, else up to 4 or 8 rows of a block at a time.
static int route_tile(int M, int b) {
    if (M == 1) return 1;
    if (M <= 4 || b <= 4) return 4;
    return 8;
}

hipError_t launch_gateup_dense(const PlanArgs& plan, const float* h, int H, int I, const uint16_t* Wg,
                               const uint16_t* Wu, float* p, int32_t* err, hipStream_t stream) {
    const int RT = route_tile(plan.R / plan.k, plan.b);
    const int Q = (H + 511) / 512;
    if (Q <= 1) return gateup_q<1, 2>(plan, RT, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 2) return gateup_q<2, 2>(plan, RT, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 4) return gateup_q<4, 2>(plan, RT, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 8) return gateup_q<8, 2>(plan, RT, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 16) return gateup_q<16, 1>(plan, RT, h, H, I, Wg, Wu, p, err, stream);
    return hipErrorInvalidValue;
}

int down_rows_per_chunk(int M, int b) { return route_tile(M, b) == 1 ? 16 : 8; }

hipError_t launch_down(const PlanArgs& plan, int H, int I, int RC, const uint16_t* Wd, const float* p, float* part,
                       int32_t* err, hipStream_t stream) {
    const int RT = route_tile(plan.R / plan.k, plan.b);
    const int CQ = (H + 2047) / 2048;
    if (CQ <= 1) return down_cq<1>(plan, RT, H, I, RC, Wd, p, part, err, stream);
    if (CQ <= 2) return down_cq<2>(plan, RT, H, I, RC, Wd, p, part, err, stream);
    if (CQ <= 4) return down_cq<4>(plan, RT, H, I, RC, Wd, p, part, err, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_combine(const int32_t* topk_ids, const float* topk_w, int M, int k, int E, int H, int nchunks,
                          const float* part, float* y, hipStream_t stream) {
    const dim3 grid((H / 4 + kThreads - 1) / kThreads, M);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, stream, topk_ids, topk_w, M, k, E, H, nchunks, part,
                       y);
    return hipGetLastError();
}

}  // namespace moe

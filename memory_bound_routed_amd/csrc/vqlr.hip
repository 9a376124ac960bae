// VQ + low-rank gate/up projections (page "A Multi-Engine Dataflow for MoE
// Decoding on Scratchpad-Based Tensor Accelerators", Sec. 2.3 blockwise VQ,
// Sec. 3.1 Eq. 1 hybrid representation, Sec. 4.2 shared-projection reuse,
// cross-expert gather batching and joint accumulation).
//
// For projection P of channel j of expert e and token t:
//     o_P[j] = sum_rho C_P,e[j][rho] z_P[t][rho]  +  sum_b h_b . B_P[J_P,e[j][b]]
// where z_P = D_P^T h (computed once per token by the GEMV-partials kernel,
// summed here over its row slices in slice order) and h_b is the b-th
// length-8 block of h.  The page materialises the projection code book
// T[b][c] = h_b . B_c; an fp32 T is 256 KiB per token and projection, larger
// than a CU's LDS, so here the two 4 KiB weight code books stay resident in
// LDS and each selected code word is applied to h_b on the fly (8 FMAs per
// index).  Both terms accumulate into one fp32 register per lane before a
// single wave reduction (the joint accumulation), then p = SiLU(o_gate)*o_up.
// One launch covers every routed expert (the gather batching); each expert's
// J and C are read once per step for all of its routes.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kCPW = 4;   // channels per wave
constexpr int kRT = 4;    // plan rows examined per group
constexpr int kD = 8;     // VQ block length supported by this kernel

__device__ __forceinline__ int run_expert_vq(const PlanArgs& plan, int blk, int* nb_out, int32_t* err) {
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

__device__ __forceinline__ int plan_route_vq(const PlanArgs& plan, int bb, int q, int e, int32_t* err) {
    if (q >= plan.b) return -1;
    const int r = plan.sorted_routes[(size_t)bb * plan.b + q];
    if (r == plan.R) return -1;
    if (r < 0 || r > plan.R || plan.topk_ids[r] != e) {
        if (threadIdx.x == 0) atomicOr(err, DEVERR_BAD_PLAN);
        return -1;
    }
    return r;
}

// Grid (plan blocks, ceil(I / (4*kCPW))).  Lane l owns VQ blocks
// 4*(l + 64*qb) .. +3 (one 4-byte index load per channel) and low-rank
// coordinates rho = l + 64*m.
template <int QB, int RM>
__global__ void __launch_bounds__(kThreads)
gateup_vqlr_kernel(PlanArgs plan, VqArgs vq, const float* __restrict__ h, int H, int I, float* __restrict__ p,
                   int32_t* __restrict__ err) {
    __shared__ uint4 book[2][256];
    const int blk = blockIdx.x;
    int nb;
    const int e = run_expert_vq(plan, blk, &nb, err);
    if (e < 0) return;  // uniform over the workgroup
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int nbk = H / kD;        // VQ blocks per channel
    const int r = vq.r;

    const int j0 = (blockIdx.y * kWaves + wave) * kCPW;
    uint32_t jw[2][kCPW][QB];
    float cv[2][kCPW][RM];
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int c = 0; c < kCPW; ++c) {
            const int j = min(j0 + c, I - 1);
            const uint8_t* jrow = vq.J[P] + ((size_t)e * I + j) * nbk;
            const uint16_t* crow = vq.C[P] + ((size_t)e * I + j) * r;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int b4 = 4 * (lane + MOE_WAVE * qb);
                jw[P][c][qb] = b4 < nbk ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(jrow + b4)) : 0u;
            }
#pragma unroll
            for (int m = 0; m < RM; ++m) {
                const int rho = lane + MOE_WAVE * m;
                cv[P][c][m] = rho < r ? bf16_lo(__builtin_nontemporal_load(crow + rho)) : 0.f;
            }
        }
    for (int i = tid; i < 2 * 256; i += kThreads) {
        const int P = i / 256, c = i % 256;
        book[P][c] = c < vq.K ? load16(vq.B[P] + (size_t)c * kD) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    if (j0 >= I) return;

    for (int bb = blk; bb < nb; ++bb) {
        if (bb > blk && plan.block_expert[bb] != e) break;
        for (int q0 = 0; q0 < plan.b; q0 += kRT) {
            int rt[kRT];
            bool any = false;
#pragma unroll
            for (int i = 0; i < kRT; ++i) {
                rt[i] = plan_route_vq(plan, bb, q0 + i, e, err);
                any |= rt[i] >= 0;
            }
            if (!any) continue;
            float acc[2][kCPW][kRT];
#pragma unroll
            for (int P = 0; P < 2; ++P)
#pragma unroll
                for (int c = 0; c < kCPW; ++c)
#pragma unroll
                    for (int i = 0; i < kRT; ++i) acc[P][c][i] = 0.f;
#pragma unroll
            for (int i = 0; i < kRT; ++i) {
                if (rt[i] < 0) continue;
                const int t = rt[i] / plan.k;
                // low-rank term: C_e[j] . z
#pragma unroll
                for (int P = 0; P < 2; ++P)
#pragma unroll
                    for (int m = 0; m < RM; ++m) {
                        const int rho = lane + MOE_WAVE * m;
                        if (rho >= r) continue;
                        float z = 0.f;
                        for (int sl = 0; sl < vq.zslices; ++sl) z += vq.zpart[P][((size_t)sl * vq.M + t) * r + rho];
#pragma unroll
                        for (int c = 0; c < kCPW; ++c) acc[P][c][i] = fmaf(cv[P][c][m], z, acc[P][c][i]);
                    }
                // VQ term: selected code words applied to the token's h blocks
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int b4 = 4 * (lane + MOE_WAVE * qb);
                    if (b4 >= nbk) continue;
                    const float* hr = h + (size_t)t * H + b4 * kD;
                    float hv[32];
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const float4 x = *reinterpret_cast<const float4*>(hr + 4 * v);
                        hv[4 * v] = x.x; hv[4 * v + 1] = x.y; hv[4 * v + 2] = x.z; hv[4 * v + 3] = x.w;
                    }
#pragma unroll
                    for (int P = 0; P < 2; ++P)
#pragma unroll
                        for (int c = 0; c < kCPW; ++c)
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                float cw[8];
                                unpack8(book[P][(jw[P][c][qb] >> (8 * x)) & 255u], cw);
#pragma unroll
                                for (int y = 0; y < 8; ++y) acc[P][c][i] = fmaf(cw[y], hv[8 * x + y], acc[P][c][i]);
                            }
                }
            }
#pragma unroll
            for (int i = 0; i < kRT; ++i) {
                if (rt[i] < 0) continue;
#pragma unroll
                for (int c = 0; c < kCPW; ++c) {
                    const float og = wave_sum(acc[0][c][i]);
                    const float ou = wave_sum(acc[1][c][i]);
                    if (lane == 0 && j0 + c < I) p[(size_t)rt[i] * I + j0 + c] = silu_mul(og, ou);
                }
            }
        }
    }
}

template <int QB>
hipError_t vq_rm(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p, int32_t* err,
                 hipStream_t stream) {
    const dim3 grid(plan.max_blocks, (I + kWaves * kCPW - 1) / (kWaves * kCPW));
    const int RM = (vq.r + 63) / 64;
    if (RM <= 1)
        MOE_LAUNCH((gateup_vqlr_kernel<QB, 1>), grid, dim3(kThreads), 0, stream, plan, vq, h, H, I, p, err);
    else if (RM <= 2)
        MOE_LAUNCH((gateup_vqlr_kernel<QB, 2>), grid, dim3(kThreads), 0, stream, plan, vq, h, H, I, p, err);
    else if (RM <= 4)
        MOE_LAUNCH((gateup_vqlr_kernel<QB, 4>), grid, dim3(kThreads), 0, stream, plan, vq, h, H, I, p, err);
    else if (RM <= 8)
        MOE_LAUNCH((gateup_vqlr_kernel<QB, 8>), grid, dim3(kThreads), 0, stream, plan, vq, h, H, I, p, err);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_vqlr(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p,
                              int32_t* err, hipStream_t stream) {
    if (vq.d != kD || vq.K < 1 || vq.K > 256) return hipErrorInvalidValue;
    const int QB = (H / kD + 255) / 256;
    if (QB <= 1) return vq_rm<1>(plan, vq, h, H, I, p, err, stream);
    if (QB <= 2) return vq_rm<2>(plan, vq, h, H, I, p, err, stream);
    if (QB <= 4) return vq_rm<4>(plan, vq, h, H, I, p, err, stream);
    return hipErrorInvalidValue;
}

}  // namespace moe

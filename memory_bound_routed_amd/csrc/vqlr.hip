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
constexpr int kRT = 4;    // routes staged together
constexpr int kD = 8;     // VQ block length supported by this kernel
constexpr int kZBatch = 16;

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

// Grid (plan blocks, ceil(I / (4*CPW))): workgroup (blk, cy) owns 4*CPW
// channels of the expert whose run of blocks starts at blk; wave w owns CPW
// of them.  Lane l owns VQ blocks 4*(l + 64*qb) .. +3 (one 4-byte index load
// per channel) and low-rank coordinates rho = l + 64*m.  The index maps and
// coefficients are requested first and kept in registers for every route of
// the expert; the two code books go to LDS.  Routes are taken rvq at a time:
// their h rows and their finished z vectors (the slice partials added in
// slice order) are staged in LDS, then every wave forms its channels'
// outputs.
template <int QB, int RM, int CPW>
__global__ void __launch_bounds__(kThreads)
gateup_vqlr_kernel(PlanArgs plan, VqArgs vq, const float* __restrict__ h, int H, int I, int rvq, float* __restrict__ p,
                   int32_t* __restrict__ err) {
    __shared__ uint4 book[2][256];
    extern __shared__ __align__(16) float dyn[];
    float* hsm = dyn;                       // [rvq][H]
    float* zsm = dyn + (size_t)rvq * H;     // [kRT][2][r]
    const int blk = blockIdx.x;
    int nb;
    const int e = run_expert_vq(plan, blk, &nb, err);
    if (e < 0) return;  // uniform over the workgroup
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int nbk = H / kD;        // VQ blocks per channel
    const int r = vq.r;
    const int j0 = (blockIdx.y * kWaves + wave) * CPW;
    const bool active = j0 < I;   // inactive waves still take part in the barriers

    uint32_t jw[2][CPW][QB];
    float cv[2][CPW][RM];
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int j = min(j0 + c, I - 1);
            const uint8_t* jrow = vq.J[P] + ((size_t)e * I + j) * nbk;
            const uint16_t* crow = vq.C[P] + ((size_t)e * I + j) * r;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int b4 = 4 * (lane + MOE_WAVE * qb);
                jw[P][c][qb] = b4 < nbk ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(jrow + min(b4, nbk - 4))) : 0u;
            }
#pragma unroll
            for (int m = 0; m < RM; ++m) {
                const int rho = lane + MOE_WAVE * m;
                cv[P][c][m] = rho < r ? bf16_lo(__builtin_nontemporal_load(crow + min(rho, r - 1))) : 0.f;
            }
        }
    for (int i = tid; i < 2 * 256; i += kThreads) {
        const int P = i / 256, c = i % 256;
        book[P][c] = c < vq.K ? load16(vq.B[P] + (size_t)c * kD) : make_uint4(0, 0, 0, 0);
    }

    // routes of the expert's run, one block at a time (lane q holds row q)
    for (int bb = blk; bb < nb; ++bb) {
        if (bb > blk && plan.block_expert[bb] != e) break;
        int rv = lane < plan.b ? plan.sorted_routes[(size_t)bb * plan.b + lane] : plan.R;
        const bool ok = rv >= 0 && rv < plan.R && plan.topk_ids[rv] == e;
        if (!ok && rv != plan.R && wave == 0 && blockIdx.y == 0) atomicOr(err, DEVERR_BAD_PLAN);
        uint64_t todo = __ballot(ok);
        while (todo) {
            int rt[kRT];
            int nr = 0;
#pragma unroll
            for (int i = 0; i < kRT; ++i) {
                rt[i] = -1;
                if (i < rvq && todo) {
                    const int q = __builtin_ctzll(todo);
                    todo &= todo - 1;
                    rt[i] = __builtin_amdgcn_readlane(rv, q);
                    nr = i + 1;
                }
            }
            __syncthreads();  // the previous group's staging (and the book) is complete / no longer read
#pragma unroll
            for (int i = 0; i < kRT; ++i) {
                if (i >= nr) break;
                const float4* src = reinterpret_cast<const float4*>(h + (size_t)(rt[i] / plan.k) * H);
                float4* dst = reinterpret_cast<float4*>(hsm + (size_t)i * H);
                for (int c4 = tid; c4 < H / 4; c4 += kThreads) dst[c4] = src[c4];
            }
            for (int it = tid; it < nr * 2 * r; it += kThreads) {
                const int i = it / (2 * r), rem = it - i * 2 * r, P = rem / r, rho = rem - P * r;
                int ti = 0;
#pragma unroll
                for (int ii = 0; ii < kRT; ++ii)
                    if (ii == i) ti = rt[ii] / plan.k;
                float z = 0.f;
                for (int sl0 = 0; sl0 < vq.zslices; sl0 += kZBatch) {
                    float x[kZBatch];
#pragma unroll
                    for (int u = 0; u < kZBatch; ++u)
                        x[u] = vq.zpart[P][((size_t)min(sl0 + u, vq.zslices - 1) * vq.M + ti) * r + rho];
#pragma unroll
                    for (int u = 0; u < kZBatch; ++u) z += sl0 + u < vq.zslices ? x[u] : 0.f;  // slice order
                }
                zsm[it] = z;
            }
            __syncthreads();
            if (!active) continue;
#pragma unroll
            for (int i = 0; i < kRT; ++i) {
                if (i >= nr) break;
                float acc[2][CPW];
#pragma unroll
                for (int P = 0; P < 2; ++P)
#pragma unroll
                    for (int c = 0; c < CPW; ++c) acc[P][c] = 0.f;
                // low-rank term: C_e[j] . z
#pragma unroll
                for (int P = 0; P < 2; ++P)
#pragma unroll
                    for (int m = 0; m < RM; ++m) {
                        const int rho = lane + MOE_WAVE * m;
                        const float z = rho < r ? zsm[(i * 2 + P) * r + rho] : 0.f;
#pragma unroll
                        for (int c = 0; c < CPW; ++c) acc[P][c] = fmaf(cv[P][c][m], z, acc[P][c]);
                    }
                // VQ term: selected code words applied to the token's h blocks
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int b4 = 4 * (lane + MOE_WAVE * qb);
                    if (b4 >= nbk) continue;
                    const float4* hr = reinterpret_cast<const float4*>(hsm + (size_t)i * H + b4 * kD);
                    float hv[32];
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const float4 x = hr[v];
                        hv[4 * v] = x.x; hv[4 * v + 1] = x.y; hv[4 * v + 2] = x.z; hv[4 * v + 3] = x.w;
                    }
#pragma unroll
                    for (int P = 0; P < 2; ++P)
#pragma unroll
                        for (int c = 0; c < CPW; ++c)
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                float cw[8];
                                unpack8(book[P][(jw[P][c][qb] >> (8 * x)) & 255u], cw);
#pragma unroll
                                for (int y = 0; y < 8; ++y) acc[P][c] = fmaf(cw[y], hv[8 * x + y], acc[P][c]);
                            }
                }
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    const float og = wave_sum(acc[0][c]);
                    const float ou = wave_sum(acc[1][c]);
                    if (lane == 0 && j0 + c < I) p[(size_t)rt[i] * I + j0 + c] = silu_mul(og, ou);
                }
            }
        }
    }
}

template <int QB, int RM, int CPW>
hipError_t vq_launch(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p, int32_t* err,
                     hipStream_t stream) {
    const dim3 grid(plan.max_blocks, (I + kWaves * CPW - 1) / (kWaves * CPW));
    const int rvq = H <= 4096 ? kRT : 2;  // staged h rows: <= 64 KiB
    const size_t lds = ((size_t)rvq * H + (size_t)kRT * 2 * vq.r) * sizeof(float);
    MOE_LAUNCH((gateup_vqlr_kernel<QB, RM, CPW>), grid, dim3(kThreads), lds, stream, plan, vq, h, H, I, rvq, p, err);
    return hipGetLastError();
}

// Channels per wave: 8 for the smallest register tile (H <= 2048, r <= 64),
// else 4.
template <int QB>
hipError_t vq_rm(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p, int32_t* err,
                 hipStream_t stream) {
    const int RM = (vq.r + 63) / 64;
    if (RM <= 1) return vq_launch<QB, 1, QB == 1 ? 8 : 4>(plan, vq, h, H, I, p, err, stream);
    if (RM <= 2) return vq_launch<QB, 2, 4>(plan, vq, h, H, I, p, err, stream);
    if (RM <= 4) return vq_launch<QB, 4, 4>(plan, vq, h, H, I, p, err, stream);
    if (RM <= 8) return vq_launch<QB, 8, 4>(plan, vq, h, H, I, p, err, stream);
    return hipErrorInvalidValue;
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

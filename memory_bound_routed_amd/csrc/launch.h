// Host-side launchers of the libmoe kernels (internal; not part of the ABI).
// Every launcher only enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- router.hip
// Row-slice partials of skinny GEMVs  part_m[slice][t][n] = sum_{i in slice} h[t][i] * W_m[i][n]
// for up to three matrices W_m (bf16 [H][N_m]) in one launch.
struct GemvJob {
    const uint16_t* W;   // bf16 [H][N]
    int N;               // columns, N % 8 == 0, N <= 2048
    float* part;         // fp32 [nslices][M][N]
};
hipError_t launch_gemv_partials(const float* h, int M, int H, int slice_rows, const GemvJob* jobs, int njobs,
                                hipStream_t stream);
hipError_t launch_router_topk(const float* part, int nslices, int M, int E, int k, const float* bias,
                              int32_t* ids, float* wts, float* logits_out, hipStream_t stream);

// ---- align.hip
size_t align_lds_bytes(int R, int E);
hipError_t launch_align(const int32_t* topk_ids, int R, int E, int b, int32_t* sorted_routes,
                        int32_t* block_expert, int32_t* counts, int32_t* err, hipStream_t stream);

// ---- dense.hip
struct PlanArgs {
    const int32_t* topk_ids;       // [M][k]
    const int32_t* sorted_routes;  // [cap]
    const int32_t* block_expert;   // [cap/b]
    const int32_t* counts;         // [2]
    int R;                         // M*k (also the pad sentinel)
    int k;
    int b;
    int max_blocks;                // cap / b
    int E;
};
hipError_t launch_gateup_dense(const PlanArgs& plan, const float* h, int H, int I, const uint16_t* Wg,
                               const uint16_t* Wu, float* p, int32_t* err, hipStream_t stream);
hipError_t launch_down(const PlanArgs& plan, int H, int I, int rows_per_chunk, const uint16_t* Wd,
                       const float* p, float* part, int32_t* err, hipStream_t stream);
hipError_t launch_combine(const int32_t* topk_ids, const float* topk_w, int M, int k, int E, int H,
                          int nchunks, const float* part, float* y, hipStream_t stream);

// ---- vqlr.hip
struct VqArgs {
    const uint16_t* C[2];   // bf16 [E][I][r]
    const uint16_t* B[2];   // bf16 [K][d]
    const uint8_t* J[2];    // u8 [E][I][H/d]
    const float* zpart[2];  // fp32 [zslices][M][r]
    int zslices;
    int M;
    int r;
    int K;
    int d;
};
hipError_t launch_gateup_vqlr(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p,
                              int32_t* err, hipStream_t stream);

// ---- chansparse.hip
size_t chan_select_lds_bytes(int n);
hipError_t launch_chan_select(const int32_t* topk_ids, const float* topk_w, const float* norms, int M, int k,
                              int I, int E, int K, int32_t* kept, hipStream_t stream);
hipError_t launch_chan_gather(const int32_t* topk_ids, const float* topk_w, const int32_t* kept, int M, int k,
                              int I, int E, int H, int K, int chunk, const float* h, const uint16_t* Wg,
                              const uint16_t* Wu, const uint16_t* Wd, float* part, hipStream_t stream);
hipError_t launch_chan_combine(int M, int H, int nchunks, const float* part, float* y, hipStream_t stream);
hipError_t launch_channel_norms(int E, int I, int H, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                                float* norms, hipStream_t stream);

}  // namespace moe

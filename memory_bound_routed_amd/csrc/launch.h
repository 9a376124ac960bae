// Host-side launchers of the libmoe kernels (internal; not part of the ABI).
// Every launcher only enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

// Events attached to the next launch while the context is profiling (set by
// the host API around each launcher).  With events, the launch goes through
// hipExtLaunchKernelGGL, which stamps them from the kernel's own dispatch:
// their elapsed time is the kernel's execution time.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();

#define MOE_LAUNCH(kernel, grid, block, shmem, stream, ...)                                                  \
    do {                                                                                                     \
        const ::moe::LaunchEvents ev_ = ::moe::launch_events();                                              \
        if (ev_.start)                                                                                       \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ev_.start, ev_.stop, 0, __VA_ARGS__);  \
        else                                                                                                 \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                             \
    } while (0)

// ---- router.hip
// Row-slice partials of skinny GEMVs  part_m[slice][t][n] = sum_{i in slice} h[t][i] * W_m[i][n]
// for up to three matrices W_m (bf16 [H][N_m]) in one launch.
struct GemvJob {
    const uint16_t* W;   // bf16 [H][N]
    int N;               // columns, N % 8 == 0, 8 <= N <= 1024
    float* part;         // fp32 [gemv_slices(H, N)][M][N]
};
int gemv_slices(int H, int N);
hipError_t launch_gemv_partials(const float* h, int M, int H, const GemvJob* jobs, int njobs, hipStream_t stream);
// Token groups of the router (4 tokens each; one group at M == 1).
int router_groups(int M);
// Router GEMV + (last workgroup of each token group) slice sum, top-k and
// softmax in one launch.  part: fp32 [gemv_slices(H, E)][M][E] (covers the
// tiles' slices); ticket: 1 + router_groups(M) zeroed uint32, left zeroed.
hipError_t launch_router(const float* h, int M, int H, const uint16_t* Wr, int E, const float* bias, int k,
                         float* part, unsigned* ticket, int32_t* ids, float* wts, float* logits_out,
                         hipStream_t stream);
// The same, followed (in the last workgroup to finish) by the canonical
// alignment of the ids.
hipError_t launch_router_align(const float* h, int M, int H, const uint16_t* Wr, int E, const float* bias, int k,
                               float* part, unsigned* ticket, int32_t* ids, float* wts, float* logits_out, int b,
                               int32_t* sorted_routes, int32_t* block_expert, int32_t* counts, int32_t* err,
                               hipStream_t stream, const GemvJob* jobs = nullptr, int njobs = 0);

// Router GEMV without the top-k: part fp32 [router_slices(H, E)][M][E]
// (row-slice partials; logit of (t, e) = 0 + part[0][t][e] + part[1][t][e]
// + ... in slice order, then + bias[e]).
int router_slices(int H, int E);
// Optional rotation job of the channel-selection reader riding along
// (reader_device.h: per token and 128-block, the scanned coordinates
// xsel u8 [M][H/128][80] and values xval fp32 [M][H/128][80]).
struct RotJob {
    const int8_t* signs;  // int8 [H] (+-1)
    uint8_t* xsel;
    float* xval;
};
hipError_t launch_router_partials(const float* h, int M, int H, const uint16_t* Wr, int E, float* part,
                                  hipStream_t stream, const RotJob* rot = nullptr, const GemvJob* jobs = nullptr,
                                  int njobs = 0);

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
    FastDiv fk;                    // division by k (route -> token)
    int b;
    FastDiv fb;                    // division by b
    int max_blocks;                // cap / b
    int E;
};
// Fused gate/up + down partials (one route per plan row group; H <= 4096).
bool dense_uses_fused(int M, int H);
// Number of down partial chunks per route of the schedule used for (M, H, I)
// and top-k k.
int dense_chunks(int M, int H, int I, int k);
int down_chunks(int I);
hipError_t launch_expert_fused(const PlanArgs& plan, const float* h, const float* topk_w, int H, int I,
                               const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, float* part, int32_t* err,
                               hipStream_t stream);
// The fused schedule for one token that routes the token itself from the
// router's slice partials (see router_slices) and writes the routing and the
// plan as moe_route_align would.  plan: R = k, max_blocks = k, E, k, b; its
// arrays are not read.
struct RouteArgs {
    const float* part;       // fp32 [nslices][E] router slice partials
    const float* bias;       // fp32 [E] or null
    int nslices;
    int32_t* ids;            // int32 [k] out
    float* wts;              // fp32 [k] out
    float* logits;           // fp32 [E] out, or null
    int32_t* sorted_routes;  // int32 [k*b] out
    int32_t* block_expert;   // int32 [k] out
    int32_t* counts;         // int32 [2] out
};
bool decode_fused_ok(int H, int E, int k, int nslices);
hipError_t launch_decode_fused(const PlanArgs& plan, const RouteArgs& route, const float* h, int H, int I,
                               const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, float* part, int32_t* err,
                               hipStream_t stream);
hipError_t launch_gateup_dense(const PlanArgs& plan, const float* h, int H, int I, const uint16_t* Wg,
                               const uint16_t* Wu, float* p, int32_t* err, hipStream_t stream);
// part[route][chunk][H] = sum over the chunk's rows of (a_route * p[route][j]) * Wd[e][j][:]
// With vq: p[r][j] = SiLU(sum_y vp[r][y][0][j]) * sum_y vp[r][y][1][j] from
// the VQ gate/up partials (rows y in order) instead of a p array.  With
// align (needs R <= 64): the plan is not read; every workgroup aligns the R
// routes from plan.topk_ids itself (the canonical plan, ballots of the id
// bits) and workgroup (0, 0) writes the plan to align's arrays.
struct VqP {
    const float* vp;
    int ny;
};
struct AlignOut {
    int32_t* sorted_routes;
    int32_t* block_expert;
    int32_t* counts;
};
hipError_t launch_down(const PlanArgs& plan, int H, int I, const uint16_t* Wd, const float* p, const float* topk_w,
                       float* part, int32_t* err, hipStream_t stream, const VqP* vq = nullptr,
                       const AlignOut* align = nullptr);
// y[t][:] = sum over valid routes of token t and chunks of part[route][chunk][:]
hipError_t launch_combine(const int32_t* topk_ids, int M, int k, int E, int H, int nchunk, const float* part, float* y,
                          hipStream_t stream);

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
// T slices per channel: ceil((H / d) / 64).
int vq_slices(int H, int d);
// One workgroup set per route r < R (token r / k, expert topk_ids[r]; ids
// outside [0, E) have no output): vp fp32 [R][vq_slices][2][I] slice
// partials of o_gate and o_up.  With route (the decode step; needs
// vq_routes_ok): no ids are read -- every workgroup routes its token from the
// router's slice partials, and the token's ids, weights and logits are
// stored to route->ids / wts / logits.
struct SelRoute;
bool vq_routes_ok(int E, int k);
hipError_t launch_gateup_vqlr(const int32_t* topk_ids, int R, int k, int E, const VqArgs& vq, const float* h, int H,
                              int I, float* vp, int32_t* err, hipStream_t stream, const SelRoute* route = nullptr);
// Partials per route and projection of the VQ gate/up launch for R routes:
// vp fp32 [R][vq_rows][2][I], row y the sum over the slices one workgroup
// took (see vqlr.hip).
int vq_rows(int R, int H, int d);
// p[r][j] = SiLU(sum_y vp[r][y][0][j]) * (sum_y vp[r][y][1][j]), sums in
// row order, for the R routes (ny <= 16 rows).  With plan: also the
// canonical alignment of the R routes from ids (written by the previous
// launch), by workgroup (0, 0).
struct VqPlanJob {
    const int32_t* ids;  // [R]
    int E, b;
    int32_t* sorted_routes;
    int32_t* block_expert;
    int32_t* counts;
    int32_t* err;
};
hipError_t launch_vq_finish(const float* vp, int R, int I, int ny, float* p, hipStream_t stream,
                            const VqPlanJob* plan = nullptr);

// ---- chansparse.hip
struct SelRoute {
    const float* part;   // fp32 [nslices][M][E] router slice partials
    const float* bias;   // fp32 [E] or null
    int nslices;
    int M;
    int32_t* ids;        // int32 [M][k] out
    float* wts;          // fp32 [M][k] out
    float* logits;       // fp32 [M][E] out, or null
};
struct ReaderArgs;
// Channel top-K and the kept channels' gate/up + down partials in one launch
// (grid ceil(K / 8) x M): mode 0 scores by the static norms (route non-null:
// each workgroup first routes its token from the router's slice partials and
// the ids / affinities are written to topk_ids / topk_w), mode 1 by the
// reader's estimates (ra).  part fp32 [M][ceil(K / 8)][H]; kept_out int32
// [M][K] (nullable): the kept set as s * I + j ascending; kept_flag u8
// [M][k][I] (nullable).
hipError_t launch_chan_topk_gather(int mode, const SelRoute* route, int32_t* topk_ids, float* topk_w,
                                   const float* norms, const ReaderArgs* ra, int M, int k, int I, int E, int H, int K,
                                   const float* h, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                                   float* part, int32_t* kept_out, uint8_t* kept_flag, hipStream_t stream);
hipError_t launch_chan_combine(int M, int H, int nchunks, const float* part, float* y, hipStream_t stream);
hipError_t launch_channel_norms(int E, int I, int H, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                                float* norms, hipStream_t stream);

// ---- reader.hip (channel selection by the ternary-sketch reader)
// Per-call buffers and load-time arrays of the reader.  Layouts:
//  sketch    u8 [E][2][nblk][128][rowb]  base-3 codes, coordinate-major rows
//  scale     fp32 [E][2][nblk][I]        per (block, channel) scale / 128
//  xsel/xval u8 / fp32 [M][nblk][80]     scanned coordinates (ascending), x''
//  est       fp32 [M][k][2][nbq][I]      partial g_hat (P = 0), v_hat (P = 1) of
//                                        each group of bpw blocks (reader_groups)
//  kept_flag u8 [M][k][I]
//  dnorm     fp32 [E][I];  rec_coef bf16 [E][I][rank];  rpart fp32 [M][k][chunks][rank]
struct ReaderArgs {
    const uint8_t* sketch;
    const float* scale;
    const uint8_t* xsel;
    const float* xval;
    float* est;
    const float* dnorm;
    uint8_t* kept_flag;
    const uint16_t* rec_coef;
    float* rpart;
    int rank;
    int nblk;
    int nbq;
    int bpw;
    int rowb;
    int I;
    int k;
    int E;
};
// Bytes of one coordinate row of the sketch: ceil(I / 5) padded to 16.
int reader_row_bytes(int I);
// Block groups of the screening: bpw = ceil(nblk / 2) blocks each; returns
// their number nbq (<= 2).
int reader_groups(int nblk, int* bpw);
// Rotation + partial scan of each 128-block of h (M tokens) in its own launch.
hipError_t launch_reader_rotate(const float* h, int M, int H, const int8_t* signs, uint8_t* xsel, float* xval,
                                hipStream_t stream);
// Screening: est for every routed (token, slot) from topk_ids, or (route
// non-null) routing each token first from the router's slice partials.
hipError_t launch_reader_screen(const ReaderArgs& ra, const SelRoute* route, const int32_t* topk_ids, int M,
                                hipStream_t stream);
// Output-level scores and the exact top K per token: slot_cnt / slot_kept as
// launch_chan_select and kept_flag in ra; optionally (non-null) the kept set
// kept_out [M][K], the summed estimates est_out [M][k][2][I] and the scores
// score_out [M][k][I].
hipError_t launch_reader_select(const ReaderArgs& ra, const int32_t* topk_ids, const float* topk_w, int M, int K,
                                int32_t* slot_cnt, int32_t* slot_kept, int32_t* kept_out, float* est_out,
                                float* score_out, hipStream_t stream);
int reader_recover_chunks(int I);
// Recovery partials rpart of the dropped candidates (ra.rank in 8..32, % 8).
hipError_t launch_reader_recover(const ReaderArgs& ra, const int32_t* topk_ids, const float* topk_w, int M,
                                 hipStream_t stream);
// y = sum of the gather's chunk partials + U (sum of the nrp recovery partials).
hipError_t launch_reader_combine(int M, int H, int nchunks, const float* part, const float* rpart, int nrp, int rank,
                                 const float* U, float* y, hipStream_t stream);
// Load time.
hipError_t launch_reader_sketch(int E, int I, int H, const uint16_t* Wg, const uint16_t* Wu, const int8_t* signs,
                                uint8_t* sketch, float* scale, hipStream_t stream);
hipError_t launch_down_norms(int E, int I, int H, const uint16_t* Wd, float* dn, hipStream_t stream);
size_t recovery_basis_scratch(int H, int rank);
hipError_t launch_recovery_basis(int E, int I, int H, const uint16_t* Wd, int rank, int iters, float* U, void* scratch,
                                 hipStream_t stream);
hipError_t launch_recovery_coefs(int E, int I, int H, const float* U, int rank, const uint16_t* Wd, uint16_t* b,
                                 hipStream_t stream);

}  // namespace moe

/*
 * moe.h -- C ABI of libmoe, a gfx950 (MI355X) library for the decode step of
 * a routed Mixture-of-Experts block at batch 1 to small batch.
 *
 * What one step computes (page "A Multi-Engine Dataflow for MoE Decoding on
 * Scratchpad-Based Tensor Accelerators", MoE-block background and Fig. 2):
 *
 *     y = sum_e a_e * W_down,e ( phi(W_gate,e h) * (W_up,e h) ),  phi = SiLU,
 *
 * over the k experts the router selects for h, in three calls:
 *     moe_route_topk     router GEMV, top-k, renormalised softmax affinities
 *     moe_align_blocks   canonical alignment of routes into padded b-row blocks
 *     moe_expert_forward gate/up GEMV + SiLU, down GEMV, weighted combine
 * plus moe_create / moe_destroy and a few helpers.
 *
 * Conventions (all entry points):
 *  - Device pointers are device (HBM) addresses on the current HIP device;
 *    `cfg`, `w` (the structs themselves), `out` and the *_host arguments are
 *    host pointers.  Every device buffer is owned by the caller.  Weights are
 *    borrowed zero-copy by moe_create and must outlive the context.  The
 *    context owns only its workspace (allocated in moe_create, freed in
 *    moe_destroy).
 *  - Every call enqueues asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream) and never synchronises, except where stated.
 *    Counts produced on the device stay on the device.
 *  - Errors are returned as moe_status.  All host-side checks run before any
 *    launch: on an error nothing is enqueued.  Unsupported shapes or formats
 *    fail closed at moe_create with MOE_ERR_UNSUPPORTED; there is no fallback
 *    path.  Anomalies only visible on the device (an expert id outside
 *    [0, E), an alignment plan inconsistent with the routes) are skipped,
 *    never read or written out of bounds, and set a sticky flag readable with
 *    moe_read_device_error.
 *  - A context serves one stream at a time and is not thread-safe; calls
 *    that overlap on one context race on its workspace.
 *  - Layouts are row-major.  bf16 values are passed as their 16-bit patterns.
 *  - Results are bitwise reproducible run to run: no floating-point atomics
 *    are used and every reduction order is a function of the shape alone.
 */
#ifndef MOE_H
#define MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null pointer, negative or oversized count, bad struct field */
    MOE_ERR_UNSUPPORTED = 2,   /* shape/format outside what the kernels implement (fail closed) */
    MOE_ERR_CAPACITY = 3,      /* M above the context's max_tokens, K above max_keep */
    MOE_ERR_HIP = 4,           /* a HIP runtime call failed */
    MOE_ERR_DEVICE = 5         /* moe_read_device_error found a sticky device flag */
} moe_status;

/* Weight formats of the gate and up projections (down is always dense bf16). */
enum {
    MOE_WFORMAT_DENSE = 0,     /* bf16 [E][I][H] */
    MOE_WFORMAT_VQLR = 1       /* VQ + low rank (see moe_weights) */
};

/* Device error flag bits (moe_read_device_error). */
enum {
    MOE_DEVERR_BAD_ROUTE_ID = 1,      /* a top-k id outside [0, E) (route skipped) */
    MOE_DEVERR_BAD_PLAN = 2,          /* a plan row whose id disagrees with its block (row skipped) */
    MOE_DEVERR_BAD_BLOCK_EXPERT = 4,  /* a block_expert entry outside [0, E) (block skipped) */
    MOE_DEVERR_BAD_COUNTS = 8         /* counts[] beyond the plan capacity (clamped) */
};

/*
 * Shapes and options of one MoE layer.
 *  H, I, E     hidden size, channels per expert, number of experts.
 *              Supported: H % 8 == 0, 8 <= H <= 8192; 1 <= I <= 16384;
 *              E % 8 == 0, 8 <= E <= 1024.
 *  top_k       experts per token, 1 <= top_k <= min(E, 32).
 *  block_b     alignment block size (8 on the pages); 1 <= block_b <= 64.
 *  max_tokens  largest M any call will pass (sizes the workspace), 1..4096,
 *              with max_tokens*top_k <= 4096 and
 *              ceil(max_tokens*top_k/64)*E <= 6144 (alignment runs in one
 *              workgroup's LDS).
 *  wformat     MOE_WFORMAT_DENSE or MOE_WFORMAT_VQLR.
 *  vq_d, vq_K, lr_r   VQ block length, code book size and low-rank rank for
 *              MOE_WFORMAT_VQLR: vq_d in {2, 4, 8}, 1 <= vq_K <= 256,
 *              H % (8*vq_d) == 0, H/vq_d <= 1024, lr_r % 8 == 0 and
 *              0 <= lr_r <= 512 (0: VQ only, no low-rank term; lr_basis
 *              and lr_coef may then be NULL).  Ignored for dense.
 *  max_keep    largest channel top-K moe_expert_forward will be asked for
 *              (0 = channel-sparse mode unused); <= top_k*I, top_k*I <= 8192,
 *              dense format only.
 *  reader      channel scores of the channel-sparse mode: 0 = the static
 *              scores chan_norm, 1 = the ternary-sketch reader (page "Channel
 *              Selection for Mixture-of-Experts Decoding Needs No Calibration
 *              Data", Stages 1 and 2): needs max_keep > 0, H % 128 == 0, and
 *              the weights rot_signs, sketch, sketch_scale, down_norm.
 *  rec_rank    with reader = 1: 0 (no recovery) or the rank of the recovery
 *              map of the discarded channels (Stage 3), 8..32, % 8 == 0;
 *              needs rec_basis and rec_coef.
 */
typedef struct {
    int32_t H, I, E, top_k, block_b, max_tokens;
    int32_t wformat;
    int32_t vq_d, vq_K, lr_r;
    int32_t max_keep;
    int32_t reader, rec_rank;
} moe_config;

/*
 * Device pointers to one layer's weights (borrowed; must outlive the ctx).
 *  router_w     bf16 [H][E]                     required
 *  router_bias  fp32 [E] added to the logits    or NULL
 *  w_gate, w_up bf16 [E][I][H]; row j of expert e is channel j's gate/up row
 *               (required for MOE_WFORMAT_DENSE, ignored for VQLR)
 *  w_down       bf16 [E][I][H]; row j is channel j's down column, stored
 *               contiguously ("transposed at load", page "Channel Selection
 *               for Mixture-of-Experts Decoding Needs No Calibration Data",
 *               Stage 2)                        required
 *  chan_norm    fp32 [E][I], static channel scores n[e][j] for the
 *               channel-sparse mode (see moe_channel_norms); or NULL
 *  For MOE_WFORMAT_VQLR, index [0] is the gate projection and [1] the up
 *  projection (page "A Multi-Engine Dataflow ...", Sec. 3.1 Eq. 1 and Sec. 2.3):
 *  lr_basis[P]  bf16 [H][lr_r]   shared basis D_P
 *  lr_coef[P]   bf16 [E][I][lr_r] private coefficients, row j = C_P,e^T column j
 *  vq_book[P]   bf16 [vq_K][vq_d] shared weight code book B_P
 *  vq_idx[P]    uint8 [E][I][H/vq_d] private index map: entry [e][j][b] picks
 *               the code word of rows vq_d*b .. vq_d*b+vq_d-1 of channel j
 *               (entries >= vq_K select a zero code word; nothing is read
 *               past the code book)
 *  The reconstructed gate/up weight of channel j, row i is
 *      sum_rho D_P[i][rho] C_P,e[j][rho] + B_P[J_P,e[j][i / vq_d]][i % vq_d].
 *  For the reader (cfg->reader = 1; nblk = H / 128, rowb =
 *  moe_sketch_row_bytes(I)), all made at load time from the weights alone:
 *  rot_signs    int8 [nblk][128] of +-1: the random signs sigma of the
 *               rotation R = H_128 diag(sigma) / sqrt(128) of every 128-block
 *               (the same for every row and for h)
 *  sketch       uint8 [E][2][nblk][128][rowb] (moe_reader_sketch): ternary
 *               codes of the rotated gate ([.][0]) and up ([.][1]) rows, base
 *               3, five channels per byte, one row per rotated coordinate
 *  sketch_scale fp32 [E][2][nblk][I] (moe_reader_sketch)
 *  down_norm    fp32 [E][I] ||down column|| (moe_down_norms)
 *  rec_basis    fp32 [H][rec_rank] (moe_recovery_basis), with rec_rank > 0
 *  rec_coef     bf16 [E][I][rec_rank] (moe_recovery_coefs), with rec_rank > 0
 *  Alignment (checked by moe_create, MOE_ERR_INVALID_ARG otherwise): the bf16
 *  arrays, vq_idx, sketch, chan_norm and down_norm 16 bytes, the other
 *  fp32 / int32 arrays 4 bytes.
 */
typedef struct {
    const uint16_t *router_w;
    const float *router_bias;
    const uint16_t *w_gate;
    const uint16_t *w_up;
    const uint16_t *w_down;
    const float *chan_norm;
    const uint16_t *lr_basis[2];
    const uint16_t *lr_coef[2];
    const uint16_t *vq_book[2];
    const uint8_t *vq_idx[2];
    const int8_t *rot_signs;
    const uint8_t *sketch;
    const float *sketch_scale;
    const float *down_norm;
    const float *rec_basis;
    const uint16_t *rec_coef;
} moe_weights;

/*
 * Create a context for one layer: validates `cfg` and the required weight
 * pointers (fail closed), allocates the workspace on the current device.
 * On success *out holds the context; on error *out is NULL.
 */
moe_status moe_create(const moe_config *cfg, const moe_weights *w, moe_ctx **out);

/* Free the workspace.  moe_destroy(NULL) is a no-op.  Waits for the device. */
void moe_destroy(moe_ctx *ctx);

/*
 * Router (page "A Multi-Engine Dataflow ...", MoE-block background; page
 * "Route-Block Membership Selects Packed-AWQ Arithmetic", Sec. 2.1: the
 * router's M x k expert-id array).
 *  h          fp32 [M][H]
 *  M          0..max_tokens (0: nothing is enqueued)
 *  topk_ids   int32 [M][k] out: per token the k largest logits, ties to the
 *             lower expert id, slot s = s-th largest
 *  topk_w     fp32 [M][k] out: softmax over the k selected logits
 *  logits_out fp32 [M][E] out (may be NULL): l = h Wr + bias, fp32 accumulation
 * Each logit is an fp32 sum whose summation tree has depth at most
 *   4 + rpt/8 + 3 + ceil(H / (4 rpt)) + 1, rpt = 2048 / c,
 *   c = 32 experts per column group (16 if E < 32, 8 if E < 16),
 * so |l - exact| <= gamma_depth * (sum_i |h_i Wr_ie| + |bias_e|).  The top-k
 * decision is exact for these fp32 logits.  One launch over (row slice,
 * column group) tiles x groups of 4 tokens; the last tile workgroup of a
 * group to finish adds the row slices in order and takes the group's top-k
 * (integer tickets, no spinning).
 */
moe_status moe_route_topk(moe_ctx *ctx, const float *h, int32_t M,
                          int32_t *topk_ids, float *topk_w, float *logits_out, void *stream);

/*
 * Canonical alignment (page "Route-Block Membership ...", Sec. 2.1, Sec. 3.1
 * Eq. 1, Sec. 5.3): flatten ids row-major into routes r = t*k + s; group the
 * routes with 0 <= id < E by expert in (expert id, route id) order; pad each
 * group with the sentinel M*k to a multiple of block_b; experts in ascending
 * id; experts without routes own no block.  The result is a function of the
 * ids alone (no atomic-order dependence).
 *  topk_ids       int32 [M][k] (device)
 *  sorted_routes  int32 [moe_align_capacity(M,k,E,b)] out; entries past
 *                 num_padded are left untouched
 *  block_expert   int32 [capacity / b] out; entries past num_blocks untouched
 *  counts         int32 [2] out: num_blocks, num_padded (stay on the device)
 * Ids outside [0, E) are skipped and set MOE_DEVERR_BAD_ROUTE_ID.
 */
moe_status moe_align_blocks(moe_ctx *ctx, const int32_t *topk_ids, int32_t M,
                            int32_t *sorted_routes, int32_t *block_expert, int32_t *counts,
                            void *stream);

/*
 * moe_route_topk followed by moe_align_blocks, the alignment done by the
 * router's last workgroup (one launch up to 4 tokens, two above).  Outputs
 * are identical to the two separate calls (same arguments, same meaning).
 */
moe_status moe_route_align(moe_ctx *ctx, const float *h, int32_t M, int32_t *topk_ids, float *topk_w,
                           float *logits_out, int32_t *sorted_routes, int32_t *block_expert, int32_t *counts,
                           void *stream);

/*
 * Experts and combine.
 * Dense / VQ mode (keep_channels == 0): for every valid route (t, s) with
 * expert e = topk_ids[t][s]:
 *     p = SiLU(W_gate,e h_t) * (W_up,e h_t)            (fp32, I values)
 *     y_(t,s) = W_down,e^T p                            (fp32, H values)
 * and y[t] = sum_{s = 0..k-1} topk_w[t][s] * y_(t,s), added in slot order
 * (page "A Multi-Engine Dataflow ...", Sec. 4.3, accumulated summation).
 * Work is organised by the plan (sorted_routes, block_expert, counts from
 * moe_align_blocks or any valid plan for the same ids): every expert's
 * weights are streamed once for all of its routes.  The arithmetic of a route
 * does not depend on its position in the plan, so any valid plan gives
 * bitwise the same y.  A plan that omits a valid route leaves that route's
 * contribution undefined.
 *
 * Channel-sparse mode (keep_channels = K > 0; needs chan_norm, dense format):
 * page "Channel Selection for Mixture-of-Experts Decoding Needs No
 * Calibration Data", Background and Stage 2.  Per token, candidate (s, j)
 * scores a_s * n[e_s][j] (exact fp64 product of two fp32 values); the K best
 * across all k experts are kept (ties: lower expert id, then lower channel,
 * then lower slot), exactly, by one workgroup per token;
 * only the kept gate rows, up rows and down rows are read, and
 *     y[t] = sum over kept (s, j) of a_s * SiLU(g_j.h_t)(v_j.h_t) * d_j.
 * The plan arguments are ignored (may be NULL).  kept_out (int32 [M][K], may
 * be NULL) receives the kept set as s*I + j in ascending order.
 *
 * Reader mode (cfg->reader = 1, keep_channels = K > 0): the same exact
 * compute of the kept channels, but the scores come from the ternary sketch
 * (page "Channel Selection ...", Stages 1 to 3):
 *  1. per 128-block of h, x'' = H_128 diag(sigma) h_blk (fp64, exact for
 *     ordinary fp32 input) and the 80 coordinates of largest |x''| (ties to
 *     the lower coordinate);
 *  2. g_hat_j = sum over blocks of scale_j,blk * sum over the 80 coordinates
 *     of code_j,i * x''_i, likewise v_hat_j from the up sketch (fp32);
 *  3. score (s, j) = (a_s * ||d_j||) * |SiLU(g_hat_j) * v_hat_j| (fp32; NaN
 *     scores as 0), the K best kept, ties to the lower expert id, channel,
 *     then slot -- an exact selection of these fp32 scores;
 *  4. with rec_rank > 0, y[t] += U * sum over the dropped (s, j) of
 *     a_s * p_hat_j * b_j with p_hat_j = SiLU(g_hat_j) * v_hat_j, U =
 *     rec_basis, b_j = rec_coef row j (fp32 sums in a fixed order).
 *
 *  h        fp32 [M][H];  topk_ids int32 [M][k];  topk_w fp32 [M][k]
 *  y        fp32 [M][H] out (fully overwritten)
 */
moe_status moe_expert_forward(moe_ctx *ctx, const float *h, int32_t M,
                              const int32_t *topk_ids, const float *topk_w,
                              const int32_t *sorted_routes, const int32_t *block_expert,
                              const int32_t *counts, int32_t keep_channels,
                              int32_t *kept_out, float *y, void *stream);

/*
 * One decode step in one call: moe_route_align (moe_route_topk when
 * keep_channels > 0) followed by moe_expert_forward, with the same arguments
 * and the same outputs bit for bit (pages "A Multi-Engine Dataflow ...",
 * MoE-block background: routing then the routed experts; "Route-Block
 * Membership ...", Sec. 2.1 and Sec. 3.1: the id array and its canonical
 * plan).  With keep_channels > 0 the plan arguments are ignored (may be NULL).
 *
 * For one token with dense weights (H <= 4096, E <= 512) the step is three
 * launches with no hand-off between workgroups: the router GEMV writes its
 * row-slice partials; every workgroup of the fused expert kernel adds them,
 * takes the top-k and softmax and finds its own expert (one block per
 * selected expert); the combine adds the partials.  In channel-sparse mode
 * (keep_channels > 0) the router GEMV writes the partials of all M tokens
 * and each workgroup of the selection-and-gather launch takes its token's
 * top-k and softmax before selecting.  In reader mode the router
 * GEMV launch also rotates and scans h in workgroups of its own, and every
 * screening workgroup routes its token before reading the sketch (E <= 256;
 * above, the routing is moe_route_topk's and the rotation a launch of its
 * own).  With VQ + low-rank weights (E <= 256, k <= 32) the router GEMV
 * launch also forms the z = D^T h partials, every gate/up workgroup routes
 * its token from the router's partials, and up to 64 routes the down
 * launch adds the gate/up partials and aligns the routes itself (above, a
 * finishing launch forms SiLU(gate) * up and the plan before it).  Otherwise
 * the calls above are made as they are.
 *  h, y: fp32 [M][H]; topk_ids, topk_w: [M][k] out; logits_out: [M][E] out
 *  or NULL; sorted_routes, block_expert, counts: as moe_align_blocks.
 */
moe_status moe_decode_step(moe_ctx *ctx, const float *h, int32_t M, int32_t *topk_ids, float *topk_w,
                           float *logits_out, int32_t *sorted_routes, int32_t *block_expert, int32_t *counts,
                           int32_t keep_channels, int32_t *kept_out, float *y, void *stream);

/*
 * moe_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no context, no allocation.  Same arguments and outputs as moe_decode_step,
 * with the layer given by `cfg` and `w` (host pointers to the structs;
 * validated on every call as moe_create would) instead of a context.
 *  - The workspace is a device array inside the library of 16 MiB per GPU,
 *    held from the first use until the process ends.  A call whose
 *    workspace (moe_workspace_bytes(cfg, max(M, 1))) exceeds it returns
 *    MOE_ERR_CAPACITY and enqueues nothing.
 *  - Every call on one GPU shares that array: calls that overlap on a GPU
 *    (several streams or threads at once) race; serialise them.
 *  - The first call on a device looks up the array's address
 *    (hipGetSymbolAddress); make it outside graph capture.
 *  - Device-side anomalies are skipped as in moe_decode_step, but their
 *    flags stay in the shared array and are not reported.
 *  - No profiling events are recorded.
 */
moe_status moe_decode_step_noalloc(const moe_config *cfg, const moe_weights *w, const float *h, int32_t M,
                                   int32_t *topk_ids, float *topk_w, float *logits_out, int32_t *sorted_routes,
                                   int32_t *block_expert, int32_t *counts, int32_t keep_channels,
                                   int32_t *kept_out, float *y, void *stream);

/*
 * Diagnostic readout of the reader's stages 1 to 3 (cfg->reader = 1) for
 * given routes: the rotation and scan of h, the screening estimates, the
 * scores and the K-best selection, exactly as moe_expert_forward computes
 * them, copied to caller buffers (device; each may be NULL):
 *  xsel   uint8 [M][H/128][80] scanned coordinates of each block, ascending
 *  xval   fp32 [M][H/128][80]  x'' of those coordinates (rounded to fp32)
 *  est    fp32 [M][k][2][I]    g_hat ([.][0]) and v_hat ([.][1])
 *  score  fp32 [M][k][I]       output-level scores
 *  kept   int32 [M][K]         the kept set as s*I + j, ascending
 * 1 <= K <= max_keep.  Asynchronous on `stream`.
 */
moe_status moe_reader_inspect(moe_ctx *ctx, const float *h, int32_t M, const int32_t *topk_ids,
                              const float *topk_w, int32_t K, uint8_t *xsel, float *xval, float *est,
                              float *score, int32_t *kept, void *stream);

/* ---------------------------------------------------------------- helpers */

/* Rows moe_align_blocks may write: M*k + min(E, M*k)*(b-1); -1 on bad args. */
int32_t moe_align_capacity(int32_t M, int32_t k, int32_t E, int32_t b);

/*
 * Bytes of device workspace a context of `cfg` with max_tokens = max_tokens
 * allocates (router and VQ partials, the p buffer of the split schedule, down
 * partials, channel-selection lists and partials, tickets); host only, no GPU
 * needed.  -1 when cfg is NULL or the configuration (with that max_tokens)
 * would be rejected by moe_create.
 */
int64_t moe_workspace_bytes(const moe_config *cfg, int32_t max_tokens);

/* Static text for a status code. */
const char *moe_status_string(moe_status s);

/*
 * Synchronises the device, copies the sticky device error flags of the
 * context to *flags (host), and clears them when `clear` is non-zero.
 * Returns MOE_ERR_DEVICE when any flag is set, MOE_OK otherwise.
 */
moe_status moe_read_device_error(moe_ctx *ctx, int32_t *flags, int32_t clear);

/*
 * Load-time channel scores for the channel-sparse mode:
 *     norms[e][j] = fp32( ||G_e[j]|| * ||V_e[j]|| * ||D_e[j]|| )
 * with the three Euclidean norms computed in fp64 and rounded once.
 * Inputs bf16 [E][I][H] (device), output fp32 [E][I] (device).  Needs only
 * cfg->H, I, E.  Asynchronous on `stream`.
 */
moe_status moe_channel_norms(const moe_config *cfg, const uint16_t *w_gate, const uint16_t *w_up,
                             const uint16_t *w_down, float *norms, void *stream);


/*
 * Load-time arrays of the reader (page "Channel Selection for
 * Mixture-of-Experts Decoding Needs No Calibration Data", "A Reader Built
 * from Weights Alone": built from the weights alone, no calibration data).
 * Each needs only cfg->H (% 128 == 0 for the sketch), I, E; inputs and
 * outputs are device arrays in the layouts of moe_weights.
 *
 * moe_sketch_row_bytes: bytes of one coordinate row of the sketch,
 * ceil(I / 5) padded to a multiple of 16; -1 when I is out of range.
 *
 * moe_reader_sketch: for every expert, projection (gate, up), block and
 * channel j, the rotated row u = H_128 diag(sigma) w_j,blk (fp64) is coded
 * by the Ternary Weight Networks rule (Li and Liu, 2016): Delta = 0.7 *
 * mean |u_i|, code sign(u_i) where |u_i| > Delta else 0, scale = mean |u_i|
 * over the nonzero codes (0 if none), both sums by pairwise halving
 * (adjacent pairs, then pairs of pairs, ...); sketch_scale = fp32(scale /
 * 128).  Codes are stored base 3 (digit code + 1; channel 5g + m of byte g
 * weighted 3^m; channels past I as code 0; padding bytes zero).  Clears the
 * sketch with hipMemsetAsync first: not for graph capture.
 *
 * moe_down_norms: down_norm[e][j] = fp32(||w_down[e][j]||), the sum of
 * squares in fp64.
 *
 * moe_recovery_basis: U [H][rank] fp32 (1 <= rank <= 32, H % 64 == 0): the
 * eigenvectors of G = sum over all experts and channels of d_j d_j^T for its
 * rank largest eigenvalues, in decreasing order, each column's entry of
 * largest magnitude made positive.  G is formed in fp32; the eigenvectors by
 * `iters` rounds (>= 1) of subspace iteration from a fixed start with
 * Cholesky QR, then a Rayleigh-Ritz step (Jacobi rotations in fp64): an
 * approximation whose accuracy grows with iters and the eigenvalue gaps.
 * Allocates and frees a scratch of about 4 H^2 bytes and synchronises the
 * stream.
 *
 * moe_recovery_coefs: b[e][j] = U^T d_j (fp32 sums), rounded to bf16
 * (nearest even): bf16 [E][I][rank], 8 <= rank <= 32, rank % 8 == 0.
 */
int32_t moe_sketch_row_bytes(int32_t I);
moe_status moe_reader_sketch(const moe_config *cfg, const uint16_t *w_gate, const uint16_t *w_up,
                             const int8_t *rot_signs, uint8_t *sketch, float *sketch_scale, void *stream);
moe_status moe_down_norms(const moe_config *cfg, const uint16_t *w_down, float *down_norm, void *stream);
moe_status moe_recovery_basis(const moe_config *cfg, const uint16_t *w_down, int32_t rank, int32_t iters,
                              float *basis, void *stream);
moe_status moe_recovery_coefs(const moe_config *cfg, const float *basis, int32_t rank, const uint16_t *w_down,
                              uint16_t *coef, void *stream);

/*
 * Host-side check of an alignment plan against its routes (all host
 * pointers; no GPU needed).  Checks: counts in range; every valid route
 * exactly once; rows of a block belong to its expert; pads only at a block's
 * tail and never a whole block; blocks of one expert contiguous and experts
 * ascending; no id outside [0, E) present.  Canonical order inside an expert
 * is NOT required (any valid plan passes).  On failure returns
 * MOE_ERR_INVALID_ARG and writes a code to *reason (host, may be NULL):
 *   1 counts out of range, 2 a route missing, 3 a route duplicated,
 *   4 a row on the wrong expert's block, 5 a pad before a route inside a
 *   block or an all-pad block, 6 blocks out of expert order, 7 an invalid
 *   route id in the plan, 8 a row value out of range.
 */
moe_status moe_validate_plan(const int32_t *topk_ids_host, int32_t M, int32_t k, int32_t E, int32_t b,
                             const int32_t *sorted_routes_host, const int32_t *block_expert_host,
                             const int32_t *counts_host, int32_t *reason);

/* ------------------------------------------------------------- profiling */

/* Kernel identifiers for moe_profile_read. */
enum {
    MOE_KERNEL_ROUTER = 0,        /* router GEMV + top-k + softmax (one launch) */
    MOE_KERNEL_VQ_SHARED = 1,     /* shared projection z = D^T h partials (VQ + low rank) */
    MOE_KERNEL_ALIGN = 2,
    MOE_KERNEL_GATEUP = 3,        /* dense gate/up GEMV + SiLU (several routes per block) */
    MOE_KERNEL_GATEUP_VQLR = 4,   /* VQ + low-rank gate/up + SiLU */
    MOE_KERNEL_DOWN = 5,          /* down GEMV partials */
    MOE_KERNEL_COMBINE = 6,       /* fixed-order weighted combine */
    MOE_KERNEL_CHAN_SELECT = 7,   /* (no longer launched: the top-K runs inside CHAN_GATHER) */
    MOE_KERNEL_CHAN_GATHER = 8,   /* channel top-K + kept-channel gate/up + down partials */
    MOE_KERNEL_CHAN_COMBINE = 9,
    MOE_KERNEL_EXPERT_FUSED = 10, /* dense gate/up + SiLU + down partials (one route per block) */
    MOE_KERNEL_ROUTER_ALIGN = 11, /* router + top-k + softmax + alignment (one launch) */
    MOE_KERNEL_ROUTER_GEMV = 12,  /* router GEMV slice partials only (decode step) */
    MOE_KERNEL_DECODE_FUSED = 13, /* per-workgroup top-k + softmax + plan, then as EXPERT_FUSED */
    MOE_KERNEL_VQ_FINISH = 14,    /* VQ + low rank, more than 64 routes: gate/up partials -> SiLU(gate) * up */
    MOE_KERNEL_READER_ROTATE = 15,  /* reader: rotation and scan of h (own launch) */
    MOE_KERNEL_READER_SCREEN = 16,  /* reader: sketch estimates (routing first in the decode step) */
    MOE_KERNEL_READER_SELECT = 17,  /* reader: output-level scores and top K of moe_reader_inspect (the
                                       forward path selects inside CHAN_GATHER) */
    MOE_KERNEL_READER_RECOVER = 18, /* reader: recovery partials of the dropped channels */
    MOE_KERNEL_READER_COMBINE = 19, /* reader: combine + recovery map */
    MOE_KERNEL_COUNT = 20
};

/*
 * When enabled, every launch of the context carries a pair of HIP events
 * stamped by the kernel's own dispatch (hipExtLaunchKernelGGL), so their
 * elapsed time is the kernel's execution time on its stream.
 * moe_profile_read synchronises, adds the elapsed times of all recorded
 * launches of each kernel into ms[kernel] and launches[kernel] (host arrays
 * of MOE_KERNEL_COUNT), and clears the record.
 */
moe_status moe_profile_enable(moe_ctx *ctx, int32_t enable);
moe_status moe_profile_read(moe_ctx *ctx, double *ms, int64_t *launches);

/* Name of a kernel identifier ("gateup", ...), or NULL. */
const char *moe_kernel_name(int32_t kernel);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */

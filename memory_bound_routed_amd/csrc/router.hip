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
#include "reader_device.h"
#include "topk_device.h"

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

// Router GEMV tiles: the grid covers row slices x column groups of cgw
// experts (32, or 16 / 8 for small E) along x, groups of kTokTile tokens
// along y;
// tpr = cgw/8 threads cover a row of the group with one 16-byte load each,
// rpt = 256/tpr rows per pass, kRowsPerThread passes per slice.  The rpt row
// groups of an output are added by 8 lanes (rpt/8 groups each, in order),
// then by a fixed butterfly over the 8 lanes (pairs, pairs of pairs, quads).  A slice partial is then
// part[slice][t][e] as for slice_partial, but there are cgw/E times fewer
// slices for the last workgroup to add.
constexpr int kRouterCG = 32;
constexpr int kRedPad = 8;  // floats after each of the 8 row-group blocks of a tile's sums
struct RouterTiles {
    int cgw, tpr, rpt, rows, nrs, ncg;
    __host__ __device__ RouterTiles(int H, int E) {
        cgw = E >= 32 ? kRouterCG : (E >= 16 ? 16 : 8);
        tpr = cgw / 8;
        rpt = kThreads / tpr;
        rows = rpt * kRowsPerThread;
        nrs = (H + rows - 1) / rows;
        ncg = (E + cgw - 1) / cgw;
    }
};

template <int TT>
__device__ __forceinline__ void router_tile(const float* __restrict__ h, int M, int t0, int H,
                                            const uint16_t* __restrict__ W, int E, const RouterTiles& tl, int rs,
                                            int cg, float* __restrict__ part, float* red) {
    const int Mg = min(TT, M - t0);  // tokens t0 .. t0+Mg-1 of this workgroup
    const int tid = threadIdx.x;
    const int c8 = tid % tl.tpr;
    const int rg = tid / tl.tpr;
    const int r0 = rs * tl.rows;
    const int e0 = cg * tl.cgw + c8 * 8;     // first of the thread's 8 experts
    const int ec = min(e0, E - 8);           // E % 8 == 0: in range
    // Every load first (rows past H read row H-1, tokens past M token M-1;
    // both are zeroed by a select afterwards).
    uint4 wv[kRowsPerThread];
    float hv[kRowsPerThread][TT];
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int i = min(r0 + rg + u * tl.rpt, H - 1);
        wv[u] = load_stream16(W + (size_t)i * E + ec);
#pragma unroll
        for (int t = 0; t < TT; ++t) hv[u][t] = h[(size_t)(t0 + min(t, Mg - 1)) * H + i];
    }
    const bool col_ok = e0 < E;
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const bool row_ok = col_ok && r0 + rg + u * tl.rpt < H;
#pragma unroll
        for (int t = 0; t < TT; ++t) hv[u][t] = (row_ok && t < Mg) ? hv[u][t] : 0.f;
    }
    float acc[TT][8];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[t][c] = 0.f;
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        float wf[8];
        unpack8(wv[u], wf);
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[t][c] = fmaf(hv[u][t], wf[c], acc[t][c]);
    }
    // red holds the row-group sums [rg][t][col] in 8 blocks of gpl row
    // groups, each block padded by kRedPad floats: a block spans 256 TT
    // floats, a multiple of the LDS banks, so without the padding the 8
    // lanes that read one column (one per block) would hit one bank.
    const int gpl = tl.rpt / 8;  // row groups per block (and per lane below), a multiple of 8
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int c = 0; c < 8; ++c) red[(rg * TT + t) * tl.cgw + c8 * 8 + c + (rg / gpl) * kRedPad] = acc[t][c];
    __syncthreads();
    // output o = t*cgw + c: lanes 8o' .. 8o'+7 of pass p (o = 32p + o'; every
    // lane takes part in the butterfly).  The row groups of a lane (gpl = 8,
    // 16 or 32) are read 8 at a time for every pass at once, and added in
    // row-group order.
    const int sub = tid % 8;
    const int nout = Mg * tl.cgw;
    constexpr int kOutPerPass = kThreads / 8;
    constexpr int NP = (TT * kRouterCG + kOutPerPass - 1) / kOutPerPass;  // passes, nout <= TT * cgw
    float v[NP];
    const float* src[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        v[p] = 0.f;
        const int o = min(p * kOutPerPass + tid / 8, nout - 1);  // clamped reads are dropped below
        const int t = o / tl.cgw, c = o - t * tl.cgw;
        src[p] = red + ((size_t)sub * gpl * TT + t) * tl.cgw + c + sub * kRedPad;
    }
    for (int g0 = 0; g0 < gpl; g0 += 8) {
        float x[NP][8];
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int u = 0; u < 8; ++u) x[p][u] = src[p][(size_t)(g0 + u) * TT * tl.cgw];
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int u = 0; u < 8; ++u) v[p] += x[p][u];
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        // xor 1, xor 2, then the two quads of the 8 lanes (half-row mirror):
        // DPP moves, no LDS round trip
        float w = v[p];
        w += dpp<MOE_DPP_QUAD_XOR1>(w);
        w += dpp<MOE_DPP_QUAD_XOR2>(w);
        w += dpp<MOE_DPP_ROW_HALF_MIRROR>(w);
        const int o = p * kOutPerPass + tid / 8;
        const int t = o / tl.cgw, c = o - t * tl.cgw;
        const int e = cg * tl.cgw + c;
        if (sub == 0 && o < nout && e < E) store_agent(part + ((size_t)rs * M + t0 + t) * E + e, w);
    }
}

// Router: tiles as above; per group of tokens, the last tile workgroup to
// finish (integer ticket) adds the slices in slice order (+ bias) -- every
// partial load is issued before the first add.  The top-k is taken per token
// by one wave from the few keys above a threshold (wave_topk), else by rank
// counting over all keys; either way under the total order (logit desc,
// expert id asc):
// rank(e) = #{e' : l[e'] > l[e] or (l[e'] == l[e] and e' < e)}, and the
// expert of rank s < k goes to slot s.  The ranks are exact, so the result
// does not depend on how the work is split.  NaN logits count as -inf.  The
// softmax over the selected logits adds the denominator in slot order.
//
// Hand-off between workgroups: the slice partials are stored and read
// device-coherently (past the XCD's L2); once every wave's stores have
// completed, one thread per workgroup takes a ticket, and the workgroup
// holding the last ticket reads every slice.  Nothing waits on another
// workgroup, and no cache is written back or invalidated.
// Slice partials requested together per thread: there are few slices, and
// device-coherent loads are served one instruction at a time (clamped
// duplicates would cost as much as real slices).
constexpr int kSliceBatchTiles = 8;

// Selected (expert, logit) of the tokens of the current pass, slot order.
struct TopkLds {
    int e[kTokTile][32];
    float l[kTokTile][32];
};

// Slice sum, top-k and softmax of the nt tokens t0 .. t0+nt-1 (nt <= kTokTile)
// by one workgroup.  LDS: keys [nt][E], then the half-row rank counts
// [2][nt][E].  COHERENT: the slice partials were written by other workgroups
// of this launch.  COHERENT_IDS: ids and weights are read back by another
// workgroup of this launch.  Ends without a barrier.
template <bool COHERENT, bool COHERENT_IDS, int SB>
__device__ __forceinline__ void topk_pass(int t0, int nt, int M, int E, int k, int nslices,
                                          const float* __restrict__ part, const float* __restrict__ bias,
                                          float* __restrict__ logits_out, int32_t* __restrict__ ids,
                                          float* __restrict__ wts, float* red, TopkLds& sel, FastDiv fE) {
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    uint64_t* skey = reinterpret_cast<uint64_t*>(red);
    int* prank = reinterpret_cast<int*>(skey + nt * E);
    const int halfE = E / 2;  // E % 8 == 0: each half is a whole number of 16-byte key pairs
    // Two (token, expert) entries per thread and round: the slice loads of
    // both are in flight together.
    for (int pr0 = tid; pr0 < nt * E; pr0 += 2 * kThreads) {
        int pe[2], te[2], ee[2];
        float bv[2], s[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            pe[i] = pr0 + i * kThreads;
            const int prc = min(pe[i], nt * E - 1);  // a clamped entry is computed and not stored
            const int tq = fE.div(prc);
            te[i] = t0 + tq;
            ee[i] = prc - tq * E;
            bv[i] = bias ? bias[ee[i]] : 0.f;  // issued with the slice loads
            s[i] = 0.f;
        }
        for (int sl0 = 0; sl0 < nslices; sl0 += SB) {
            float x[2][SB];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    const float* q = part + ((size_t)min(sl0 + u, nslices - 1) * M + te[i]) * E + ee[i];
                    x[i][u] = COHERENT ? load_agent(q) : *q;
                }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int u = 0; u < SB; ++u) s[i] += sl0 + u < nslices ? x[i][u] : 0.f;  // slice order
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (pe[i] >= nt * E) continue;
            if (bias) s[i] += bv[i];
            if (logits_out) logits_out[(size_t)te[i] * E + ee[i]] = s[i];
            skey[pe[i]] = order_key((s[i] != s[i]) ? -INFINITY : s[i], ee[i]);
        }
    }
    __shared__ int s_slow;
    __shared__ uint64_t wk[kTokTile][MOE_WAVE];
    __shared__ int wi[kTokTile][MOE_WAVE];
    if (tid == 0) s_slow = E > 4 * MOE_WAVE;
    __syncthreads();
    // Wave w selects token t0 + w by itself (see wave_topk); a token with too
    // many candidates sends the workgroup to the count of every key.
    if (E <= 4 * MOE_WAVE && wave < nt && !wave_topk<4>(skey + wave * E, E, k, sel.e[wave], sel.l[wave], wk[wave],
                                                         wi[wave]))
        s_slow = 1;
    __syncthreads();
    if (s_slow) {
        // rank = # keys of the token above the expert's key, counted in two halves
        for (int it = tid; it < 2 * nt * E; it += kThreads) {
            const int half = it >= nt * E ? 1 : 0, pr = it - half * nt * E;
            const int tl = fE.div(pr);
            prank[it] = count_greater(skey + tl * E, half * halfE, halfE, skey[pr]);
        }
        __syncthreads();
        for (int pr = tid; pr < nt * E; pr += kThreads) {
            const int rank = prank[pr] + prank[nt * E + pr];
            if (rank < k) {
                const int tl = fE.div(pr);
                const uint64_t key = skey[pr];
                sel.e[tl][rank] = key_expert(key);
                sel.l[tl][rank] = key_logit(key);
            }
        }
        __syncthreads();
    }
    if (wave < nt) {  // wave w: token t0 + w; lane s: slot s
        const int t = t0 + wave;
        const float w = topk_softmax(sel.l[wave][min(lane, k - 1)], lane, k);
        if (lane < k) {
            if (COHERENT_IDS) {
                store_agent(ids + (size_t)t * k + lane, sel.e[wave][lane]);
                store_agent(wts + (size_t)t * k + lane, w);
            } else {
                ids[(size_t)t * k + lane] = sel.e[wave][lane];
                wts[(size_t)t * k + lane] = w;
            }
        }
    }
}

// Token group g = blockIdx.y (tokens g*TT ..): the group's tiles, then -- in
// the last tile workgroup of the group to finish (ticket 1 + g) -- the slice
// sum, top-k and softmax of the group's tokens.  Returns true in that
// workgroup (which has written the group's ids and weights; its selections
// stay in sel).  COHERENT_IDS: the ids are read by another workgroup of the
// launch.
template <int TT, bool COHERENT_IDS>
__device__ __forceinline__ bool router_body(const float* __restrict__ h, int M, int H, const uint16_t* __restrict__ Wr,
                                            int E, const float* __restrict__ bias, int k, float* __restrict__ part,
                                            unsigned* __restrict__ ticket, int32_t* __restrict__ ids,
                                            float* __restrict__ wts, float* __restrict__ logits_out, float* red,
                                            TopkLds& sel, FastDiv fE) {
    __shared__ int s_last;
    const RouterTiles tl(H, E);
    const int t0 = blockIdx.y * TT;
    router_tile<TT>(h, M, t0, H, Wr, E, tl, blockIdx.x % tl.nrs, blockIdx.x / tl.nrs, part, red);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(ticket + 1 + blockIdx.y, 1u) == (unsigned)(tl.nrs * tl.ncg - 1);
    __syncthreads();
    if (!s_last) return false;
    topk_pass<true, COHERENT_IDS, kSliceBatchTiles>(t0, min(TT, M - t0), M, E, k, tl.nrs, part, bias, logits_out, ids,
                                                    wts, red, sel, fE);
    return true;
}

// A ticket's last workgroup re-arms it for the next call on this context
// (after its last barrier, so nothing waits for the atomic).
__device__ __forceinline__ void rearm_ticket(unsigned* ticket) {
    if (threadIdx.x == 0) atomicExch(ticket, 0u);
}

// ticket: [0] alignment ticket, [1 + g] token group g; zeroed, left zeroed.
__global__ void __launch_bounds__(kThreads)
router_kernel(const float* __restrict__ h, int M, int H, const uint16_t* __restrict__ Wr, int E,
              const float* __restrict__ bias, int k, float* __restrict__ part, unsigned* __restrict__ ticket,
              int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits_out, FastDiv fE) {
    extern __shared__ __align__(16) float red[];
    __shared__ TopkLds sel;
    pin_arg(bias); pin_arg(k); pin_arg(E); pin_arg(M); pin_arg(ids); pin_arg(wts); pin_arg(logits_out);
    pin_arg(ticket); pin_arg(part); pin_arg(fE.m); pin_arg(fE.s);
    const bool last =
        M == 1 ? router_body<1, false>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red, sel, fE)
               : router_body<kTokTile, false>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red, sel,
                                              fE);
    if (last) rearm_ticket(ticket + 1 + blockIdx.y);
}

// Router, then the canonical alignment of all M*k routes.  One token group
// (M <= 4): its last workgroup aligns -- up to 64 routes by wave 0 from the
// selections still in LDS, else the whole workgroup from the ids it has
// written (the barrier makes them visible to it).  Several groups: each
// group's last workgroup publishes its ids device-coherently and, once its
// stores have completed, takes the alignment ticket; the last one aligns,
// reading the ids device-coherently.
//
// Workgroups past the router's tiles (x >= its tile count) compute the
// tiles of up to kMaxJobs skinny GEMVs on the same h instead (the VQ +
// low-rank format's z = D^T h, as gemv_partials_kernel) and take no ticket.
__global__ void __launch_bounds__(kThreads)
router_align_kernel(const float* __restrict__ h, int M, int H, const uint16_t* __restrict__ Wr, int E,
                    const float* __restrict__ bias, int k, float* __restrict__ part, unsigned* __restrict__ ticket,
                    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits_out, int b,
                    int32_t* __restrict__ sorted_routes, int32_t* __restrict__ block_expert,
                    int32_t* __restrict__ counts, int32_t* __restrict__ err, FastDiv fE, FastDiv fk, FastDiv fb,
                    GemvJobs jobs, int njobs) {
    extern __shared__ __align__(16) float red[];
    __shared__ TopkLds sel;
    __shared__ int s_last;
    {
        const RouterTiles rt(H, E);
        int x = (int)blockIdx.x - rt.nrs * rt.ncg;
        if (x >= 0) {
            for (int j = 0; j < njobs; ++j) {  // uniform
                const GemvJob& jb = jobs.job[j];
                const RouterTiles tj(H, jb.N);
                if (x < tj.nrs * tj.ncg) {
                    if (M == 1)
                        router_tile<1>(h, M, 0, H, jb.W, jb.N, tj, x % tj.nrs, x / tj.nrs, jb.part, red);
                    else
                        router_tile<kTokTile>(h, M, blockIdx.y * kTokTile, H, jb.W, jb.N, tj, x % tj.nrs,
                                              x / tj.nrs, jb.part, red);
                    return;
                }
                x -= tj.nrs * tj.ncg;
            }
            return;
        }
    }
    pin_arg(bias); pin_arg(k); pin_arg(E); pin_arg(M); pin_arg(ids); pin_arg(wts); pin_arg(logits_out);
    pin_arg(ticket); pin_arg(part); pin_arg(b); pin_arg(sorted_routes); pin_arg(block_expert); pin_arg(counts);
    pin_arg(err); pin_arg(fE.m); pin_arg(fE.s); pin_arg(fk.m); pin_arg(fk.s); pin_arg(fb.m); pin_arg(fb.s);
    const bool last =
        M == 1 ? router_body<1, false>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red, sel, fE)
               : router_body<kTokTile, true>(h, M, H, Wr, E, bias, k, part, ticket, ids, wts, logits_out, red, sel,
                                             fE);
    if (!last) return;
    const int R = M * k;
    if (gridDim.y == 1) {
        if (R <= MOE_WAVE) {
            // sel was complete at the top-k's last barrier and is only read
            // since; the wave after the softmax waves aligns (the last wave
            // also does a softmax when M == 4), beside the softmax
            const int aw = min(M, kThreads / MOE_WAVE - 1);
            if ((int)threadIdx.x / MOE_WAVE == aw)
                align_wave([&](int r) { const int t = fk.div(r); return sel.e[t][r - t * k]; }, R, E, fb,
                           sorted_routes, block_expert, counts, err);
        } else {
            __syncthreads();
            align_workgroup([&](int r) { return ids[r]; }, R, E, fb, sorted_routes, block_expert, counts, err,
                            reinterpret_cast<int*>(red));
        }
        rearm_ticket(ticket + 1);
        return;
    }
    rearm_ticket(ticket + 1 + blockIdx.y);  // every tile of the group has taken its ticket
    __builtin_amdgcn_s_waitcnt(0);          // this wave's id and weight stores have completed
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(ticket, 1u) == (unsigned)(gridDim.y - 1);
    __syncthreads();
    if (!s_last) return;
    if (R <= MOE_WAVE) {
        if (threadIdx.x < MOE_WAVE)
            align_wave([&](int r) { return load_agent(ids + r); }, R, E, fb, sorted_routes, block_expert, counts, err);
    } else {
        align_workgroup([&](int r) { return load_agent(ids + r); }, R, E, fb, sorted_routes, block_expert, counts, err,
                        reinterpret_cast<int*>(red));
    }
    rearm_ticket(ticket);
}

// Router GEMV only: the tiles' slice partials part[slice][t][e], stored for
// a later launch, whose workgroups add them and take the top-k themselves
// (the expert kernel of the batch-1 decode step, the channel selection, the
// VQ gate/up of the decode step).  Workgroups past the router's tiles compute
// the tiles of up to kMaxJobs skinny GEMVs on the same h first (the VQ +
// low-rank format's z = D^T h, as gemv_partials_kernel), then, with a
// rotation job (rot.signs non-null), rotate and scan the 128-blocks of the
// group's tokens for the channel-selection reader, one block per wave.
__global__ void __launch_bounds__(kThreads)
router_partials_kernel(const float* __restrict__ h, int M, int H, const uint16_t* __restrict__ Wr, int E,
                       float* __restrict__ part, RotJob rot, GemvJobs jobs, int njobs) {
    extern __shared__ __align__(16) float red[];
    const RouterTiles tl(H, E);
    int x = (int)blockIdx.x - tl.nrs * tl.ncg;
    for (int j = 0; x >= 0 && j < njobs; ++j) {  // uniform
        const GemvJob& jb = jobs.job[j];
        const RouterTiles tj(H, jb.N);
        if (x < tj.nrs * tj.ncg) {
            if (M == 1)
                router_tile<1>(h, M, 0, H, jb.W, jb.N, tj, x % tj.nrs, x / tj.nrs, jb.part, red);
            else
                router_tile<kTokTile>(h, M, blockIdx.y * kTokTile, H, jb.W, jb.N, tj, x % tj.nrs, x / tj.nrs,
                                      jb.part, red);
            return;
        }
        x -= tj.nrs * tj.ncg;
    }
    if (x >= 0) {
        const int nblk = H / kReaderBlock;
        const int TT = M == 1 ? 1 : kTokTile;
        const int t0 = blockIdx.y * TT;
        const int job = x * (kThreads / MOE_WAVE) + (int)threadIdx.x / MOE_WAVE;  // (token in group, block)
        const int tt = job / nblk, b = job - tt * nblk;
        if (tt >= TT || t0 + tt >= M) return;  // whole waves; no barrier follows
        const size_t jb = (size_t)(t0 + tt) * nblk + b;
        rotate_scan_wave(h + (size_t)(t0 + tt) * H + b * kReaderBlock, rot.signs + b * kReaderBlock,
                         rot.xsel + jb * kReaderScan, rot.xval + jb * kReaderScan);
        return;
    }
    if (M == 1)
        router_tile<1>(h, M, 0, H, Wr, E, tl, blockIdx.x % tl.nrs, blockIdx.x / tl.nrs, part, red);
    else
        router_tile<kTokTile>(h, M, blockIdx.y * kTokTile, H, Wr, E, tl, blockIdx.x % tl.nrs, blockIdx.x / tl.nrs,
                              part, red);
}

// Slice partials of up to kMaxJobs skinny GEMVs (the VQ + low-rank format's
// z = D^T h of the gate and the up basis), one matrix per grid z, tiled as
// the router: part[slice][t][n] = sum_{i in slice} h[t][i] W[i][n] with
// RouterTiles(H, N).nrs slices (8 at H = 2048 for N >= 32), so a consumer
// adds few slices whatever N is.
__global__ void __launch_bounds__(kThreads)
gemv_partials_kernel(const float* __restrict__ h, int M, int H, GemvJobs jobs) {
    extern __shared__ __align__(16) float red[];
    const GemvJob& jb = jobs.job[blockIdx.z];
    const RouterTiles tl(H, jb.N);
    if ((int)blockIdx.x >= tl.nrs * tl.ncg) return;
    if (M == 1)
        router_tile<1>(h, M, 0, H, jb.W, jb.N, tl, blockIdx.x % tl.nrs, blockIdx.x / tl.nrs, jb.part, red);
    else
        router_tile<kTokTile>(h, M, blockIdx.y * kTokTile, H, jb.W, jb.N, tl, blockIdx.x % tl.nrs,
                              blockIdx.x / tl.nrs, jb.part, red);
}

size_t tile_lds_bytes(int H, int N) {
    const RouterTiles tl(H, N);
    return ((size_t)tl.rpt * kTokTile * tl.cgw + 8 * kRedPad) * sizeof(float);
}

// LDS of the one-launch router: the tile's row-group sums, or the keys and
// rank counts of the top-k (8 + 2*4 bytes per token and expert), whichever
// is larger.
size_t router_lds_bytes(int H, int E) {
    const size_t tile = tile_lds_bytes(H, E);
    const size_t topk = (size_t)kTokTile * E * (sizeof(uint64_t) + 2 * sizeof(int));
    return tile > topk ? tile : topk;
}

int router_grid(int H, int E) {
    const RouterTiles tl(H, E);
    return tl.nrs * tl.ncg;
}

}  // namespace

int router_groups(int M) { return M == 1 ? 1 : (M + kTokTile - 1) / kTokTile; }

int gemv_slices(int H, int N) { return RouterTiles(H, N).nrs; }

hipError_t launch_gemv_partials(const float* h, int M, int H, const GemvJob* jobs, int njobs, hipStream_t stream) {
    if (njobs < 1 || njobs > kMaxJobs || M < 1) return hipErrorInvalidValue;
    GemvJobs js{};
    size_t lds = 0;
    int grid = 0;
    for (int i = 0; i < njobs; ++i) {
        if (jobs[i].N < 8 || jobs[i].N % 8) return hipErrorInvalidValue;
        js.job[i] = jobs[i];
        lds = tile_lds_bytes(H, jobs[i].N) > lds ? tile_lds_bytes(H, jobs[i].N) : lds;
        grid = router_grid(H, jobs[i].N) > grid ? router_grid(H, jobs[i].N) : grid;
    }
    MOE_LAUNCH(gemv_partials_kernel, dim3(grid, router_groups(M), njobs), dim3(kThreads), lds, stream, h, M, H, js);
    return hipGetLastError();
}

int router_slices(int H, int E) { return RouterTiles(H, E).nrs; }

hipError_t launch_router_partials(const float* h, int M, int H, const uint16_t* Wr, int E, float* part,
                                  hipStream_t stream, const RotJob* rot, const GemvJob* jobs, int njobs) {
    if (M < 1 || E % 8 != 0 || njobs < 0 || njobs > kMaxJobs || (njobs > 0 && !jobs)) return hipErrorInvalidValue;
    const RouterTiles tl(H, E);
    size_t lds = ((size_t)tl.rpt * (M == 1 ? 1 : kTokTile) * tl.cgw + 8 * kRedPad) * sizeof(float);
    int grid = router_grid(H, E);
    GemvJobs js{};
    for (int i = 0; i < njobs; ++i) {
        if (jobs[i].N < 8 || jobs[i].N % 8) return hipErrorInvalidValue;
        js.job[i] = jobs[i];
        lds = tile_lds_bytes(H, jobs[i].N) > lds ? tile_lds_bytes(H, jobs[i].N) : lds;
        grid += router_grid(H, jobs[i].N);
    }
    RotJob rj{};
    if (rot) {
        if (H % kReaderBlock || !rot->signs || !rot->xsel || !rot->xval) return hipErrorInvalidValue;
        const int jobs = (M == 1 ? 1 : kTokTile) * (H / kReaderBlock);
        grid += (jobs + kThreads / MOE_WAVE - 1) / (kThreads / MOE_WAVE);
        rj = *rot;
    }
    MOE_LAUNCH(router_partials_kernel, dim3(grid, router_groups(M)), dim3(kThreads), lds, stream, h, M, H, Wr, E,
               part, rj, js, njobs);
    return hipGetLastError();
}

hipError_t launch_router_align(const float* h, int M, int H, const uint16_t* Wr, int E, const float* bias, int k,
                               float* part, unsigned* ticket, int32_t* ids, float* wts, float* logits_out, int b,
                               int32_t* sorted_routes, int32_t* block_expert, int32_t* counts, int32_t* err,
                               hipStream_t stream, const GemvJob* jobs, int njobs) {
    if (M < 1 || E % 8 != 0 || njobs < 0 || njobs > kMaxJobs || (njobs > 0 && !jobs)) return hipErrorInvalidValue;
    const size_t la = align_lds_bytes(M * k, E);
    size_t lds = router_lds_bytes(H, E) > la ? router_lds_bytes(H, E) : la;
    GemvJobs js{};
    int grid = router_grid(H, E);
    for (int i = 0; i < njobs; ++i) {
        if (jobs[i].N < 8 || jobs[i].N % 8) return hipErrorInvalidValue;
        js.job[i] = jobs[i];
        lds = tile_lds_bytes(H, jobs[i].N) > lds ? tile_lds_bytes(H, jobs[i].N) : lds;
        grid += router_grid(H, jobs[i].N);
    }
    MOE_LAUNCH(router_align_kernel, dim3(grid, router_groups(M)), dim3(kThreads), lds, stream, h, M, H, Wr, E, bias,
               k, part, ticket, ids, wts, logits_out, b, sorted_routes, block_expert, counts, err,
               FastDiv((uint32_t)E), FastDiv((uint32_t)k), FastDiv((uint32_t)b), js, njobs);
    return hipGetLastError();
}

hipError_t launch_router(const float* h, int M, int H, const uint16_t* Wr, int E, const float* bias, int k,
                         float* part, unsigned* ticket, int32_t* ids, float* wts, float* logits_out,
                         hipStream_t stream) {
    if (M < 1 || E % 8 != 0) return hipErrorInvalidValue;
    MOE_LAUNCH(router_kernel, dim3(router_grid(H, E), router_groups(M)), dim3(kThreads), router_lds_bytes(H, E), stream,
               h, M, H, Wr, E,
                       bias, k, part, ticket, ids, wts, logits_out, FastDiv((uint32_t)E));
    return hipGetLastError();
}

}  // namespace moe

// The channel-selection reader (page "Channel Selection for Mixture-of-
// Experts Decoding Needs No Calibration Data": "A Reader Built from Weights
// Alone", Stage 1 "Screen with a Ternary Sketch", Stage 2 "Compute the Top k
// Exactly with Output-Level Scores", Stage 3 "Recover Discarded Channels with
// a rank-32 Map"; the sketch format, Eq. 1 and Eq. 2 are lost in the page's
// text -- the readings are stated where they are used).
//
// Decode time, per token:
//  1. rotation and partial scan of h (reader_device.h): per 128-block the 80
//     coordinates of largest |x''|, x'' = H_128 diag(sigma) h exact in fp64;
//  2. screening (reader_screen_kernel): for every routed expert, gate and up,
//     g_hat_j = sum over blocks of scale_j,blk * sum over the scanned
//     coordinates of c_j,i x''_i, from the base-3 sketch rows of the scanned
//     coordinates only;
//  3. selection (reader_select_kernel): score w_s ||d_j|| |SiLU(g_hat) v_hat|,
//     the K best of the token's k * I candidates by an exact radix select
//     over a total order (score, then expert id, channel, slot), the kept
//     lists per slot for the gather of chansparse.hip;
//  4. with the recovery map: (reader_recover_kernel) r = sum over the dropped
//     candidates of w_s p_hat_j b_j, p_hat_j = SiLU(g_hat_j) v_hat_j, then
//     (reader_combine_kernel) y = sum of the gather's chunk partials + U r.
// Load time: the sketch (reader_sketch_kernel), the down-column norms, the
// recovery basis U (top-32 eigenvectors of the Gram matrix of the stacked down
// columns, by subspace iteration with a Rayleigh-Ritz step) and b_j = U^T d_j.
//
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "device_common.h"
#include "launch.h"
#include "reader_device.h"
#include "select_device.h"
#include "topk_device.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kRowGroups = 64;   // screening: row groups of a workgroup (4 lanes each)
constexpr int kRangeCh = 80;     // screening: channels per workgroup (16 bytes of a row)
constexpr int kMaxRank = 32;

// ---------------------------------------------------------------------------
// Rotation jobs of a launch of their own (the separate-calls path; the
// one-call decode step does them in the router launch's spare workgroups).
__global__ void __launch_bounds__(kThreads)
reader_rotate_kernel(const float* __restrict__ h, int M, int H, const int8_t* __restrict__ signs,
                     uint8_t* __restrict__ xsel, float* __restrict__ xval) {
    const int nblk = H / kReaderBlock;
    const int job = blockIdx.x * kWaves + threadIdx.x / MOE_WAVE;
    if (job >= M * nblk) return;  // whole waves
    const int t = job / nblk, b = job - t * nblk;
    rotate_scan_wave(h + (size_t)t * H + b * kReaderBlock, signs + b * kReaderBlock,
                     xsel + (size_t)job * kReaderScan, xval + (size_t)job * kReaderScan);
}

// ---------------------------------------------------------------------------
// Screening.  The work of one token is cut into units (pair, c, bq): pair =
// 2 s + P (projection P of slot s's expert), c the range of 80 channels
// 80 c .. 80 c + 79 (bytes 16 c .. 16 c + 15 of every coordinate row) and bq
// the group of bpw consecutive 128-blocks bq * bpw .. (nbq = ceil(nblk /
// bpw) groups, bpw = ceil(nblk / 2)).  A workgroup per unit writes the
// group's partial estimate est[t][s][P][bq][j]; the selection adds the nbq
// partials in order.  The grid's x runs over groups of 8 pairs times the
// (c, bq) units with the pair varying fastest (x = pair % 8 + 8 (u + nu
// (pair / 8)), u = c + nseg bq): workgroups are dealt to the 8 XCDs
// round-robin by their linear id, so all units of one pair -- which read the
// same cache lines of the same rows -- share one XCD's L2, while the pairs
// spread over the XCDs.
//
// Thread (row group rg = tid / 4, word w = tid % 4): local block bl = rg %
// bpw, the scanned coordinates n = q, q + Pb, ... with q = rg / bpw and Pb =
// 64 / bpw groups per block; bytes 16 c + 4 w .. + 3 of each such row
// (channels 80 c + 20 w .. + 19).  Each row's 4 bytes are decoded with a
// 243-entry table of codes in LDS and accumulated against x''; the sum of a
// row group is scaled by its block's scale, and the 64 row groups are added
// in order.  The group's scanned coordinates are staged in LDS (their loads
// issued before the routing); the scales are loaded with the rows.  ROUTE:
// every workgroup first routes its token from the router's slice partials
// with the router's arithmetic (E <= 256).
constexpr int kMaxBpw = 32;                                      // nblk <= 64
constexpr int kMaxGroups = kReaderMaxGroups;
constexpr int kStageS = (kMaxBpw * kReaderScan / 16 + kThreads - 1) / kThreads;  // 16-byte coordinate chunks per thread
constexpr int kStageV = (kMaxBpw * kReaderScan / 4 + kThreads - 1) / kThreads;   // 16-byte value chunks per thread
static_assert(kReaderScan % 16 == 0, "a block's scanned coordinates are whole 16-byte chunks");
constexpr int kRowBatch = 10;                                    // rows in flight per thread

template <bool ROUTE>
__global__ void __launch_bounds__(kThreads)
reader_screen_kernel(ReaderArgs ra, SelRoute route, const int32_t* __restrict__ topk_ids, int nseg) {
    __shared__ float4 lut4[243];
    __shared__ float lut1[243];
    __shared__ float red[kRowGroups][kRangeCh + 1];
    __shared__ __align__(16) uint8_t s_sel[kMaxBpw * kReaderScan];
    __shared__ __align__(16) float s_val[kMaxBpw * kReaderScan];
    __shared__ int s_e;
    const int x = blockIdx.x;
    const int nbq = ra.nbq, bpw = ra.bpw;
    const int nu = nseg * nbq;
    const int pair = x % 8 + 8 * (x / (8 * nu));
    const int u0 = (x / 8) % nu;
    const int c = u0 % nseg;
    const int bq = u0 / nseg;
    const int t = blockIdx.y;
    const int k = ra.k;
    if (pair >= 2 * k) return;  // whole workgroup, before any barrier
    const int s = pair >> 1;
    const int P = pair & 1;
    const int tid = threadIdx.x;
    const int w = tid % 4;
    const int rg = tid / 4;
    const int nblk = ra.nblk;
    const int I = ra.I;
    const int b0 = bq * bpw;
    const int nbh = min(bpw, nblk - b0);  // blocks of this group

    // scanned coordinates and values of the group's blocks (independent of
    // the routing), as 16-byte buffer loads: nst is a multiple of 80, so of 16
    const int nst = nbh * kReaderScan;
    uint4 st_sel[kStageS];
    uint4 st_val[kStageV];
    {
        const __amdgpu_buffer_rsrc_t gs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(ra.xsel) + ((size_t)t * nblk + b0) * kReaderScan, (short)0, nst, 0x00020000);
        const __amdgpu_buffer_rsrc_t gv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(ra.xval) + ((size_t)t * nblk + b0) * kReaderScan, (short)0, nst * 4, 0x00020000);
#pragma unroll
        for (int u = 0; u < kStageS; ++u) {
            const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(gs, 16 * (tid + kThreads * u), 0, 0);
            st_sel[u] = make_uint4(x.x, x.y, x.z, x.w);
        }
#pragma unroll
        for (int u = 0; u < kStageV; ++u) {
            const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(gv, 16 * (tid + kThreads * u), 0, 0);
            st_val[u] = make_uint4(x.x, x.y, x.z, x.w);
        }
    }
    // the code table: digit m of byte v (base 3) minus 1
    if (tid < 243) {
        int v = tid;
        float d[5];
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            d[m] = (float)(v % 3 - 1);
            v /= 3;
        }
        lut4[tid] = make_float4(d[0], d[1], d[2], d[3]);
        lut1[tid] = d[4];
    }

    if constexpr (ROUTE) {
        // the token's routing (the router's arithmetic); pair 0, unit 0
        // stores the ids, weights and logits
        __shared__ RouteLds<kThreads> rlt;
        route_token<kThreads>(route.part, route.bias, route.nslices, route.M, t, ra.E, k, x == 0, route.logits,
                              route.ids, route.wts, rlt, false);
        if (tid == 0) s_e = rlt.sel_e[s];
    } else {
        if (tid == 0) s_e = topk_ids[(size_t)t * k + s];
    }
#pragma unroll
    for (int u = 0; u < kStageS; ++u) {
        const int i = tid + kThreads * u;  // 16-byte chunk
        if (16 * i < nst) reinterpret_cast<uint4*>(s_sel)[i] = st_sel[u];
    }
#pragma unroll
    for (int u = 0; u < kStageV; ++u) {
        const int i = tid + kThreads * u;
        if (4 * i < nst) reinterpret_cast<uint4*>(s_val)[i] = st_val[u];
    }
    __syncthreads();
    const int e = s_e;
    const bool valid = e >= 0 && e < ra.E;
    const int ec = valid ? e : 0;

    // this thread's rows: local block bl, scanned coordinates q, q + Pb, ... (< 80)
    const int Pb = kRowGroups / bpw;
    const int bl = rg % bpw;
    const int q = rg / bpw;
    const bool active = q < Pb && bl < nbh;
    const int b = b0 + min(bl, nbh - 1);
    const int nrows = active ? (kReaderScan - q + Pb - 1) / Pb : 0;  // rows of this group
    const uint8_t* rows = ra.sketch + (((size_t)ec * 2 + P) * nblk + b) * kReaderBlock * ra.rowb + 16 * c + 4 * w;
    const uint8_t* ssel = s_sel + min(bl, nbh - 1) * kReaderScan;
    const float* sval = s_val + min(bl, nbh - 1) * kReaderScan;
    // the block's scales of this thread's 20 channels, loaded with the first rows
    const int ch0 = kRangeCh * c + 20 * w;
    const float* scl = ra.scale + (((size_t)ec * 2 + P) * nblk + b) * I;
    float sv[20];
    if (I % 4 == 0 && ch0 + 20 <= I && (reinterpret_cast<uintptr_t>(ra.scale) & 15u) == 0) {
        // five 16-byte loads (16-byte aligned: rows of I fp32, offsets of 20 channels); the
        // screening's time goes into issuing its many small loads, so fewer instructions count
#pragma unroll
        for (int m4 = 0; m4 < 5; ++m4) {
            const float4 v = *reinterpret_cast<const float4*>(scl + ch0 + 4 * m4);
            sv[4 * m4] = v.x;
            sv[4 * m4 + 1] = v.y;
            sv[4 * m4 + 2] = v.z;
            sv[4 * m4 + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int m = 0; m < 20; ++m) sv[m] = scl[min(ch0 + m, I - 1)];
    }
    float acc[20];
#pragma unroll
    for (int m = 0; m < 20; ++m) acc[m] = 0.f;
    for (int n0 = 0; n0 < nrows; n0 += kRowBatch) {  // uniform per row group
        uint32_t wd[kRowBatch];
        float xv[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            const int n = min(q + (n0 + u) * Pb, kReaderScan - 1);
            wd[u] = *reinterpret_cast<const uint32_t*>(rows + (size_t)ssel[n] * ra.rowb);
            xv[u] = n0 + u < nrows ? sval[n] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                const uint32_t v = (wd[u] >> (8 * y)) & 255u;
                const uint32_t vc = v < 243u ? v : 121u;  // bytes past the codes read as code 0
                const float4 d4 = lut4[vc];
                const float d1 = lut1[vc];
                acc[5 * y] = fmaf(d4.x, xv[u], acc[5 * y]);
                acc[5 * y + 1] = fmaf(d4.y, xv[u], acc[5 * y + 1]);
                acc[5 * y + 2] = fmaf(d4.z, xv[u], acc[5 * y + 2]);
                acc[5 * y + 3] = fmaf(d4.w, xv[u], acc[5 * y + 3]);
                acc[5 * y + 4] = fmaf(d1, xv[u], acc[5 * y + 4]);
            }
        }
    }
    // the block's scale per channel, then the row groups in order
#pragma unroll
    for (int m = 0; m < 20; ++m) red[rg][20 * w + m] = (active && ch0 + m < I) ? sv[m] * acc[m] : 0.f;
    __syncthreads();
    if (tid < kRangeCh && kRangeCh * c + tid < I) {
        float g = 0.f;
        for (int r2 = 0; r2 < kRowGroups; ++r2) g += red[r2][tid];
        ra.est[((((size_t)t * k + s) * 2 + P) * nbq + bq) * I + kRangeCh * c + tid] = valid ? g : 0.f;
    }
}

// ---------------------------------------------------------------------------
// Selection, one workgroup per token.  Candidate idx = s * I + j, thread tid
// owning idx = 8 tid .. 8 tid + 7 (a contiguous run, for the scan of the kept
// flags).  g_hat and v_hat are the screening's group partials added in
// order; the score (w_s * ||d_j||) * |SiLU(g_hat) v_hat| is a non-negative
// fp32 (NaN and invalid slots score 0) whose bit pattern orders like its
// value.
//
// The K best are taken by select_top (select_device.h): bins linear in the
// score between its minimum and maximum, then inside the threshold bin the
// score bits and the complement of the tie key e << 19 | j << 5 | s (invalid
// slots as expert 8191), so that equal scores order by expert id, channel,
// then slot.
__global__ void __launch_bounds__(kSelThreads)
reader_select_kernel(ReaderArgs ra, const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w, int K,
                     FastDiv fI, int32_t* __restrict__ slot_cnt, int32_t* __restrict__ slot_kept,
                     int32_t* __restrict__ kept_out, float* __restrict__ est_out, float* __restrict__ score_out) {
    __shared__ int se[32];
    __shared__ float sw[32];
    __shared__ RadixLds rl;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int I = ra.I, k = ra.k, E = ra.E;
    const int n = k * I;
    if (tid < k) {
        const int e = topk_ids[(size_t)t * k + tid];
        se[tid] = (e >= 0 && e < E) ? e : -1;
        sw[tid] = topk_w[(size_t)t * k + tid];
    }
    __syncthreads();
    uint32_t sb[kSelPer], tb[kSelPer], smax, smin;
    unsigned vmask;
    reader_scores(ra, t, fI, se, sw, sb, tb, vmask, smax, smin, est_out, score_out);
    const bool all = K >= n;
    unsigned kmask = vmask;
    if (!all) {
        uint32_t mx, mn;
        block_max_min(smax, smin, rl, &mx, &mn);  // non-negative scores: bits order like values
        const float lo = __uint_as_float(mn);
        const float scl = linear_scale(lo, __uint_as_float(mx), kRadixBins);
        int bin[kSelPer];
        uint32_t key[2][kSelPer];
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            bin[u] = linear_bin(__uint_as_float(sb[u]), lo, scl, kRadixBins);
            key[0][u] = sb[u];
            key[1][u] = ~tb[u];
        }
        kmask = select_top<2>(bin, key, vmask, K, rl);
    }
    emit_kept(kmask, t, k, I, K, all, fI, rl, slot_cnt, slot_kept, kept_out, ra.kept_flag);
}

// ---------------------------------------------------------------------------
// Recovery partials.  Grid (channel chunks of 256, k, M): thread j of slot s
// adds, for a dropped candidate, (w_s p_hat_j) b_j[r] for r < rank, with
// p_hat_j = SiLU(g_hat_j) v_hat_j from the screening's group partials added
// as the selection adds them; the 256 threads are added by a fixed butterfly
// per wave, then the waves in order: rpart[t][s][chunk][r].
__global__ void __launch_bounds__(kThreads)
reader_recover_kernel(ReaderArgs ra, const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w) {
    __shared__ float wpart[kWaves][kMaxRank];
    const int chunk = blockIdx.x, s = blockIdx.y, t = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % MOE_WAVE, wave = tid / MOE_WAVE;
    const int I = ra.I, k = ra.k, rank = ra.rank, nbq = ra.nbq;
    const int j = chunk * kThreads + tid;
    const int e = topk_ids[(size_t)t * k + s];
    const float a = topk_w[(size_t)t * k + s];
    const bool ev = e >= 0 && e < ra.E;
    const int jc = min(j, I - 1);
    const float* eg = ra.est + (((size_t)t * k + s) * 2 * nbq) * I + jc;
    float gp[kMaxGroups], vp[kMaxGroups];
#pragma unroll
    for (int q = 0; q < kMaxGroups; ++q) {
        gp[q] = eg[(size_t)min(q, nbq - 1) * I];
        vp[q] = eg[(size_t)(nbq + min(q, nbq - 1)) * I];
    }
    const bool use = ev && j < I && !ra.kept_flag[((size_t)t * k + s) * I + jc];
    const uint16_t* brow = ra.rec_coef + ((size_t)(ev ? e : 0) * I + jc) * rank;
    uint4 bw[kMaxRank / 8];
#pragma unroll
    for (int r8 = 0; r8 < kMaxRank / 8; ++r8)
        bw[r8] = 8 * r8 < rank ? load16(brow + 8 * r8) : make_uint4(0u, 0u, 0u, 0u);
    float g = gp[0], v = vp[0];
#pragma unroll
    for (int q = 1; q < kMaxGroups; ++q) {
        g += q < nbq ? gp[q] : 0.f;
        v += q < nbq ? vp[q] : 0.f;
    }
    const float coef = use ? a * silu_mul(g, v) : 0.f;
    float contrib[kMaxRank];
#pragma unroll
    for (int r8 = 0; r8 < kMaxRank / 8; ++r8) {
        float f[8];
        unpack8(bw[r8], f);
#pragma unroll
        for (int x = 0; x < 8; ++x) contrib[8 * r8 + x] = use ? coef * f[x] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < kMaxRank; ++r) {
        const float v2 = wave_sum(contrib[r]);
        if (lane == 0) wpart[wave][r] = v2;
    }
    __syncthreads();
    if (tid < rank)
        ra.rpart[(((size_t)t * k + s) * gridDim.x + chunk) * rank + tid] =
            (wpart[0][tid] + wpart[1][tid]) + (wpart[2][tid] + wpart[3][tid]);
}

// y[t][col] = sum over the gather chunks of part[t][chunk][col] plus the
// recovery map's sum_r U[col][r] R[r], R[r] = the token's nrp recovery
// partials added in order.  One wave per workgroup, 16 columns: lane (row
// group g, float4 column c4) adds chunks g, g + 16, ... in order and the
// map's ranks 2g and 2g + 1; the 16 row groups are then combined by a
// butterfly over the lane bits above the column bits (a fixed order).
constexpr int kCombCG = 4;
constexpr int kCombRG = MOE_WAVE / kCombCG;
constexpr int kCombBatch = 8;
constexpr int kRecBatch = 32;

__global__ void __launch_bounds__(MOE_WAVE)
reader_combine_kernel(int H, int nchunks, const float* __restrict__ part, const float* __restrict__ rpart, int nrp,
                      int rank, const float* __restrict__ U, float* __restrict__ y) {
    const int t = blockIdx.y;
    const int lane = threadIdx.x;
    const int cg = lane % kCombCG;
    const int rg = lane / kCombCG;
    const int col = (blockIdx.x * kCombCG + cg) * 4;
    const int r0 = 2 * rg;
    const bool rin = r0 < rank;  // rank is even
    const int rc = rin ? r0 : 0;
    // the map's inputs first: this lane's two ranks of the partials and of U
    float R0 = 0.f, R1 = 0.f;
    const float* rp = rpart + (size_t)t * nrp * rank + rc;
    for (int i0 = 0; i0 < nrp; i0 += kRecBatch) {
        float2 v[kRecBatch];
#pragma unroll
        for (int u = 0; u < kRecBatch; ++u)
            v[u] = *reinterpret_cast<const float2*>(rp + (size_t)min(i0 + u, nrp - 1) * rank);
#pragma unroll
        for (int u = 0; u < kRecBatch; ++u) {
            R0 += i0 + u < nrp ? v[u].x : 0.f;
            R1 += i0 + u < nrp ? v[u].y : 0.f;
        }
    }
    float2 uu[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) uu[x] = *reinterpret_cast<const float2*>(U + (size_t)min(col + x, H - 1) * rank + rc);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* src = part + (size_t)t * nchunks * H + min(col, H - 4);
    for (int c0 = rg; c0 < nchunks; c0 += kCombBatch * kCombRG) {
        float4 v[kCombBatch];
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u)
            v[u] = *reinterpret_cast<const float4*>(src + (size_t)min(c0 + u * kCombRG, nchunks - 1) * H);
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const bool use = c0 + u * kCombRG < nchunks;
            acc.x += use ? v[u].x : 0.f;
            acc.y += use ? v[u].y : 0.f;
            acc.z += use ? v[u].z : 0.f;
            acc.w += use ? v[u].w : 0.f;
        }
    }
    if (rin) {
        acc.x += uu[0].x * R0 + uu[0].y * R1;
        acc.y += uu[1].x * R0 + uu[1].y * R1;
        acc.z += uu[2].x * R0 + uu[2].y * R1;
        acc.w += uu[3].x * R0 + uu[3].y * R1;
    }
#pragma unroll
    for (int m = kCombCG; m < MOE_WAVE; m <<= 1) {
        acc.x += __shfl_xor(acc.x, m, MOE_WAVE);
        acc.y += __shfl_xor(acc.y, m, MOE_WAVE);
        acc.z += __shfl_xor(acc.z, m, MOE_WAVE);
        acc.w += __shfl_xor(acc.w, m, MOE_WAVE);
    }
    if (rg == 0 && col < H) *reinterpret_cast<float4*>(y + (size_t)t * H + col) = acc;
}

// ---------------------------------------------------------------------------
// Load time: the sketch.  Grid (ceil(I / 20), nblk, 2 E): workgroup (cg, b,
// 2 e + P) sketches block b of projection P's rows j = 20 cg .. 20 cg + 19 of
// expert e, five rows per wave: each row's block is rotated as in
// rotate_scan_wave (fp64 butterflies), the ternary threshold
// 0.7 * (sum |u|) / 128 and the scale (sum of the kept |u|) / (their number)
// are taken with the sums by pairwise halving (in-lane pair, then lane
// distances 1, 2, ..., 32) -- the order of their definition -- and the codes
// go to LDS; then the 128 coordinate rows get their 4 bytes (20 channels,
// base 3) each.  Rows past I are code 0; bytes past ceil(I / 5) are left as
// they are (zero).
__global__ void __launch_bounds__(kThreads)
reader_sketch_kernel(const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu,
                     const int8_t* __restrict__ signs, int H, int I, int rowb, uint8_t* __restrict__ sketch,
                     float* __restrict__ scale) {
    __shared__ int8_t codes[20][kReaderBlock];
    const int cg = blockIdx.x, b = blockIdx.y;
    const int e = blockIdx.z >> 1, P = blockIdx.z & 1;
    const int nblk = H / kReaderBlock;
    const int tid = threadIdx.x, lane = tid % MOE_WAVE, wave = tid / MOE_WAVE;
    const uint16_t* W = P ? Wu : Wg;
    const int s0 = signs[b * kReaderBlock + 2 * lane], s1 = signs[b * kReaderBlock + 2 * lane + 1];
    for (int rr = 0; rr < 5; ++rr) {
        const int r = wave * 5 + rr;
        const int j = 20 * cg + r;
        if (j >= I) {  // past the channels: code 0 (uniform per wave)
            codes[r][2 * lane] = 0;
            codes[r][2 * lane + 1] = 0;
            continue;
        }
        const uint32_t hv = *reinterpret_cast<const uint32_t*>(W + ((size_t)e * I + j) * H + b * kReaderBlock + 2 * lane);
        double a = (double)bf16_lo(hv) * (double)s0;
        double c = (double)bf16_hi(hv) * (double)s1;
        {
            const double x = a + c, y = a - c;
            a = x;
            c = y;
        }
#pragma unroll
        for (int d = 1; d < MOE_WAVE; d <<= 1) {
            const double pa = __shfl_xor(a, d, MOE_WAVE);
            const double pc = __shfl_xor(c, d, MOE_WAVE);
            if (lane & d) {
                a = pa - a;
                c = pc - c;
            } else {
                a = a + pa;
                c = c + pc;
            }
        }
        const double ma = fabs(a), mc = fabs(c);
        double tot = ma + mc;  // pairwise halving: the lane's pair, then lanes 1, 2, ..., 32 apart
#pragma unroll
        for (int d = 1; d < MOE_WAVE; d <<= 1) tot = tot + __shfl_xor(tot, d, MOE_WAVE);
        const double delta = 0.7 * (tot / 128.0);
        const bool na = ma > delta, nc = mc > delta;
        double snz = (na ? ma : 0.0) + (nc ? mc : 0.0);
#pragma unroll
        for (int d = 1; d < MOE_WAVE; d <<= 1) snz = snz + __shfl_xor(snz, d, MOE_WAVE);
        const int cnt = __popcll(__ballot(na)) + __popcll(__ballot(nc));
        const double sc = cnt > 0 ? snz / (double)cnt : 0.0;
        codes[r][2 * lane] = na ? (a > 0.0 ? 1 : -1) : 0;
        codes[r][2 * lane + 1] = nc ? (c > 0.0 ? 1 : -1) : 0;
        if (lane == 0) scale[(((size_t)e * 2 + P) * nblk + b) * I + j] = (float)(sc / 128.0);
    }
    __syncthreads();
    const int ng = (I + 4) / 5;  // code bytes of a row
    for (int x = tid; x < kReaderBlock * 4; x += kThreads) {
        const int i = x >> 2, by = x & 3;
        const int g = 4 * cg + by;
        if (g >= ng) continue;
        int v = 0, p3 = 1;
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            v += (codes[5 * by + m][i] + 1) * p3;
            p3 *= 3;
        }
        sketch[((((size_t)e * 2 + P) * nblk + b) * kReaderBlock + i) * rowb + g] = (uint8_t)v;
    }
}

// ||d_j|| of every channel: one wave per channel, fp64 sum of squares (fixed
// butterfly), rounded once.
__global__ void __launch_bounds__(kThreads)
down_norms_kernel(int EI, int H, const uint16_t* __restrict__ Wd, float* __restrict__ dn) {
    const int ch = blockIdx.x * kWaves + threadIdx.x / MOE_WAVE;
    const int lane = threadIdx.x % MOE_WAVE;
    if (ch >= EI) return;
    double sd = 0.0;
    for (int col = lane * 8; col < H; col += MOE_WAVE * 8) {
        float c[8];
        unpack8(load16(Wd + (size_t)ch * H + col), c);
#pragma unroll
        for (int x = 0; x < 8; ++x) sd += (double)c[x] * (double)c[x];
    }
    sd = wave_sum_f64(sd);
    if (lane == 0) dn[ch] = (float)sqrt(sd);
}

// ---------------------------------------------------------------------------
// Load time: the recovery basis.  G = sum over all channels of d d^T (fp32,
// [H][H]), tiles of 64 x 64 (upper triangle, mirrored), each thread a 4 x 4
// block, the channels walked in order 16 at a time through LDS.
__global__ void __launch_bounds__(kThreads)
gram_kernel(const uint16_t* __restrict__ Wd, int N, int H, float* __restrict__ G) {
    __shared__ float As[16][64];
    __shared__ float Bs[16][64];
    const int ta = blockIdx.x, tb = blockIdx.y;
    if (ta > tb) return;
    const int tid = threadIdx.x;
    const int ti = tid / 16, tj = tid % 16;  // 16 x 16 threads, 4 x 4 each
    float acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int z = 0; z < 4; ++z) acc[x][z] = 0.f;
    for (int n0 = 0; n0 < N; n0 += 16) {
        // 16 rows x 64 columns of each tile: thread loads 4 + 4 bf16 values
        {
            const int r = tid / 16, cq = (tid % 16) * 4;
            const int nn = min(n0 + r, N - 1);
            const bool in = n0 + r < N;
            const uint2 va = *reinterpret_cast<const uint2*>(Wd + (size_t)nn * H + 64 * ta + cq);
            const uint2 vb = *reinterpret_cast<const uint2*>(Wd + (size_t)nn * H + 64 * tb + cq);
            As[r][cq] = in ? bf16_lo(va.x) : 0.f; As[r][cq + 1] = in ? bf16_hi(va.x) : 0.f;
            As[r][cq + 2] = in ? bf16_lo(va.y) : 0.f; As[r][cq + 3] = in ? bf16_hi(va.y) : 0.f;
            Bs[r][cq] = in ? bf16_lo(vb.x) : 0.f; Bs[r][cq + 1] = in ? bf16_hi(vb.x) : 0.f;
            Bs[r][cq + 2] = in ? bf16_lo(vb.y) : 0.f; Bs[r][cq + 3] = in ? bf16_hi(vb.y) : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int r = 0; r < 16; ++r) {
            const float4 av = *reinterpret_cast<const float4*>(&As[r][4 * ti]);
            const float4 bv = *reinterpret_cast<const float4*>(&Bs[r][4 * tj]);
            const float a4[4] = {av.x, av.y, av.z, av.w};
            const float b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[x][z] = fmaf(a4[x], b4[z], acc[x][z]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            const int i = 64 * ta + 4 * ti + x, jj = 64 * tb + 4 * tj + z;
            G[(size_t)i * H + jj] = acc[x][z];
            G[(size_t)jj * H + i] = acc[x][z];
        }
}

// Z = A Q, A fp32 [H][H], Q [H][rank] (rank <= 32): one thread per (row,
// column), the row of A walked in order.
__global__ void __launch_bounds__(kThreads)
gemm_aq_kernel(const float* __restrict__ A, const float* __restrict__ Q, int H, int rank, float* __restrict__ Z) {
    const int idx = blockIdx.x * kThreads + threadIdx.x;
    if (idx >= H * rank) return;
    const int i = idx / rank, r = idx - i * rank;
    float acc = 0.f;
    for (int a = 0; a < H; ++a) acc = fmaf(A[(size_t)i * H + a], Q[(size_t)a * rank + r], acc);
    Z[idx] = acc;
}

// S = X^T Y (rank x rank, fp64), X and Y [H][rank]: one workgroup, thread
// (r, c) of the first rank^2 threads walks the rows in order.
__global__ void __launch_bounds__(1024)
xty_kernel(const float* __restrict__ X, const float* __restrict__ Y, int H, int rank, double* __restrict__ S) {
    const int tid = threadIdx.x;
    if (tid >= rank * rank) return;
    const int r = tid / rank, c = tid - r * rank;
    double acc = 0.0;
    for (int i = 0; i < H; ++i) acc += (double)X[(size_t)i * rank + r] * (double)Y[(size_t)i * rank + c];
    S[tid] = acc;
}

// Orthonormalise the columns of Z by Cholesky QR: S = Z^T Z = L L^T, Q =
// Z L^{-T}.  One workgroup; the factorisation by thread 0 (rank <= 32), the
// rows of Q by all threads.
__global__ void __launch_bounds__(1024)
cholqr_kernel(const float* __restrict__ Z, const double* __restrict__ S, int H, int rank, float* __restrict__ Q) {
    __shared__ double L[kMaxRank][kMaxRank];
    __shared__ double Li[kMaxRank][kMaxRank];  // L^{-1}
    const int tid = threadIdx.x;
    if (tid == 0) {
        for (int c = 0; c < rank; ++c) {
            for (int r = 0; r < rank; ++r) L[r][c] = 0.0;
        }
        for (int c = 0; c < rank; ++c) {
            double d = S[c * rank + c];
            for (int m = 0; m < c; ++m) d -= L[c][m] * L[c][m];
            d = d > 0.0 ? sqrt(d) : 1e-300;
            L[c][c] = d;
            for (int r = c + 1; r < rank; ++r) {
                double v = S[r * rank + c];
                for (int m = 0; m < c; ++m) v -= L[r][m] * L[c][m];
                L[r][c] = v / d;
            }
        }
        for (int c = 0; c < rank; ++c) {  // forward substitution, column by column
            for (int r = 0; r < rank; ++r) {
                double v = (r == c) ? 1.0 : 0.0;
                for (int m = 0; m < r; ++m) v -= L[r][m] * Li[m][c];
                Li[r][c] = r < c ? 0.0 : v / L[r][r];
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < H; i += 1024) {
        double z[kMaxRank];
        for (int m = 0; m < rank; ++m) z[m] = Z[(size_t)i * rank + m];
        for (int c = 0; c < rank; ++c) {  // (Z L^{-T})[i][c] = sum_m z[m] Li[c][m]
            double v = 0.0;
            for (int m = 0; m <= c; ++m) v += z[m] * Li[c][m];
            Q[(size_t)i * rank + c] = (float)v;
        }
    }
}

// Rayleigh-Ritz: B = Q^T G Q (symmetric, rank x rank) -> eigenvectors V by
// cyclic Jacobi rotations (fp64, one thread), U = Q V with the columns in
// decreasing eigenvalue order and each column's entry of largest magnitude
// made positive.
__global__ void __launch_bounds__(1024)
ritz_kernel(const float* __restrict__ Q, const double* __restrict__ B, int H, int rank, float* __restrict__ U) {
    __shared__ double A[kMaxRank][kMaxRank];
    __shared__ double V[kMaxRank][kMaxRank];
    __shared__ int ord[kMaxRank];
    __shared__ float cmax[kMaxRank];
    __shared__ int csgn[kMaxRank];
    const int tid = threadIdx.x;
    if (tid == 0) {
        for (int r = 0; r < rank; ++r)
            for (int c = 0; c < rank; ++c) {
                A[r][c] = 0.5 * (B[r * rank + c] + B[c * rank + r]);
                V[r][c] = r == c ? 1.0 : 0.0;
            }
        for (int sweep = 0; sweep < 60; ++sweep) {
            double off = 0.0;
            for (int p = 0; p < rank; ++p)
                for (int q = p + 1; q < rank; ++q) off += A[p][q] * A[p][q];
            if (off < 1e-30) break;
            for (int p = 0; p < rank; ++p)
                for (int q = p + 1; q < rank; ++q) {
                    if (A[p][q] == 0.0) continue;
                    const double th = (A[q][q] - A[p][p]) / (2.0 * A[p][q]);
                    const double tt = (th >= 0 ? 1.0 : -1.0) / (fabs(th) + sqrt(th * th + 1.0));
                    const double cs = 1.0 / sqrt(tt * tt + 1.0), sn = tt * cs;
                    for (int m = 0; m < rank; ++m) {  // A <- J^T A J
                        const double amp = A[m][p], amq = A[m][q];
                        A[m][p] = cs * amp - sn * amq;
                        A[m][q] = sn * amp + cs * amq;
                    }
                    for (int m = 0; m < rank; ++m) {
                        const double apm = A[p][m], aqm = A[q][m];
                        A[p][m] = cs * apm - sn * aqm;
                        A[q][m] = sn * apm + cs * aqm;
                    }
                    for (int m = 0; m < rank; ++m) {
                        const double vmp = V[m][p], vmq = V[m][q];
                        V[m][p] = cs * vmp - sn * vmq;
                        V[m][q] = sn * vmp + cs * vmq;
                    }
                }
        }
        for (int r = 0; r < rank; ++r) ord[r] = r;  // decreasing eigenvalue (stable)
        for (int r = 1; r < rank; ++r)
            for (int x = r; x > 0 && A[ord[x]][ord[x]] > A[ord[x - 1]][ord[x - 1]]; --x) {
                const int tmp = ord[x];
                ord[x] = ord[x - 1];
                ord[x - 1] = tmp;
            }
        for (int c = 0; c < rank; ++c) {
            cmax[c] = -1.f;
            csgn[c] = 1;
        }
    }
    __syncthreads();
    // U = Q V[:, ord]; the sign of each column from its largest-magnitude entry
    // (first such row in row order)
    if (tid < rank) {
        const int c = tid, vc = ord[c];
        float best = -1.f;
        int sg = 1;
        for (int i = 0; i < H; ++i) {
            double v = 0.0;
            for (int m = 0; m < rank; ++m) v += (double)Q[(size_t)i * rank + m] * V[m][vc];
            const float fv = (float)v;
            if (fabsf(fv) > best) {
                best = fabsf(fv);
                sg = fv < 0.f ? -1 : 1;
            }
        }
        csgn[c] = sg;
    }
    __syncthreads();
    for (int i = tid; i < H; i += 1024) {
        for (int c = 0; c < rank; ++c) {
            const int vc = ord[c];
            double v = 0.0;
            for (int m = 0; m < rank; ++m) v += (double)Q[(size_t)i * rank + m] * V[m][vc];
            U[(size_t)i * rank + c] = (float)(csgn[c] * v);
        }
    }
}

// Deterministic start of the subspace iteration: a hash of (row, column)
// mapped to [-1, 1).
__global__ void __launch_bounds__(kThreads) init_q_kernel(int H, int rank, float* __restrict__ Q) {
    const int idx = blockIdx.x * kThreads + threadIdx.x;
    if (idx >= H * rank) return;
    uint32_t x = (uint32_t)idx * 0x9E3779B9u + 0x7F4A7C15u;
    x ^= x >> 16;
    x *= 0x85EBCA6Bu;
    x ^= x >> 13;
    x *= 0xC2B2AE35u;
    x ^= x >> 16;
    Q[idx] = (float)((double)x / 2147483648.0 - 1.0);
}

// b_j = U^T d_j for every channel, rounded to bf16: thread (channel, r)
// walks the column in order in fp32.
__global__ void __launch_bounds__(kThreads)
recovery_coefs_kernel(const float* __restrict__ U, const uint16_t* __restrict__ Wd, int EI, int H, int rank,
                      uint16_t* __restrict__ b) {
    const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (size_t)EI * rank) return;
    const size_t ch = idx / rank;
    const int r = (int)(idx - ch * rank);
    float acc = 0.f;
    for (int i = 0; i < H; i += 8) {
        float f[8];
        unpack8(load16(Wd + ch * H + i), f);
#pragma unroll
        for (int x = 0; x < 8; ++x) acc = fmaf(f[x], U[(size_t)(i + x) * rank + r], acc);
    }
    const uint32_t u = __float_as_uint(acc);
    b[idx] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace

// ---------------------------------------------------------------------------

int reader_row_bytes(int I) { return ((I + 4) / 5 + 15) / 16 * 16; }

hipError_t launch_reader_rotate(const float* h, int M, int H, const int8_t* signs, uint8_t* xsel, float* xval,
                                hipStream_t stream) {
    if (H % kReaderBlock || M < 1) return hipErrorInvalidValue;
    const int jobs = M * (H / kReaderBlock);
    MOE_LAUNCH(reader_rotate_kernel, dim3((jobs + kWaves - 1) / kWaves), dim3(kThreads), 0, stream, h, M, H, signs,
               xsel, xval);
    return hipGetLastError();
}

int reader_groups(int nblk, int* bpw) {
    const int b = (nblk + kMaxGroups - 1) / kMaxGroups;
    if (bpw) *bpw = b;
    return (nblk + b - 1) / b;
}

hipError_t launch_reader_screen(const ReaderArgs& ra, const SelRoute* route, const int32_t* topk_ids, int M,
                                hipStream_t stream) {
    int bpw = 0;
    const int nbq = ra.nblk >= 1 ? reader_groups(ra.nblk, &bpw) : 0;
    if (ra.nblk < 1 || ra.nblk > kRowGroups || ra.k < 1 || ra.k > 32 || ra.rowb != reader_row_bytes(ra.I) || M < 1 ||
        ra.nbq != nbq || ra.bpw != bpw || bpw > kMaxBpw)
        return hipErrorInvalidValue;
    const int nseg = ra.rowb / 16;
    const dim3 grid((2 * ra.k + 7) / 8 * 8 * nseg * nbq, M);
    if (route) {
        if (ra.E > kThreads || route->M != M) return hipErrorInvalidValue;
        MOE_LAUNCH(reader_screen_kernel<true>, grid, dim3(kThreads), 0, stream, ra, *route, nullptr, nseg);
    } else {
        MOE_LAUNCH(reader_screen_kernel<false>, grid, dim3(kThreads), 0, stream, ra, SelRoute{}, topk_ids, nseg);
    }
    return hipGetLastError();
}

hipError_t launch_reader_select(const ReaderArgs& ra, const int32_t* topk_ids, const float* topk_w, int M, int K,
                                int32_t* slot_cnt, int32_t* slot_kept, int32_t* kept_out, float* est_out,
                                float* score_out, hipStream_t stream) {
    if (ra.k * ra.I > kSelThreads * kSelPer || ra.k > 32 || ra.E > 8192 || ra.I > 16384 || ra.nbq < 1 ||
        ra.nbq > kMaxGroups || K < 1)
        return hipErrorInvalidValue;
    MOE_LAUNCH(reader_select_kernel, dim3(M), dim3(kSelThreads), 0, stream, ra, topk_ids, topk_w, K,
               FastDiv((uint32_t)ra.I), slot_cnt, slot_kept, kept_out, est_out, score_out);
    return hipGetLastError();
}

int reader_recover_chunks(int I) { return (I + kThreads - 1) / kThreads; }

hipError_t launch_reader_recover(const ReaderArgs& ra, const int32_t* topk_ids, const float* topk_w, int M,
                                 hipStream_t stream) {
    if (ra.rank < 1 || ra.rank > kMaxRank || ra.rank % 8) return hipErrorInvalidValue;
    MOE_LAUNCH(reader_recover_kernel, dim3(reader_recover_chunks(ra.I), ra.k, M), dim3(kThreads), 0, stream, ra,
               topk_ids, topk_w);
    return hipGetLastError();
}

hipError_t launch_reader_combine(int M, int H, int nchunks, const float* part, const float* rpart, int nrp, int rank,
                                 const float* U, float* y, hipStream_t stream) {
    const dim3 grid((H / 4 + kCombCG - 1) / kCombCG, M);
    MOE_LAUNCH(reader_combine_kernel, grid, dim3(MOE_WAVE), 0, stream, H, nchunks, part, rpart, nrp, rank, U, y);
    return hipGetLastError();
}

hipError_t launch_reader_sketch(int E, int I, int H, const uint16_t* Wg, const uint16_t* Wu, const int8_t* signs,
                                uint8_t* sketch, float* scale, hipStream_t stream) {
    if (H % kReaderBlock) return hipErrorInvalidValue;
    const dim3 grid((I + 19) / 20, H / kReaderBlock, 2 * E);
    hipLaunchKernelGGL(reader_sketch_kernel, grid, dim3(kThreads), 0, stream, Wg, Wu, signs, H, I, reader_row_bytes(I),
                       sketch, scale);
    return hipGetLastError();
}

hipError_t launch_down_norms(int E, int I, int H, const uint16_t* Wd, float* dn, hipStream_t stream) {
    const int EI = E * I;
    hipLaunchKernelGGL(down_norms_kernel, dim3((EI + kWaves - 1) / kWaves), dim3(kThreads), 0, stream, EI, H, Wd, dn);
    return hipGetLastError();
}

// Workspace of launch_recovery_basis: G [H][H] fp32, Q, Z [H][rank] fp32, S [rank][rank] fp64.
size_t recovery_basis_scratch(int H, int rank) {
    return (size_t)H * H * 4 + 2 * (size_t)H * rank * 4 + (size_t)rank * rank * 8 + 1024;
}

hipError_t launch_recovery_basis(int E, int I, int H, const uint16_t* Wd, int rank, int iters, float* U, void* scratch,
                                 hipStream_t stream) {
    if (rank < 1 || rank > kMaxRank || H % 64 || iters < 1) return hipErrorInvalidValue;
    char* p = static_cast<char*>(scratch);
    float* G = reinterpret_cast<float*>(p);
    float* Q = reinterpret_cast<float*>(p + (size_t)H * H * 4);
    float* Z = Q + (size_t)H * rank;
    double* S = reinterpret_cast<double*>(reinterpret_cast<char*>(Z + (size_t)H * rank) + 256 -
                                          (reinterpret_cast<uintptr_t>(Z + (size_t)H * rank) % 256));
    const int nt = H / 64;
    hipLaunchKernelGGL(gram_kernel, dim3(nt, nt), dim3(kThreads), 0, stream, Wd, E * I, H, G);
    const int gq = (H * rank + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(init_q_kernel, dim3(gq), dim3(kThreads), 0, stream, H, rank, Q);
    for (int it = 0; it < iters; ++it) {
        hipLaunchKernelGGL(gemm_aq_kernel, dim3(gq), dim3(kThreads), 0, stream, G, Q, H, rank, Z);
        hipLaunchKernelGGL(xty_kernel, dim3(1), dim3(1024), 0, stream, Z, Z, H, rank, S);
        hipLaunchKernelGGL(cholqr_kernel, dim3(1), dim3(1024), 0, stream, Z, S, H, rank, Q);
    }
    hipLaunchKernelGGL(gemm_aq_kernel, dim3(gq), dim3(kThreads), 0, stream, G, Q, H, rank, Z);
    hipLaunchKernelGGL(xty_kernel, dim3(1), dim3(1024), 0, stream, Q, Z, H, rank, S);
    hipLaunchKernelGGL(ritz_kernel, dim3(1), dim3(1024), 0, stream, Q, S, H, rank, U);
    return hipGetLastError();
}

hipError_t launch_recovery_coefs(int E, int I, int H, const float* U, int rank, const uint16_t* Wd, uint16_t* b,
                                 hipStream_t stream) {
    const size_t n = (size_t)E * I * rank;
    hipLaunchKernelGGL(recovery_coefs_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, U, Wd, E * I, H, rank, b);
    return hipGetLastError();
}

}  // namespace moe

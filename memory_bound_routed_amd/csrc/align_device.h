// Canonical alignment of routes into padded expert blocks (page "Route-Block
// Membership Selects Packed-AWQ Arithmetic", Sec. 2.1 alignment and padded
// blocks, Sec. 3.1 Eq. 1 route-block membership, Sec. 5.3 stable (expert id,
// route id) order).
//
// The placement of a route is computed, not raced for:
//   pos(r) = b * blocks_before(e) + (# routes of e before r),
// with e = id(r) and blocks_before(e) = sum over the experts e' < e of
// ceil(n(e') / b).  Inside a wave the counts come from ballots of the id bits
// (ids < 1024, so ten ballots): a lane's id is matched against every lane at
// once, which gives the lanes of the same expert (their count, and the rank
// of the lane among them by mbcnt) and the lanes of a lower expert.  No LDS
// round trips and no atomics are on this path, so the output is a pure
// function of the ids and the phase costs a few hundred instructions.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kAlignThreads = 256;
constexpr int kIdBits = 10;  // expert ids < 1024

// LDS bytes align_workgroup needs for R routes and E experts: ids and ranks
// of the routes, the per-chunk counts, the blocks below each expert and the
// wave totals of the expert scan.
__host__ __device__ inline size_t align_lds_bytes_inline(int R, int E) {
    const int nchunk = (R + MOE_WAVE - 1) / MOE_WAVE;
    return sizeof(int) * ((size_t)2 * R + (size_t)(nchunk + 1) * E + kAlignThreads / MOE_WAVE);
}

// Lanes of the wave holding a valid id (V) with the same id as this lane
// (eq), and with a lower id (lt).  bs[j] = lanes whose id has bit j set.
// From the top bit down, a lane is lower once it agrees on the bits above
// and has 0 where this lane's id has 1.
__device__ __forceinline__ void id_match(int id, uint64_t V, const uint64_t (&bs)[kIdBits], uint64_t& eq,
                                         uint64_t& lt) {
    eq = V;
    lt = 0;
#pragma unroll
    for (int j = kIdBits - 1; j >= 0; --j) {
        const bool one = (id >> j) & 1;
        lt |= one ? (eq & ~bs[j]) : 0ull;
        eq &= one ? bs[j] : ~bs[j];
    }
}

__device__ __forceinline__ void id_ballots(int id, bool ok, uint64_t (&bs)[kIdBits]) {
#pragma unroll
    for (int j = 0; j < kIdBits; ++j) bs[j] = __ballot(ok && ((id >> j) & 1));
}

// Inclusive prefix sum over the lanes of a wave: row_shr by 1, 2, 4 and 8
// inside each row of 16 lanes (lanes shifted in from outside the row add
// 0), then the totals of the lower rows.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
    const int row = (threadIdx.x % MOE_WAVE) >> 4;
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47);
    return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Alignment of R <= 64 routes by one wave (lane r holds route r), in
// registers only.  Each expert's first route (rank 0) holds its block count
// nblk <= 64; F[k] = the first routes whose nblk has bit k set, so
//   blocks_before(e) = sum_k 2^k * popcount(lt & F[k])
// and the total is sum_k 2^k * popcount(F[k]).  Each first route writes its
// expert's padding rows and blocks.  id_of(r) returns route r's id; every
// lane of the calling wave must call.
template <typename IdOf>
__device__ inline void align_wave(IdOf id_of, int R, int E, FastDiv fb, int32_t* __restrict__ sorted_routes,
                                  int32_t* __restrict__ block_expert, int32_t* __restrict__ counts,
                                  int32_t* __restrict__ err) {
    const int lane = threadIdx.x % MOE_WAVE;
    const int raw = lane < R ? id_of(lane) : 0;
    const bool ok = lane < R && raw >= 0 && raw < E;
    const int id = ok ? raw : 0;
    if (__ballot(lane < R && !ok) != 0 && lane == 0) atomicOr(err, DEVERR_BAD_ROUTE_ID);
    const uint64_t V = __ballot(ok);
    uint64_t bs[kIdBits];
    id_ballots(id, ok, bs);
    uint64_t eq, lt;
    id_match(id, V, bs, eq, lt);
    const int cnt = __popcll(eq);
    const int rank = mbcnt64(eq);
    const bool first = ok && rank == 0;
    const int b = (int)fb.d;
    const int nblk = first ? (int)fb.div(cnt + b - 1) : 0;
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 7; ++q) {  // nblk <= 64
        const uint64_t F = __ballot(first && ((nblk >> q) & 1));
        before += __popcll(lt & F) << q;
        total += __popcll(F) << q;
    }
    const int off = before * b;
    if (ok) sorted_routes[off + rank] = lane;
    if (first) {
        for (int q = cnt; q < nblk * b; ++q) sorted_routes[off + q] = R;
        for (int j = 0; j < nblk; ++j) block_expert[before + j] = id;
    }
    if (lane == 0) {
        counts[0] = total;
        counts[1] = total * b;
    }
}

// The same alignment for any R by all 256 threads of one workgroup; smem
// holds align_lds_bytes(R, E) bytes.  Chunk c (routes 64c ..) goes to wave
// c % 4: the ballots give each route its rank inside the chunk, and the
// expert's first route in the chunk stores the chunk's count n_c(e).  Then
// thread t owns experts t*EPT .. (EPT = ceil(E / 256)): it turns n_c(e) into
// the count of e in earlier chunks, forms nblk(e), and an exclusive scan of
// nblk over the threads (expert order) gives blocks_before(e); the owner
// writes e's padding rows and blocks.  Last, every route is placed at
// b * blocks_before(e) + (earlier chunks' count) + rank.  id_of(r) returns
// route r's id.
template <typename IdOf>
__device__ inline void align_workgroup(IdOf id_of, int R, int E, FastDiv fb, int32_t* __restrict__ sorted_routes,
                                       int32_t* __restrict__ block_expert, int32_t* __restrict__ counts,
                                       int32_t* __restrict__ err, int* smem) {
    constexpr int kWavesA = kAlignThreads / MOE_WAVE;
    const int nchunk = (R + MOE_WAVE - 1) / MOE_WAVE;
    int* sid = smem;               // [R]  expert of each route, -1 if invalid
    int* srank = sid + R;          // [R]  rank inside its chunk among same-expert routes
    int* cnt = srank + R;          // [nchunk][E]  n_c(e), then the count of e in chunks < c
    int* bbefore = cnt + nchunk * E;  // [E]  blocks of the experts below e
    int* wtot = bbefore + E;          // [kWavesA]  wave totals of the block-count scan
    __shared__ int bad;
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int b = (int)fb.d;

    for (int i = tid; i < nchunk * E; i += kAlignThreads) cnt[i] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int c = wave; c < nchunk; c += kWavesA) {
        const int r = c * MOE_WAVE + lane;
        const int raw = r < R ? id_of(r) : 0;
        const bool ok = r < R && raw >= 0 && raw < E;
        const int id = ok ? raw : 0;
        if (r < R && !ok) bad = 1;
        const uint64_t V = __ballot(ok);
        uint64_t bs[kIdBits];
        id_ballots(id, ok, bs);
        uint64_t eq, lt;
        id_match(id, V, bs, eq, lt);
        const int rank = mbcnt64(eq);
        if (r < R) {
            sid[r] = ok ? id : -1;
            srank[r] = rank;
        }
        if (ok && rank == 0) cnt[c * E + id] = __popcll(eq);
    }
    __syncthreads();
    if (tid == 0 && bad) atomicOr(err, DEVERR_BAD_ROUTE_ID);

    const int EPT = (E + kAlignThreads - 1) / kAlignThreads;  // <= 4
    int tot[4], nblk[4];
    int tsum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = tid * EPT + u;
        tot[u] = 0;
        if (u < EPT && e < E) {
            int run = 0;
            for (int c = 0; c < nchunk; ++c) {
                const int x = cnt[c * E + e];
                cnt[c * E + e] = run;
                run += x;
            }
            tot[u] = run;
        }
        nblk[u] = (int)fb.div(tot[u] + b - 1);
        tsum += nblk[u];
    }
    const int incl = wave_incl_scan(tsum);
    if (lane == MOE_WAVE - 1) wtot[wave] = incl;
    __syncthreads();
    int before = incl - tsum, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesA; ++w) {
        const int x = wtot[w];
        before += w < wave ? x : 0;
        total += x;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = tid * EPT + u;
        if (u < EPT && e < E) {
            bbefore[e] = before;
            const int off = before * b;
            for (int q = tot[u]; q < nblk[u] * b; ++q) sorted_routes[off + q] = R;
            for (int j = 0; j < nblk[u]; ++j) block_expert[before + j] = e;
        }
        before += nblk[u];
    }
    __syncthreads();
    for (int r = tid; r < R; r += kAlignThreads) {
        const int id = sid[r];
        if (id >= 0) sorted_routes[bbefore[id] * b + cnt[(r / MOE_WAVE) * E + id] + srank[r]] = r;
    }
    if (tid == 0) {
        counts[0] = total;
        counts[1] = total * b;
    }
}

}  // namespace moe

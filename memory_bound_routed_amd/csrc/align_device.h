// Canonical alignment of routes into padded expert blocks, run by one
// workgroup of 256 threads (page "Route-Block Membership Selects Packed-AWQ
// Arithmetic", Sec. 2.1 alignment and padded blocks, Sec. 3.1 Eq. 1
// route-block membership, Sec. 5.3 stable (expert id, route id) order).
//
// The placement of a route is computed, not raced for:
//   pos(r) = off[e] + (# routes of e in earlier 64-route chunks)
//                   + (# lanes below r in r's chunk with the same expert),
// with e = id(r) and off[] the exclusive prefix of the padded counts.  The
// per-chunk counts use LDS integer atomics, whose result does not depend on
// their order, so the output is a pure function of the ids.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kAlignThreads = 256;

// LDS bytes align_workgroup needs for R routes and E experts.
__host__ __device__ inline size_t align_lds_bytes_inline(int R, int E) {
    const int nchunk = (R + MOE_WAVE - 1) / MOE_WAVE;
    const size_t wg = sizeof(int) * ((size_t)2 * R + (size_t)nchunk * E + 2 * (size_t)E + 1);
    return wg > sizeof(int) * 2 * MOE_WAVE ? wg : sizeof(int) * 2 * MOE_WAVE;
}

// Run by all 256 threads of one workgroup; smem holds align_lds_bytes(R, E) bytes.
// id_of(r) returns route r's id.
template <typename IdOf>
__device__ inline void align_workgroup(IdOf id_of, int R, int E, int b,
                                int32_t* __restrict__ sorted_routes, int32_t* __restrict__ block_expert,
                                int32_t* __restrict__ counts, int32_t* __restrict__ err, int* smem) {
    const int nchunk = (R + MOE_WAVE - 1) / MOE_WAVE;
    int* sid = smem;                 // [R]  expert of each route, -1 if invalid
    int* srank = sid + R;            // [R]  rank inside its chunk among same-expert routes
    int* cnt = srank + R;            // [nchunk][E]  counts, then exclusive prefix over chunks
    int* tot = cnt + nchunk * E;     // [E]
    int* off = tot + E;              // [E + 1]
    __shared__ int bad;
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;

    for (int i = tid; i < nchunk * E; i += kAlignThreads) cnt[i] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int r = tid; r < R; r += kAlignThreads) {
        const int id = id_of(r);
        const bool ok = id >= 0 && id < E;
        sid[r] = ok ? id : -1;
        if (!ok) bad = 1;
    }
    __syncthreads();
    if (tid == 0 && bad) atomicOr(err, DEVERR_BAD_ROUTE_ID);

    for (int c = wave; c < nchunk; c += kAlignThreads / MOE_WAVE) {
        const int r = c * MOE_WAVE + lane;
        const int id = r < R ? sid[r] : -1;
        int rank = 0;
        const int nl = min(MOE_WAVE, R - c * MOE_WAVE);  // routes in this chunk (uniform)
        for (int l2 = 0; l2 < nl; ++l2) {
            const int o = __builtin_amdgcn_readlane(id, l2);
            rank += (l2 < lane && o == id) ? 1 : 0;
        }
        if (r < R) srank[r] = rank;
        if (id >= 0) atomicAdd(&cnt[c * E + id], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads) {
        int run = 0;
        for (int c = 0; c < nchunk; ++c) {
            const int x = cnt[c * E + e];
            cnt[c * E + e] = run;
            run += x;
        }
        tot[e] = run;
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the padded counts, 64 experts at a time
        int carry = 0;
        for (int e0 = 0; e0 < E; e0 += MOE_WAVE) {
            const int e = e0 + lane;
            const int pc = e < E ? ((tot[e] + b - 1) / b) * b : 0;
            int x = pc;
#pragma unroll
            for (int d = 1; d < MOE_WAVE; d <<= 1) {
                const int y = __shfl_up(x, d, MOE_WAVE);
                if (lane >= d) x += y;
            }
            if (e < E) off[e] = carry + x - pc;
            carry += __shfl(x, MOE_WAVE - 1, MOE_WAVE);
        }
        if (lane == 0) off[E] = carry;
    }
    __syncthreads();
    for (int r = tid; r < R; r += kAlignThreads) {
        const int id = sid[r];
        if (id >= 0) sorted_routes[off[id] + cnt[(r / MOE_WAVE) * E + id] + srank[r]] = r;
    }
    for (int e = tid; e < E; e += kAlignThreads) {
        const int o = off[e];
        const int padded = off[e + 1] - o;
        for (int q = tot[e]; q < padded; ++q) sorted_routes[o + q] = R;
        for (int j = 0; j < padded / b; ++j) block_expert[o / b + j] = e;
    }
    if (tid == 0) {
        counts[0] = off[E] / b;
        counts[1] = off[E];
    }
}

// The same alignment for R <= 64 routes by one wave: lane r holds route r.
// With id the lane's expert (-1 if invalid),
//   cnt(r)  = # routes with the same expert,   rank(r) = # of them below r,
//   first   = the lowest route of its expert (rank 0),
//   off(e)  = sum of the padded counts ceil(cnt/b)*b of the experts below e
//             (summed over the first routes of those experts),
// route r goes to off(e) + rank(r); each expert's first route writes its
// padding rows and its blocks.  The output equals align_workgroup's: the same
// (expert id, route id) order, the same padding, the same counts.  The sums
// over routes read the ids and padded counts from the wave's own LDS scratch
// (2 * 64 ints; a wave's LDS accesses execute in order), four routes per
// read.  id_of(r) returns route r's id; every lane of the calling wave must
// call.
template <typename IdOf>
__device__ inline void align_wave(IdOf id_of, int R, int E, FastDiv fb, int32_t* __restrict__ sorted_routes,
                                  int32_t* __restrict__ block_expert, int32_t* __restrict__ counts,
                                  int32_t* __restrict__ err, int* scratch) {
    const int lane = threadIdx.x % MOE_WAVE;
    const int raw = lane < R ? id_of(lane) : 0;
    const bool ok = lane < R && raw >= 0 && raw < E;
    const int id = ok ? raw : -1;
    if (__ballot(lane < R && !ok) != 0 && lane == 0) atomicOr(err, DEVERR_BAD_ROUTE_ID);
    int* sid = scratch;               // [64] expert of each route; -2 past R (equal to no id)
    int* spad = scratch + MOE_WAVE;   // [64] padded count on an expert's first route, else 0
    sid[lane] = lane < R ? id : -2;
    __builtin_amdgcn_wave_barrier();
    const int nq = (R + 3) / 4;       // groups of four routes (uniform)
    const int4* sid4 = reinterpret_cast<const int4*>(sid);
    int cnt = 0, rank = 0;
    for (int q0 = 0; q0 < nq; q0 += 8) {
        int4 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = sid4[min(q0 + u, MOE_WAVE / 4 - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (q0 + u >= nq) break;  // uniform
            const int r2 = 4 * (q0 + u);
            cnt += (o[u].x == id) + (o[u].y == id) + (o[u].z == id) + (o[u].w == id);
            rank += (o[u].x == id && r2 < lane) + (o[u].y == id && r2 + 1 < lane) + (o[u].z == id && r2 + 2 < lane) +
                    (o[u].w == id && r2 + 3 < lane);
        }
    }
    const int b = (int)fb.d;
    const int padded = fb.div(cnt + b - 1) * b;
    const int first_pad = (ok && rank == 0) ? padded : 0;  // padded count, on the expert's first route only
    spad[lane] = first_pad;
    __builtin_amdgcn_wave_barrier();
    const int4* spad4 = reinterpret_cast<const int4*>(spad);
    int off = 0, total = 0;
    for (int q0 = 0; q0 < nq; q0 += 8) {
        int4 o[8], p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            o[u] = sid4[min(q0 + u, MOE_WAVE / 4 - 1)];
            p[u] = spad4[min(q0 + u, MOE_WAVE / 4 - 1)];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (q0 + u >= nq) break;  // uniform
            off += (o[u].x < id ? p[u].x : 0) + (o[u].y < id ? p[u].y : 0) + (o[u].z < id ? p[u].z : 0) +
                   (o[u].w < id ? p[u].w : 0);
            total += (p[u].x + p[u].y) + (p[u].z + p[u].w);
        }
    }
    if (ok) sorted_routes[off + rank] = lane;
    if (first_pad) {
        for (int q = cnt; q < padded; ++q) sorted_routes[off + q] = R;
        const int b0 = fb.div(off);
        for (int j = 0, nbk = fb.div(padded); j < nbk; ++j) block_expert[b0 + j] = id;
    }
    if (lane == 0) {
        counts[0] = fb.div(total);
        counts[1] = total;
    }
}

}  // namespace moe

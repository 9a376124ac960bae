// Dense bf16 experts: gate/up GEMV with SiLU(gate)*up kept in registers, the
// down GEMV and the fixed-order weighted combine (page "A Multi-Engine
// Dataflow for MoE Decoding on Scratchpad-Based Tensor Accelerators",
// MoE-block background and Sec. 4.3; page "Channel Selection for
// Mixture-of-Experts Decoding Needs No Calibration Data", Background: the
// channel view of the same computation).
//
// Work is expert-major: the workgroups of the alignment block that starts an
// expert's run of blocks walk every block of that run, so each routed
// expert's weights are streamed from HBM once per step whatever its number of
// routes.  Weights a workgroup needs are requested before anything else and
// kept in registers for every route that uses them.
//
// The arithmetic of one route never depends on its position in the plan or
// on the grid: per lane the hidden dimension is walked in ascending order,
// lanes are added by a fixed butterfly, channel chunks have a size fixed by
// the shape, and every result is stored by route id.  The combine adds the
// partials of a token in a fixed order, so y is bitwise reproducible.
//
// Two schedules:
//  * fused (one route per block row, the batch-1 case): a workgroup owns a
//    chunk of CH channels of one expert.  It issues the loads of the CH gate
//    rows, CH up rows and CH down rows at once, so the down weights stream
//    while gate/up is still being reduced (the GPU form of issuing the down
//    transfers during gate/up compute), then writes a down partial
//    part[route][chunk][:] = sum_{j in chunk} (a_route * p_j) * d_j.
//  * split (several routes per block): the gate/up kernel writes p, then a
//    down kernel over column blocks writes one full-length partial per route
//    (256-column blocks on the matrix cores, 128-column blocks on the vector
//    ALUs).
// Both feed combine_kernel: y[t] = sum over the token's routes and chunks.
#include <type_traits>

#include "align_device.h"
#include "device_common.h"
#include "launch.h"
#include "topk_device.h"

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

// ---------------------------------------------------------------------------
// Fused schedule.  Grid (plan blocks, ceil(I / (NCH*CH))).  A workgroup owns
// NCH consecutive chunks of CH = NW*CPW channels of one expert and walks
// them with the weights of chunk i+1 requested before chunk i is computed
// (double buffering in registers), so its arithmetic overlaps the stream
// instead of piling up after it.  Per chunk, wave w computes gate/up of
// CPW channels (lane l covers hidden columns 8*(l + 64*q)) from h held in
// LDS; thread t multiplies its row group's down rows at hidden columns
// 8*(t%256 + 256*cq) and accumulates across the chunks; the row groups are
// added in group order at the end and the workgroup writes one partial
//     part[route][range][:] = sum_{j in range} (a_route * p_j) * d_j.
// The weight addresses depend only on the block's expert, so the first two
// chunks are requested right after the plan rows arrive; the route checks,
// affinities and h (whose addresses depend on the same rows) are issued just
// before them, since a load queued behind the stream would wait for it.
//
// ROUTE (one token, the decode step): there is no plan to read.  Each
// workgroup adds the router's slice partials itself, takes the top-k by rank
// counting and the renormalised softmax -- the same arithmetic as the router
// kernel, so the same ids and affinities bit for bit -- and finds its block's
// expert in the canonical plan of the token (one block per selected expert,
// in ascending expert order).  Workgroup (0, 0) writes the ids, affinities,
// logits and plan.  This replaces the router's last-workgroup hand-off (a
// store, a ticket and a reload across the device) by 4 KiB of redundant
// loads per workgroup.
constexpr int kRouteSlices = 16;  // router row slices a routing workgroup adds
constexpr int kRouteMaxE = 512;   // experts (one per thread of the workgroup)

template <int Q, int CQ, int NW, int CPW, int NCH, bool FULL, int XG>
__global__ void __launch_bounds__(NW * MOE_WAVE)
expert_fused_kernel(PlanArgs plan, RouteArgs route, const float* __restrict__ h, const float* __restrict__ topk_w,
                    int H, int I, const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu,
                    const uint16_t* __restrict__ Wd, float* __restrict__ part, int nrange,
                    int32_t* __restrict__ err) {
    constexpr bool ROUTE = XG > 0;        // experts in XG groups of 64
    constexpr int NT = NW * MOE_WAVE;     // threads
    constexpr int CH = NW * CPW;          // channels per chunk
    constexpr int RG = NT / kThreads;     // down row groups (256 column threads each)
    constexpr int RPG = CH / RG;          // down rows per row group and chunk
    static_assert(NT % kThreads == 0 && CH % RG == 0, "tile");
    __shared__ float sp[2][CH];  // alternating per chunk: one barrier per chunk
    __shared__ float4 hs[Q * MOE_WAVE * 2];
    __shared__ float4 red[RG > 1 ? (RG - 1) * kThreads * CQ * 2 : 1];
    __shared__ __align__(16) uint64_t rkey[ROUTE ? kRouteMaxE : 2];
    __shared__ int4 rrank4[ROUTE ? XG * MOE_WAVE : 1];  // per expert: the P partial ranks, 0-padded
    __shared__ int rsel_e[ROUTE ? MOE_WAVE : 1];
    __shared__ float rsel_l[ROUTE ? MOE_WAVE : 1];
    __shared__ int rsel_p[ROUTE ? MOE_WAVE : 1];
    static_assert(!ROUTE || NT >= XG * MOE_WAVE, "one thread per expert");
    if constexpr (ROUTE) {
        // Every argument is read from the kernel-argument segment at entry:
        // a late read would be a memory round trip before the weight stream.
        pin_arg(route.part); pin_arg(route.bias); pin_arg(route.nslices); pin_arg(route.ids);
        pin_arg(route.wts); pin_arg(route.logits); pin_arg(route.sorted_routes); pin_arg(route.block_expert);
        pin_arg(route.counts); pin_arg(plan.E); pin_arg(plan.k); pin_arg(plan.b); pin_arg(h); pin_arg(Wg);
        pin_arg(Wu); pin_arg(Wd); pin_arg(part); pin_arg(nrange); pin_arg(H); pin_arg(I);
    }
    const int blk = blockIdx.x;
    const int range = blockIdx.y;
    const int b = plan.b;
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int ct = tid % kThreads;        // down column thread
    const int rgp = tid / kThreads;       // down row group

    constexpr int HPT = (Q * MOE_WAVE * 2 + NT - 1) / NT;  // float4 of h per thread
    float4 hreg[HPT];  // h of the first route, for the LDS stage
    int e, r0, nb, rv;
    float av;
    bool spec;
    uint64_t todo;
    int rk[ROUTE ? XG : 1], below[ROUTE ? XG : 1];  // ROUTE: ranks and plan positions of experts 64 g + lane
    float lg = 0.f;                                  // ROUTE: logit of expert tid
    if constexpr (ROUTE) {
        // The workgroup routes the (single) token itself.  Round 1: h and the
        // router's slice partials of logit tid, none of which depends on the
        // routing.  Every workgroup adds the slices in the same order, so all
        // hold the same logits, top-k and affinities.
#pragma unroll
        for (int u = 0; u < HPT; ++u)
            hreg[u] = *reinterpret_cast<const float4*>(h + min((tid + NT * u) * 4, H - 4));
        const int E = plan.E, k = plan.k;
        const int ex = min(tid, E - 1);
        // only the waves that hold experts load, one 4-byte buffer load per
        // slice (slices past nslices are out of the buffer's range and read 0)
        float xs[kRouteSlices];
        if (wave * MOE_WAVE < E) {  // uniform
            const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(route.part), (short)0, route.nslices * E * 4, 0x00020000);
#pragma unroll
            for (int u = 0; u < kRouteSlices; ++u)
                xs[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pr, (u * E + ex) * 4, 0, 0));
        } else {
#pragma unroll
            for (int u = 0; u < kRouteSlices; ++u) xs[u] = 0.f;
        }
        const float bv = route.bias ? route.bias[ex] : 0.f;
#pragma unroll
        for (int u = 0; u < kRouteSlices; ++u) lg += u < route.nslices ? xs[u] : 0.f;  // slice order
        if (route.bias) lg += bv;
        if (tid < E) {
            rkey[tid] = order_key((lg != lg) ? -INFINITY : lg, tid);  // NaN ranks as -inf
            if (route.logits && blk == 0 && range == 0) route.logits[tid] = lg;
        }
        __syncthreads();
        // rank(x) = # keys above x's key, counted in P parts of E/P keys
        const int lp = 4 * E <= NT ? 2 : (2 * E <= NT ? 1 : 0);
        const int P = 1 << lp;
        const int n = E >> lp;
        if (tid < P * E) {
            const int pt = (tid >= E) + (tid >= 2 * E) + (tid >= 3 * E);
            const int x = tid - pt * E;
            int* dst = reinterpret_cast<int*>(rrank4 + x);
            dst[pt] = count_greater(rkey, pt * n, n, rkey[x]);
            if (pt == 0)
                for (int j = P; j < 4; ++j) dst[j] = 0;
        }
        __syncthreads();
        // Every wave: lane l looks at experts l + 64 g.  The canonical plan of
        // one token has one block per selected expert, in ascending expert
        // order, so block blk belongs to the (blk+1)-th selected expert in id
        // order; its slot (route id) is its rank.  That is all the weight
        // stream needs; the affinities follow once it is in flight.
#pragma unroll
        for (int g = 0; g < XG; ++g) {
            const int4 v = rrank4[min(lane + MOE_WAVE * g, E - 1)];
            rk[g] = lane + MOE_WAVE * g < E ? (v.x + v.y) + (v.z + v.w) : k;
        }
        int before = 0;
        e = -1;
        r0 = 0;
#pragma unroll
        for (int g = 0; g < XG; ++g) {
            const bool sel = rk[g] < k;
            const uint64_t m = __ballot(sel);
            below[g] = before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const uint64_t hit = __ballot(sel && below[g] == blk);
            if (hit) {
                const int q = __builtin_ctzll(hit);
                e = q + MOE_WAVE * g;
                r0 = __builtin_amdgcn_readlane(rk[g], q);
            }
            before += __popcll(m);
        }
        if (e < 0) return;  // no such block (uniform)
        av = 0.f;  // set once the selected logits are in LDS
        rv = -1;
        nb = 0;
        spec = true;
        todo = 1;
    } else {
    // First round of independent loads: counts, this and the previous block's
    // expert, and the block's rows (lane q holds row q; b <= 64).
    nb = plan.counts[0];
    e = plan.block_expert[blk];
    const int eprev = blk > 0 ? plan.block_expert[blk - 1] : -1;
    rv = plan.sorted_routes[(size_t)blk * b + min(lane, b - 1)];
    if (lane >= b) rv = plan.R;
    if (nb < 0 || nb > plan.max_blocks) {
        if (blk == 0 && range == 0 && tid == 0) atomicOr(err, DEVERR_BAD_COUNTS);
        nb = nb < 0 ? 0 : plan.max_blocks;
    }
    if (blk >= nb) return;
    if (e < 0 || e >= plan.E) {
        if (range == 0 && tid == 0) atomicOr(err, DEVERR_BAD_BLOCK_EXPERT);
        return;
    }
    if (eprev == e) return;  // not the first block of the expert's run (uniform)
    }

    const int cbase = range * NCH * CH;
    const size_t ebase = (size_t)e * I * H;
    const uint16_t* gbase = Wg + ebase + lane * 8;
    const uint16_t* ubase = Wu + ebase + lane * 8;
    const uint16_t* dbase = Wd + ebase + ct * 8;
    uint4 wg[2][CPW][Q], wu[2][CPW][Q], wd[2][RPG][CQ];
    // Rows past I load row 0 of the expert and are multiplied by zero; with
    // FULL (H == 512*Q == 2048*CQ) every column is in range and the loads
    // share one base address with constant offsets.
    auto issue_gu = [&](int ci, int buf) {
        const int j0 = cbase + ci * CH;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int j = j0 + wave * CPW + c;
            const size_t row = (size_t)(j < I ? j : 0) * H;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                if (FULL || (lane + MOE_WAVE * q) * 8 < H) {
                    wg[buf][c][q] = load_stream16(gbase + row + MOE_WAVE * 8 * q);
                    wu[buf][c][q] = load_stream16(ubase + row + MOE_WAVE * 8 * q);
                } else {
                    wg[buf][c][q] = wu[buf][c][q] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    };
    auto issue_d = [&](int ci, int buf) {
        const int j0 = cbase + ci * CH;
#pragma unroll
        for (int rr = 0; rr < RPG; ++rr) {
            const int j = j0 + rgp * RPG + rr;
            const size_t row = (size_t)(j < I ? j : 0) * H;
#pragma unroll
            for (int cq = 0; cq < CQ; ++cq) {
                if (FULL || (ct + kThreads * cq) * 8 < H)
                    wd[buf][rr][cq] = load_stream16(dbase + row + kThreads * 8 * cq);
                else
                    wd[buf][rr][cq] = make_uint4(0, 0, 0, 0);
            }
        }
    };

    if constexpr (ROUTE) {
        // The weight stream of the token's route starts now, two chunks deep.
        issue_gu(0, 0);
        issue_d(0, 0);
        if (NCH > 1) {
            issue_gu(1, 1);
            issue_d(1, 1);
        }
        // Slot rank of each selected expert: its id, logit and plan position
        // (wave g holds the logits of experts 64 g + lane).
        const int k = plan.k;
#pragma unroll
        for (int g = 0; g < XG; ++g) {
            if (wave == g && rk[g] < k) {
                rsel_e[rk[g]] = tid;
                rsel_l[rk[g]] = (lg != lg) ? -INFINITY : lg + 0.0f;  // the logit of the order key
                rsel_p[rk[g]] = below[g];
            }
        }
    } else {
    // Second round, issued before any weight: every row's id check and
    // affinity (unconditional loads, the row is in range) and h of row 0,
    // which is the expert's first route whenever the plan is well formed.
    // The loads take clamped, always-valid addresses and their values are
    // selected afterwards: a load inside a branch would be waited for at the
    // branch's end, one round trip at a time.
    const bool inr = rv >= 0 && rv < plan.R;
    const int rc = min(max(rv, 0), plan.R - 1);
    const int idv0 = plan.topk_ids[rc];
    const float avv0 = topk_w[rc];
    r0 = __builtin_amdgcn_readfirstlane(rv);
    spec = r0 >= 0 && r0 < plan.R;  // uniform
    const float* h0row = h + (size_t)(min(max(r0, 0), plan.R - 1) / plan.k) * H;
#pragma unroll
    for (int u = 0; u < HPT; ++u)
        hreg[u] = *reinterpret_cast<const float4*>(h0row + min((tid + NT * u) * 4, H - 4));
    // The weight stream of the expert's first route starts now, two chunks deep.
    issue_gu(0, 0);
    issue_d(0, 0);
    if (NCH > 1) {
        issue_gu(1, 1);
        issue_d(1, 1);
    }
    const bool ok = inr && idv0 == e;
    if (!ok && rv != plan.R && range == 0 && tid < MOE_WAVE) atomicOr(err, DEVERR_BAD_PLAN);
    if (!ok) rv = -1;
    av = ok ? avv0 : 0.f;
    todo = __ballot(rv >= 0);  // valid rows of the first block (wave-uniform)
    }

    // Gate/up of one chunk from h in LDS: sp[c] = a * SiLU(g_j) * u_j.
    auto gateup = [&](int ci, int buf, float a) {
        float* spc = sp[ci & 1];
        const int j0 = cbase + ci * CH;
        float ag[CPW], au[CPW];
#pragma unroll
        for (int c = 0; c < CPW; ++c) ag[c] = au[c] = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (!FULL && (lane + MOE_WAVE * q) * 8 >= H) continue;
            const float4 h0 = hs[(lane + MOE_WAVE * q) * 2];
            const float4 h1 = hs[(lane + MOE_WAVE * q) * 2 + 1];
            const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                float gf[8], uf[8];
                unpack8(wg[buf][c][q], gf);
                unpack8(wu[buf][c][q], uf);
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    ag[c] = fmaf(gf[x], hv[x], ag[c]);
                    au[c] = fmaf(uf[x], hv[x], au[c]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const float g = wave_sum(ag[c]);
            const float u = wave_sum(au[c]);
            const int j = j0 + wave * CPW + c;
            if (lane == 0) spc[wave * CPW + c] = j < I ? a * silu_mul(g, u) : 0.f;
        }
    };
    // Down rows of one chunk scaled by sp, accumulated per column thread.
    auto down = [&](int ci, int buf, float (&acc)[CQ][8]) {
        const float* spc = sp[ci & 1];
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq)
#pragma unroll
            for (int rr = 0; rr < RPG; ++rr) {
                float wf[8];
                unpack8(wd[buf][rr][cq], wf);
                const float s = spc[rgp * RPG + rr];
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[cq][x] = fmaf(s, wf[x], acc[cq][x]);
            }
    };
    // Row groups 1.. hand their sums to row group 0 (added in group order),
    // which writes part[route][range][:].
    auto finish = [&](int r, float (&acc)[CQ][8]) {
        if (RG > 1) {
            if (rgp > 0) {
#pragma unroll
                for (int cq = 0; cq < CQ; ++cq) {
                    float4* o = red + (((size_t)(rgp - 1) * kThreads + ct) * CQ + cq) * 2;
                    o[0] = make_float4(acc[cq][0], acc[cq][1], acc[cq][2], acc[cq][3]);
                    o[1] = make_float4(acc[cq][4], acc[cq][5], acc[cq][6], acc[cq][7]);
                }
            }
            __syncthreads();
            if (rgp == 0) {
#pragma unroll
                for (int g2 = 1; g2 < RG; ++g2)
#pragma unroll
                    for (int cq = 0; cq < CQ; ++cq) {
                        const float4* o = red + (((size_t)(g2 - 1) * kThreads + ct) * CQ + cq) * 2;
                        const float4 u0 = o[0], u1 = o[1];
                        acc[cq][0] += u0.x; acc[cq][1] += u0.y; acc[cq][2] += u0.z; acc[cq][3] += u0.w;
                        acc[cq][4] += u1.x; acc[cq][5] += u1.y; acc[cq][6] += u1.z; acc[cq][7] += u1.w;
                    }
            }
        }
        if (rgp == 0) {
#pragma unroll
            for (int cq = 0; cq < CQ; ++cq) {
                const int col = (ct + kThreads * cq) * 8;
                if (col >= H) continue;
                float* dst = part + ((size_t)r * nrange + range) * H + col;
                *reinterpret_cast<float4*>(dst) = make_float4(acc[cq][0], acc[cq][1], acc[cq][2], acc[cq][3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[cq][4], acc[cq][5], acc[cq][6], acc[cq][7]);
            }
        }
        __syncthreads();  // red and hs are reused by the next route
    };

    if (spec && (todo & 1ull)) {
        // Row 0 is the first route: its h and the first two chunks are in
        // flight.  Chunk ci+2 refills buffer ci&1 as soon as chunk ci's gate/up
        // (then down) rows have been consumed.
        todo &= ~1ull;
#pragma unroll
        for (int u = 0; u < HPT; ++u) {
            const int i = tid + NT * u;
            if (i < Q * MOE_WAVE * 2) hs[i] = i * 4 < H ? hreg[u] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float acc[CQ][8];
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq)
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[cq][x] = 0.f;
        __syncthreads();  // hs ready (ROUTE: and the selected experts)
        if constexpr (ROUTE) {
            // Lane s: slot s.  The renormalised softmax over the selected
            // logits (as the router computes it); workgroup (0, 0) writes the
            // token's ids, affinities and plan, as the router and the
            // alignment would.
            const int k = plan.k;
            const int s = min(lane, k - 1);
            const int se = rsel_e[s];
            const float sw = topk_softmax(rsel_l[s], lane, k);
            av = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sw), r0));
            if (blk == 0 && range == 0 && wave == 0) {
                const int pos = rsel_p[s];
                if (lane < k) {
                    route.ids[lane] = se;
                    route.wts[lane] = sw;
                    route.block_expert[pos] = se;
                    route.sorted_routes[pos * b] = lane;
                }
                for (int i = lane; i < k * b; i += MOE_WAVE)
                    if (i % b) route.sorted_routes[i] = k;  // pad sentinel M*k
                if (lane == 0) {
                    route.counts[0] = k;
                    route.counts[1] = k * b;
                }
            }
        }
        const float a = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(av)));
        // sp alternates per chunk, so the barrier of chunk ci+1 already
        // orders chunk ci's reads before chunk ci+2 overwrites them.
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci) {
            const int buf = ci & 1;
            gateup(ci, buf, a);
            if (ci + 2 < NCH) issue_gu(ci + 2, buf);
            __syncthreads();
            down(ci, buf, acc);
            if (ci + 2 < NCH) issue_d(ci + 2, buf);
        }
        finish(r0, acc);
    }
    // Every other route (an expert routed more than once by one token, or a
    // plan whose row 0 is not a route): h to LDS, then the chunks one at a
    // time, the rows of the first block first, then the following blocks of
    // the run, resolved row by row.
    int bb = blk + 1, q0 = 0;
    for (;;) {
        int r;
        float a;
        if (todo) {
            const int q = __builtin_ctzll(todo);
            todo &= todo - 1;
            r = __builtin_amdgcn_readlane(rv, q);
            a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(av), q));
        } else {
            if (bb >= nb || plan.block_expert[bb] != e) break;
            r = plan_route(plan, bb, q0, e, err);
            a = r >= 0 ? topk_w[r] : 0.f;
            if (++q0 == b) { ++bb; q0 = 0; }
            if (r < 0) continue;  // uniform
        }
        const float* hr = h + (size_t)(r / plan.k) * H;
        for (int i = tid; i < Q * MOE_WAVE * 2; i += NT) {
            const int col = i * 4;
            hs[i] = col < H ? *reinterpret_cast<const float4*>(hr + col) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float acc[CQ][8];
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq)
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[cq][x] = 0.f;
        __syncthreads();  // hs ready
        for (int ci = 0; ci < NCH; ++ci) {
            issue_gu(ci, 0);
            issue_d(ci, 0);
            gateup(ci, 0, a);
            __syncthreads();
            down(ci, 0, acc);
        }
        finish(r, acc);
    }
}

// ---------------------------------------------------------------------------
// Split schedule, gate/up.  Grid (plan blocks, ceil(I / (4*CPW))); wave w of
// workgroup (blk, cy) owns channels (cy*4 + w)*CPW + c of the expert whose
// run of blocks starts at blk.  Its weights are loaded once into registers
// and applied to every route of the run, G routes at a time: their h rows
// are staged in LDS, then each wave forms its channels' p values (weights
// unpacked per route, so that only the packed form stays live).
// The plan rows of the first block arrive with the first round of loads; the
// row checks and the h rows of the first G rows of the block (the expert's
// first routes in a well-formed plan) follow as the second round and are in
// LDS before the weights are requested, since a load queued behind the
// weight stream would wait for all of it (the other workgroups on the CU keep
// it streaming meanwhile).  Every such load has a clamped, always-valid
// address.  A first group that turns out to differ from those rows, and every
// later group, is staged again.
template <int Q, int CPW, int G>
__global__ void __launch_bounds__(kThreads)
gateup_dense_kernel(PlanArgs plan, const float* __restrict__ h, int H, int I, const uint16_t* __restrict__ Wg,
                    const uint16_t* __restrict__ Wu, float* __restrict__ p, int32_t* __restrict__ err) {
    extern __shared__ __align__(16) float4 hst[];  // [G][RS]: h rows, padded to RS float4
    constexpr int PR = (Q * MOE_WAVE * 2 + kThreads - 1) / kThreads;  // float4 of one h row per thread
    constexpr int RS = PR * kThreads;
    const int blk = blockIdx.x;
    const int b = plan.b;
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int H4 = H / 4;

    // Round 1: counts, this and the previous block's expert, the block's rows.
    int nb = plan.counts[0];
    const int e = plan.block_expert[blk];
    const int eprev = blk > 0 ? plan.block_expert[blk - 1] : -1;
    int rv = plan.sorted_routes[(size_t)blk * b + min(lane, b - 1)];
    if (lane >= b) rv = plan.R;
    if (nb < 0 || nb > plan.max_blocks) {
        if (blk == 0 && blockIdx.y == 0 && tid == 0) atomicOr(err, DEVERR_BAD_COUNTS);
        nb = nb < 0 ? 0 : plan.max_blocks;
    }
    if (blk >= nb) return;
    if (e < 0 || e >= plan.E) {
        if (blockIdx.y == 0 && tid == 0) atomicOr(err, DEVERR_BAD_BLOCK_EXPERT);
        return;
    }
    if (eprev == e) return;  // not the first block of the expert's run (uniform)

    // Round 2, before the weights: the row checks, and h of rows 0..G-1
    // staged in LDS (lanes past b hold the pad sentinel).
    const int idv = plan.topk_ids[min(max(rv, 0), plan.R - 1)];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int r = __builtin_amdgcn_readlane(rv, i);
        const float* hr = h + (size_t)plan.fk.div(min(max(r, 0), plan.R - 1)) * H;
#pragma unroll
        for (int v = 0; v < PR; ++v)
            hst[i * RS + tid + kThreads * v] = *reinterpret_cast<const float4*>(hr + min(tid + kThreads * v, H4 - 1) * 4);
    }

    const int j0 = (blockIdx.y * kWaves + wave) * CPW;  // waves past I still take part in the barriers
    uint4 wg[CPW][Q], wu[CPW][Q];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int j = min(j0 + c, I - 1);  // clamped rows are computed and discarded
        const uint16_t* rg = Wg + ((size_t)e * I + j) * H;
        const uint16_t* ru = Wu + ((size_t)e * I + j) * H;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int col = min((lane + MOE_WAVE * q) * 8, H - 8);
            wg[c][q] = load_stream16(rg + col);
            wu[c][q] = load_stream16(ru + col);
        }
    }

    auto rows_ok = [&](int rvx, int idx) {
        const bool ok = rvx >= 0 && rvx < plan.R && idx == e;
        if (!ok && rvx != plan.R && blockIdx.y == 0 && tid < MOE_WAVE) atomicOr(err, DEVERR_BAD_PLAN);
        return __ballot(ok);
    };
    uint64_t todo = rows_ok(rv, idv);
    // the staged rows 0..n-1 are the first group iff the valid rows begin with them
    const int n0 = min(G, __popcll(todo));
    bool staged = (todo & ((1ull << G) - 1)) == ((1ull << n0) - 1);  // else staged again below
    int bb = blk;
    for (;;) {
        if (!todo) {  // the run's next block: its rows, then their checks
            if (++bb >= nb || plan.block_expert[bb] != e) break;
            int rv2 = plan.sorted_routes[(size_t)bb * b + min(lane, b - 1)];
            if (lane >= b) rv2 = plan.R;
            todo = rows_ok(rv2, plan.topk_ids[min(max(rv2, 0), plan.R - 1)]);
            rv = rv2;
            continue;
        }
        int rt[G];
        int ng = 0;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            rt[i] = -1;
            if (todo) {
                const int q = __builtin_ctzll(todo);
                todo &= todo - 1;
                rt[i] = __builtin_amdgcn_readlane(rv, q);
                ng = i + 1;
            }
        }
        if (!staged) {
            __syncthreads();  // the previous group's h is no longer read
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float* hr = h + (size_t)plan.fk.div(max(rt[i], 0)) * H;
#pragma unroll
                for (int v = 0; v < PR; ++v)
                    hst[i * RS + tid + kThreads * v] =
                        *reinterpret_cast<const float4*>(hr + min(tid + kThreads * v, H4 - 1) * 4);
            }
        }
        staged = false;
        __syncthreads();
        for (int i = 0; i < ng; ++i) {  // uniform
            const float4* hr = hst + i * RS;
            float ag[CPW], au[CPW];
#pragma unroll
            for (int c = 0; c < CPW; ++c) ag[c] = au[c] = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int c8 = lane + MOE_WAVE * q;
                if (c8 * 8 >= H) continue;
                const float4 h0 = hr[c8 * 2];
                const float4 h1 = hr[c8 * 2 + 1];
                const float hx[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    float gf[8], uf[8];
                    unpack8(opaque(wg[c][q]), gf);
                    unpack8(opaque(wu[c][q]), uf);
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        ag[c] = fmaf(gf[x], hx[x], ag[c]);
                        au[c] = fmaf(uf[x], hx[x], au[c]);
                    }
                }
            }
            int r = rt[0];
#pragma unroll
            for (int ii = 1; ii < G; ++ii)
                if (ii == i) r = rt[ii];
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const float g = wave_sum(ag[c]);
                const float u = wave_sum(au[c]);
                if (lane == 0 && j0 + c < I) p[(size_t)r * I + j0 + c] = silu_mul(g, u);
            }
        }
    }
}

// Split schedule, down.  Grid (ceil(H / CB) column blocks, plan blocks).
// Workgroup (cb, blk) multiplies the routes of plan block blk (8 rows at a
// time) by columns [cb*CB, cb*CB + CB) of W_down,e over all I rows, so each
// route's output for those columns is complete: one partial per route, and
// the combine adds only the k routes of a token.  Column blocks run along x,
// so the consecutive plan blocks of an expert's run land on one XCD next to
// each other in dispatch order, and a second block's weight reads can hit in
// that XCD's L2.
// Thread t covers columns cb*CB + 8*(t % TPR) .. +8 and rows rg, rg + RGS, ...
// (rg = t / TPR).  The scaled intermediates s[j][i] = a_i * p[route_i][j] of
// the 8 rows are staged route-minor in LDS (kDownStage rows at a time), the
// weight rows stream through registers kDownNB at a time, double-buffered,
// and the RGS row groups are added at the end: by an xor butterfly inside
// each wave, then the waves in wave order.  Rows that are not routes of the
// expert (pads) get s = 0 and no output; RT = 2, 4 or 8 accumulators cover
// the leading rows up to the last route.  This is the vector-ALU form; the
// matrix-core form (down_pass_mfma) computes the same partials.
constexpr int kDownStage = 1024;  // rows of s staged at a time (32 KiB)
constexpr int kDownNB = 4;        // weight rows per thread and buffer

// The staged p values of one thread for a stage of down rows js .. js + jn:
// its route's rows 4 q .. 4 q + 3 for the row quads q = (tid >> 3) + 32 u,
// as 16-byte buffer loads (rows past I read zero) when I % 4 == 0, else one
// by one (rows past the stage clamped).  Issued before the weights.
constexpr int kDownQuads = kDownStage / 4 / (kThreads / 8);  // row quads per thread and stage

__device__ __forceinline__ void down_load_p(const float* __restrict__ p, int sr, int I, int js, int jn,
                                            float4 (&pv)[kDownQuads]) {
    const int tid = threadIdx.x;
    if (I % 4 == 0) {  // uniform
        const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(p + (size_t)sr * I), (short)0, I * 4, 0x00020000);
#pragma unroll
        for (int u = 0; u < kDownQuads; ++u) {
            const int jq = (tid >> 3) + (kThreads / 8) * u;
            const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(prs, (js + 4 * jq) * 4, 0, 0);
            pv[u] = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                                __uint_as_float(x.w));
        }
    } else {
#pragma unroll
        for (int u = 0; u < kDownQuads; ++u) {
            const int j4 = 4 * ((tid >> 3) + (kThreads / 8) * u);
            const float* q = p + (size_t)sr * I + js;
            pv[u] = make_float4(q[min(j4, jn - 1)], q[min(j4 + 1, jn - 1)], q[min(j4 + 2, jn - 1)],
                                q[min(j4 + 3, jn - 1)]);
        }
    }
}

// The staged s values of a stage (rows js .. js + jn) from the VQ gate/up
// partials vp [R][ny][2][I]: s_i[j] = a_i * SiLU(og) * ou, og and ou the sums
// over the partial rows y in order, for the pass's routes i (8 slots; slots
// not in `valid` get 0).  Thread t takes rows t, t + 256, ... of each valid
// route, all of a route's loads in flight (partial rows in batches of 4).
// Rows nz .. (nz >= jn) of each slot are zero-filled.  MINOR: dsm[j * 8 + i]
// (the vector-ALU pass); else dsm[i * kDownStage + j] (the matrix-core pass).
// first() (the caller's first weight requests) runs once the first slot's
// loads are out, then a barrier (the previous stage's s is no longer read)
// precedes the first write: waiting for those loads does not wait for the
// weights.
constexpr int kVqRowsPT = kDownStage / kThreads;  // rows per thread and stage

template <bool MINOR, typename F>
__device__ __forceinline__ void stage_vq(const VqP& vq, int I, int js, int jn, int nz, const int (&rr)[8],
                                         const float (&ra)[8], uint32_t valid, float* dsm, F&& first) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float sv[kVqRowsPT];
        if ((valid >> i) & 1) {  // uniform
            const float* src = vq.vp + (size_t)rr[i] * vq.ny * 2 * I + js;
            float og[kVqRowsPT], ou[kVqRowsPT];
#pragma unroll
            for (int u = 0; u < kVqRowsPT; ++u) og[u] = ou[u] = 0.f;
            constexpr int YB = 4;  // partial rows per batch (8 measured slower: fewer waves per SIMD)
            for (int y0 = 0; y0 < vq.ny; y0 += YB) {
                float g4[kVqRowsPT][YB], u4[kVqRowsPT][YB];
#pragma unroll
                for (int u = 0; u < kVqRowsPT; ++u) {
                    const int j = min(tid + kThreads * u, jn - 1);
#pragma unroll
                    for (int y = 0; y < YB; ++y) {
                        const int yy = min(y0 + y, vq.ny - 1);
                        g4[u][y] = src[(size_t)(2 * yy) * I + j];
                        u4[u][y] = src[(size_t)(2 * yy + 1) * I + j];
                    }
                }
                if (i == 0 && y0 == 0) {  // uniform
                    first();
                    __syncthreads();
                }
#pragma unroll
                for (int u = 0; u < kVqRowsPT; ++u)
#pragma unroll
                    for (int y = 0; y < YB; ++y) {
                        og[u] += y0 + y < vq.ny ? g4[u][y] : 0.f;
                        ou[u] += y0 + y < vq.ny ? u4[u][y] : 0.f;
                    }
            }
#pragma unroll
            for (int u = 0; u < kVqRowsPT; ++u) sv[u] = ra[i] * silu_mul(og[u], ou[u]);
        } else {
#pragma unroll
            for (int u = 0; u < kVqRowsPT; ++u) sv[u] = 0.f;
            if (i == 0) {  // uniform
                first();
                __syncthreads();
            }
        }
#pragma unroll
        for (int u = 0; u < kVqRowsPT; ++u) {
            const int j = tid + kThreads * u;
            if (j < nz) {
                const float v = j < jn ? sv[u] : 0.f;
                if (MINOR)
                    dsm[j * 8 + i] = v;
                else
                    dsm[i * kDownStage + j] = v;
            }
        }
    }
}

template <int CB, int RT, bool VQ>
__device__ __forceinline__ void down_pass(int e, int H, int I, const uint16_t* __restrict__ Wd,
                                          const float* __restrict__ p, const VqP& vq, const int (&rr)[8],
                                          const float (&ra)[8], uint32_t valid, float* __restrict__ part,
                                          float* dsm) {
    constexpr int TPR = CB / 8;
    constexpr int RGS = kThreads / TPR;
    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;
    const int wave = tid / MOE_WAVE;
    const int c8 = tid % TPR;
    const int rg = tid / TPR;
    const int col = blockIdx.x * CB + c8 * 8;
    const uint16_t* wbase = Wd + (size_t)e * I * H + min(col, H - 8);
    // the route this thread stages (route-minor layout: thread t takes route t % 8)
    const int si = tid & 7;
    int sr = 0;
    float sa = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i == si && ((valid >> i) & 1)) {
            sr = rr[i];
            sa = ra[i];
        }
    const bool sv = si < RT && ((valid >> si) & 1);

    float acc[RT][8];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[i][x] = 0.f;
    uint4 w0[kDownNB], w1[kDownNB];
    for (int js = 0; js < I; js += kDownStage) {
        const int jn = min(kDownStage, I - js);
        const int nu = (jn + RGS - 1) / RGS;  // rows per thread in this stage (clamped beyond jn)
        // Rows past the stage load its last row (same address for all, cached)
        // and are multiplied by s = 0.
        auto issue = [&](uint4 (&w)[kDownNB], int u0) {
#pragma unroll
            for (int r = 0; r < kDownNB; ++r) {
                const int jl = min(rg + RGS * (u0 + r), jn - 1);
                w[r] = load_stream16(wbase + (size_t)(js + jl) * H);
            }
        };
        auto compute = [&](const uint4 (&w)[kDownNB], int u0) {
#pragma unroll
            for (int r = 0; r < kDownNB; ++r) {
                const int jl = rg + RGS * (u0 + r);
                const float4* s4 = reinterpret_cast<const float4*>(dsm + (size_t)min(jl, jn - 1) * 8);
                const float4 a = s4[0];
                float sv8[8] = {a.x, a.y, a.z, a.w, 0.f, 0.f, 0.f, 0.f};
                if (RT > 4) {
                    const float4 b4 = s4[1];
                    sv8[4] = b4.x; sv8[5] = b4.y; sv8[6] = b4.z; sv8[7] = b4.w;
                }
                const bool in = jl < jn;
                float wf[8];
                unpack8(w[r], wf);
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    const float sx = in ? sv8[i] : 0.f;
#pragma unroll
                    for (int x = 0; x < 8; ++x) acc[i][x] = fmaf(sx, wf[x], acc[i][x]);
                }
            }
        };
        if constexpr (VQ) {
            // stage s from the gate/up partials (the first weights go out
            // right after the first route's partial loads)
            stage_vq<true>(vq, I, js, jn, jn, rr, ra, valid, dsm, [&] { issue(w0, 0); });
        } else {
            // stage s (the p loads go out before the first weights)
            float4 pv[kDownQuads];
            down_load_p(p, sr, I, js, jn, pv);
            issue(w0, 0);
            __syncthreads();  // the previous stage's s is no longer read
#pragma unroll
            for (int u = 0; u < kDownQuads; ++u) {
                const int j4 = 4 * ((tid >> 3) + (kThreads / 8) * u);
                const float v4[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (j4 + c < jn) dsm[(j4 + c) * 8 + si] = sv ? sa * v4[c] : 0.f;
            }
        }
        __syncthreads();
        for (int u0 = 0; u0 < nu; u0 += 2 * kDownNB) {
            issue(w1, u0 + kDownNB);
            compute(w0, u0);
            issue(w0, u0 + 2 * kDownNB);
            compute(w1, u0 + kDownNB);
        }
    }
    // row groups: xor butterfly over the lane bits above the column bits, then
    // the waves added in wave order
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int x = 0; x < 8; ++x)
#pragma unroll
            for (int m = TPR; m < MOE_WAVE; m <<= 1) acc[i][x] += __shfl_xor(acc[i][x], m, MOE_WAVE);
    __syncthreads();  // s is no longer read
    if (lane < TPR) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            float4* o = reinterpret_cast<float4*>(dsm + ((size_t)wave * RT + i) * CB + c8 * 8);
            o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
            o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
        }
    }
    __syncthreads();
    if (wave == 0 && lane < TPR && col < H) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            if (!((valid >> i) & 1)) continue;
            float o[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) o[x] = 0.f;
            float4 v[kWaves][2];
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float4* q = reinterpret_cast<const float4*>(dsm + ((size_t)w * RT + i) * CB + c8 * 8);
                v[w][0] = q[0];
                v[w][1] = q[1];
            }
            // (w0 + w1) + (w2 + w3)
            const float4 l0 = v[0][0], l1 = v[1][0], l2 = v[2][0], l3 = v[3][0];
            const float4 h0 = v[0][1], h1 = v[1][1], h2 = v[2][1], h3 = v[3][1];
            o[0] = (l0.x + l1.x) + (l2.x + l3.x); o[1] = (l0.y + l1.y) + (l2.y + l3.y);
            o[2] = (l0.z + l1.z) + (l2.z + l3.z); o[3] = (l0.w + l1.w) + (l2.w + l3.w);
            o[4] = (h0.x + h1.x) + (h2.x + h3.x); o[5] = (h0.y + h1.y) + (h2.y + h3.y);
            o[6] = (h0.z + h1.z) + (h2.z + h3.z); o[7] = (h0.w + h1.w) + (h2.w + h3.w);
            float* dst = part + (size_t)rr[i] * H + col;
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
    __syncthreads();  // dsm is reused by the next pass
}

// The same product on the matrix cores (bf16 16x16x32, fp32 accumulation)
// for a pass of up to 8 routes and the CB columns of the workgroup (CB = 128
// or 256): NCG = CB / 128 column groups of 128, NKG = 4 / NCG channel
// groups.  Wave w covers columns cb*CB + 128*(w % NCG) + [0, 128) and the K
// tiles of 32 channels kt = w / NCG, w / NCG + NKG, ... of each stage.  MFMA rows
// 0..7 are the hi bf16 parts of s = a_i * p[route_i][j] for routes i = 0..7,
// rows 8..15 their lo parts (s = hi + lo + O(2^-18 |s|)); the weights are
// exact in bf16.  Lane l loads 16 bytes (8 columns) of each of the 8 rows
// j0 + 8 (l / 16) + i of the tile at columns 8 (l % 16) .. +7 of the wave's
// 128; MFMA g (g = 0..7) takes column 8 n + g of lane n = l % 16 from each
// row -- two rows per register, by byte permutes -- so the 8 products of a
// tile cover the wave's 128 columns with no transpose in memory.  At the end
// hi and lo rows are added (lane l + 32 into lane l), then the NKG waves of a
// column group in wave order, and row i of the result is route i's partial.
constexpr int kMfmaTile = 32;

template <int CB, bool VQ>
__device__ __forceinline__ void down_pass_mfma(int e, int H, int I, const uint16_t* __restrict__ Wd,
                                               const float* __restrict__ p, const VqP& vq, const int (&rr)[8],
                                               const float (&ra)[8], uint32_t valid, float* __restrict__ part,
                                               float* dsm) {
    constexpr int NCG = CB / 128, NKG = kWaves / NCG;
    static_assert((CB == 128 || CB == 256) && kWaves == 4, "column groups of 128 over four waves");
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;
    const int wave = tid / MOE_WAVE;
    const int chf = wave % NCG, kh = wave / NCG;
    const int colw = blockIdx.x * CB + 128 * chf;         // the wave's first column
    const int coll = colw + 8 * (lane % 16);              // this lane's 8 columns
    const uint16_t* wbase = Wd + (size_t)e * I * H + min(coll, H - 8);
    const int rsub = 8 * (lane / 16);                     // the lane's 8 rows of a tile
    // the route this thread stages: s route-major in LDS, dsm[i][j] (i < 8)
    const int si = tid & 7;
    int sr = 0;
    float sa = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i == si && ((valid >> i) & 1)) {
            sr = rr[i];
            sa = ra[i];
        }
    const bool sv = (valid >> si) & 1;
    f32x4_t acc[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 wb[2][8];
    for (int js = 0; js < I; js += kDownStage) {
        const int jn = min(kDownStage, I - js);
        const int nt = (jn + kMfmaTile - 1) / kMfmaTile;  // tiles of the stage
        auto issue = [&](uint4 (&w)[8], int kt) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int jl = min(kMfmaTile * kt + rsub + i, jn - 1);
                w[i] = load_stream16(wbase + (size_t)(js + jl) * H);
            }
        };
        if constexpr (VQ) {
            // stage s from the gate/up partials (the first weights go out
            // right after the first route's partial loads)
            stage_vq<false>(vq, I, js, jn, nt * kMfmaTile, rr, ra, valid, dsm, [&] {
                if (kh < nt) issue(wb[0], kh);
            });
        } else {
            // stage s (the p loads go out before the first weights; one by one
            // here: the 16-byte form of the VALU pass measured slower in this one)
            constexpr int SPT = kDownStage / (kThreads / 8);
            float pv[SPT];
#pragma unroll
            for (int u = 0; u < SPT; ++u) {
                const int jj = min((tid >> 3) + (kThreads / 8) * u, jn - 1);
                pv[u] = p[(size_t)sr * I + js + jj];
            }
            if (kh < nt) issue(wb[0], kh);
            __syncthreads();  // the previous stage's s is no longer read
#pragma unroll
            for (int u = 0; u < SPT; ++u) {
                const int jj = (tid >> 3) + (kThreads / 8) * u;
                if (jj < nt * kMfmaTile) dsm[si * kDownStage + jj] = (sv && jj < jn) ? sa * pv[u] : 0.f;
            }
        }
        __syncthreads();
        // one tile: A from the staged s of channels kt*32 + rsub .., B from w
        auto tile = [&](const uint4 (&w)[8], int kt) {
            // A: row lane % 16 (hi of route m, or lo of route m - 8), channels rsub .. rsub + 7 of the tile
            const int m = lane % 16;
            const float4* srow = reinterpret_cast<const float4*>(dsm + (m & 7) * kDownStage + kMfmaTile * kt + rsub);
            const float4 s0 = srow[0], s1 = srow[1];
            const float sx[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            uint32_t ak[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const uint32_t u = __float_as_uint(sx[x]);
                const uint32_t hi = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
                const float rem = sx[x] - __uint_as_float(hi << 16);
                const uint32_t ur = __float_as_uint(rem);
                const uint32_t lo = (ur + 0x7FFFu + ((ur >> 16) & 1u)) >> 16;
                ak[x] = m < 8 ? hi : lo;
            }
            const uint4 aw = make_uint4(ak[0] | (ak[1] << 16), ak[2] | (ak[3] << 16), ak[4] | (ak[5] << 16),
                                        ak[6] | (ak[7] << 16));
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                // column g of each row: the 16-bit half g % 2 of word g / 2; rows 2t, 2t + 1 into word t
                const uint32_t sel = (g & 1) ? 0x07060302u : 0x05040100u;
                auto word = [&](const uint4& v) { return (g >> 1) == 0 ? v.x : ((g >> 1) == 1 ? v.y : ((g >> 1) == 2 ? v.z : v.w)); };
                const uint4 bw = make_uint4(__builtin_amdgcn_perm(word(w[1]), word(w[0]), sel),
                                            __builtin_amdgcn_perm(word(w[3]), word(w[2]), sel),
                                            __builtin_amdgcn_perm(word(w[5]), word(w[4]), sel),
                                            __builtin_amdgcn_perm(word(w[7]), word(w[6]), sel));
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aw),
                                                                 __builtin_bit_cast(bf16x8_t, bw), acc[g], 0, 0, 0);
            }
        };
        // two register buffers in turn (indices fixed at compile time)
        for (int kt = kh; kt < nt; kt += 2 * NKG) {  // uniform per wave
            if (kt + NKG < nt) issue(wb[1], kt + NKG);
            tile(wb[0], kt);
            if (kt + NKG < nt) {
                if (kt + 2 * NKG < nt) issue(wb[0], kt + 2 * NKG);
                tile(wb[1], kt + NKG);
            }
        }
    }
    // hi + lo: lane l < 32 holds rows 4 (l / 16) + q (routes), lane l + 32 their lo parts
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[g][q] += __shfl_xor(acc[g][q], 32, MOE_WAVE);
    __syncthreads();  // s is no longer read
    // the other channel groups hand their sums to group 0 (added in wave order)
    float* red = dsm;  // [NKG - 1][NCG][32 lanes][8 g][4 q]
    if (kh > 0 && lane < 32) {
#pragma unroll
        for (int g = 0; g < 8; ++g)
            *reinterpret_cast<float4*>(red + ((((kh - 1) * NCG + chf) * 32 + lane) * 8 + g) * 4) =
                make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
    }
    __syncthreads();
    if (kh == 0 && lane < 32 && coll < H) {
        float o[4][8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            o[0][g] = acc[g][0];
            o[1][g] = acc[g][1];
            o[2][g] = acc[g][2];
            o[3][g] = acc[g][3];
#pragma unroll
            for (int k2 = 1; k2 < NKG; ++k2) {
                const float4 v =
                    *reinterpret_cast<const float4*>(red + ((((k2 - 1) * NCG + chf) * 32 + lane) * 8 + g) * 4);
                o[0][g] += v.x;
                o[1][g] += v.y;
                o[2][g] += v.z;
                o[3][g] += v.w;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * (lane / 16) + q;  // route row
            if (!((valid >> i) & 1)) continue;
            float* dst = part + (size_t)rr[i] * H + coll;
            *reinterpret_cast<float4*>(dst) = make_float4(o[q][0], o[q][1], o[q][2], o[q][3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[q][4], o[q][5], o[q][6], o[q][7]);
        }
    }
    __syncthreads();  // dsm is reused by the next pass
}

// The pass of up to 8 rows (routes rr[i], affinities ra[i], slots in valid).
template <int CB, bool MFMA, bool VQ>
__device__ __forceinline__ void down_rows(int e, int H, int I, const uint16_t* __restrict__ Wd,
                                          const float* __restrict__ p, const VqP& vq, const int (&rr)[8],
                                          const float (&ra)[8], uint32_t valid, float* __restrict__ part,
                                          float* dsm) {
    const int nv = 32 - __builtin_clz(valid);  // rows up to the last route
    if constexpr (MFMA)
        down_pass_mfma<CB, VQ>(e, H, I, Wd, p, vq, rr, ra, valid, part, dsm);
    else if (nv <= 2)
        down_pass<CB, 2, VQ>(e, H, I, Wd, p, vq, rr, ra, valid, part, dsm);
    else if (nv <= 4)
        down_pass<CB, 4, VQ>(e, H, I, Wd, p, vq, rr, ra, valid, part, dsm);
    else
        down_pass<CB, 8, VQ>(e, H, I, Wd, p, vq, rr, ra, valid, part, dsm);
}

// VQ: p from the gate/up partials (stage_vq).  ALIGN (R <= 64): no plan is
// read; lane r of every wave loads route r's id and affinity, the ballots of
// the id bits give each expert's count, rank and the blocks before it (the
// canonical plan of align_device.h), and block blk is found among them:
// its expert and its routes (the routes of that expert ranked b (blk -
// first block) .. + b - 1, ascending).  Workgroup (0, 0) also writes the
// whole plan.
template <int CB, bool MFMA, bool VQ, bool ALIGN>
__global__ void __launch_bounds__(kThreads)
down_kernel(PlanArgs plan, int H, int I, const uint16_t* __restrict__ Wd, const float* __restrict__ p,
            const float* __restrict__ topk_w, float* __restrict__ part, int32_t* __restrict__ err, VqP vq,
            AlignOut ao) {
    static_assert(kWaves == 4, "the final wave sum is written for four waves");
    extern __shared__ __align__(16) float dsm[];
    const int blk = blockIdx.y;
    const int b = plan.b;
    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;
    if constexpr (ALIGN) {
        const int R = plan.R;
        const int raw = lane < R ? plan.topk_ids[lane] : 0;
        const float wv = topk_w[min(lane, R - 1)];
        const bool ok = lane < R && raw >= 0 && raw < plan.E;
        if (blk == 0 && blockIdx.x == 0 && tid < MOE_WAVE)
            align_wave([&](int) { return raw; }, R, plan.E, plan.fb, ao.sorted_routes, ao.block_expert, ao.counts,
                       err);
        const int id = ok ? raw : 0;
        const uint64_t V = __ballot(ok);
        uint64_t bs[kIdBits];
        id_ballots(id, ok, bs);
        uint64_t eq, lt;
        id_match(id, V, bs, eq, lt);
        const int cnt = __popcll(eq);
        const bool first = ok && mbcnt64(eq) == 0;
        const int nblk = first ? (int)plan.fb.div(cnt + b - 1) : 0;
        int before = 0;
#pragma unroll
        for (int q = 0; q < 7; ++q) {  // nblk <= 64
            const uint64_t F = __ballot(first && ((nblk >> q) & 1));
            before += __popcll(lt & F) << q;
        }
        const uint64_t own = __ballot(first && before <= blk && blk < before + nblk);
        if (!own) return;  // past the last block (uniform)
        const int L = __builtin_ctzll(own);
        const int e = __builtin_amdgcn_readlane(id, L);
        const int skip = (blk - __builtin_amdgcn_readlane(before, L)) * b;  // routes of e in earlier blocks
        const uint32_t elo = __builtin_amdgcn_readlane((uint32_t)eq, L), ehi = __builtin_amdgcn_readlane((uint32_t)(eq >> 32), L);
        uint64_t rest = ((uint64_t)ehi << 32) | elo;  // the routes of e, ascending
        for (int i = 0; i < skip; ++i) rest &= rest - 1;
        for (int q0 = 0; q0 < b && rest; q0 += 8) {  // uniform
            int rr[8];
            float ra[8];
            uint32_t valid = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                rr[i] = 0;
                ra[i] = 0.f;
                if (rest && q0 + i < b) {
                    const int q = __builtin_ctzll(rest);
                    rest &= rest - 1;
                    rr[i] = q;
                    ra[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), q));
                    valid |= 1u << i;
                }
            }
            down_rows<CB, MFMA, VQ>(e, H, I, Wd, p, vq, rr, ra, valid, part, dsm);
        }
        return;
    }
    // First round: counts, the block's expert, its rows (lane q holds row q).
    int nb = plan.counts[0];
    const int e = plan.block_expert[blk];
    int rv = plan.sorted_routes[(size_t)blk * b + min(lane, b - 1)];
    if (lane >= b) rv = plan.R;
    if (nb < 0 || nb > plan.max_blocks) {
        if (blk == 0 && blockIdx.x == 0 && tid == 0) atomicOr(err, DEVERR_BAD_COUNTS);
        nb = nb < 0 ? 0 : plan.max_blocks;
    }
    if (blk >= nb) return;
    if (e < 0 || e >= plan.E) {
        if (blockIdx.x == 0 && tid == 0) atomicOr(err, DEVERR_BAD_BLOCK_EXPERT);
        return;
    }
    // Second round: row checks and affinities (clamped addresses).
    const int rc = min(max(rv, 0), plan.R - 1);
    const int idv = plan.topk_ids[rc];
    const float av = topk_w[rc];
    const bool ok = rv >= 0 && rv < plan.R && idv == e;
    if (!ok && rv != plan.R && blockIdx.x == 0 && tid < MOE_WAVE) atomicOr(err, DEVERR_BAD_PLAN);
    const uint64_t m = __ballot(ok);
    for (int q0 = 0; q0 < b; q0 += 8) {  // uniform
        const uint32_t valid = (uint32_t)(m >> q0) & 0xFFu;
        if (!valid) continue;
        int rr[8];
        float ra[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = min(q0 + i, MOE_WAVE - 1);
            rr[i] = ((valid >> i) & 1) ? __builtin_amdgcn_readlane(rv, q) : 0;
            ra[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(av), q));
        }
        down_rows<CB, MFMA, VQ>(e, H, I, Wd, p, vq, rr, ra, valid, part, dsm);
    }
}

// ---------------------------------------------------------------------------
// y[t][col] = sum over the valid routes s of token t and the chunks c of
// part[t*k+s][c][col].  One wave per workgroup (column block, t): lane
// (row group g, float4 column c4), kCombCG column groups x kCombRG row
// groups.  Row group g adds rows g, g + kCombRG, ... (row = s*nchunk + c) in
// order -- every load of a batch issued before the first add -- then the row
// groups are combined by a butterfly over the lane bits above the column
// bits (xor 4, 8, 16, 32: a fixed order).  No LDS, no barrier.  Routes with
// an id outside [0, E) have no partial and add nothing.
constexpr int kCombCG = 4;
constexpr int kCombRG = MOE_WAVE / kCombCG;
constexpr int kCombBatch = 16;

__global__ void __launch_bounds__(MOE_WAVE)
combine_kernel(const int32_t* __restrict__ topk_ids, int M, int k, int E, int H, int nchunk,
               const float* __restrict__ part, float* __restrict__ y, FastDiv fchunk) {
    const int t = blockIdx.y;
    const int lane = threadIdx.x;
    const int cg = lane % kCombCG;
    const int rg = lane / kCombCG;
    const int col = (blockIdx.x * kCombCG + cg) * 4;
    const int rows = k * nchunk;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // The partial loads do not wait for the ids: rows are clamped into the
    // token's range and the rows of invalid routes (never written) are
    // dropped by a select once the ids have arrived.
    const float* src = part + (size_t)t * k * nchunk * H + min(col, H - 4);
    for (int row0 = rg; row0 < rows; row0 += kCombBatch * kCombRG) {
        float4 v[kCombBatch];
        int e[kCombBatch];
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const int rr = min(row0 + u * kCombRG, rows - 1);
            v[u] = *reinterpret_cast<const float4*>(src + (size_t)rr * H);
            e[u] = topk_ids[(size_t)t * k + fchunk.div(rr)];
        }
#pragma unroll
        for (int u = 0; u < kCombBatch; ++u) {
            const bool use = row0 + u * kCombRG < rows && e[u] >= 0 && e[u] < E;
            acc.x += use ? v[u].x : 0.f;
            acc.y += use ? v[u].y : 0.f;
            acc.z += use ? v[u].z : 0.f;
            acc.w += use ? v[u].w : 0.f;
        }
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

// Staged route group of the split gate/up: h rows of G routes in LDS, each
// padded to a whole number of float4 per thread (at most 32 KiB).
constexpr int gateup_group(int Q) { return Q <= 4 ? 4 : (Q <= 8 ? 2 : 1); }
constexpr size_t gateup_lds(int Q) {
    return (size_t)gateup_group(Q) * ((Q * MOE_WAVE * 2 + kThreads - 1) / kThreads) * kThreads * 16;
}

template <int Q, int CPW>
hipError_t gateup_q(const PlanArgs& plan, const float* h, int H, int I, const uint16_t* Wg, const uint16_t* Wu,
                    float* p, int32_t* err, hipStream_t stream) {
    constexpr int G = gateup_group(Q);
    const dim3 grid(plan.max_blocks, (I + kWaves * CPW - 1) / (kWaves * CPW));
    MOE_LAUNCH((gateup_dense_kernel<Q, CPW, G>), grid, dim3(kThreads), gateup_lds(Q), stream, plan, h,
               H, I, Wg, Wu, p, err);
    return hipGetLastError();
}

// Fused tiling: 8 waves, one gate/up channel per wave and chunk; three
// double-buffered chunks per workgroup (24 channels) up to H = 2048, one
// chunk (8 channels, no second buffer) up to H = 4096.  Narrow experts (one
// GPU's 96-channel share of a 768-channel expert under channel sharding, say)
// would leave most CUs idle: where one chunk per workgroup still gives at
// most one workgroup per CU, each workgroup takes one chunk, so that three
// times as many CUs stream.  (4-wave workgroups of 4 channels measured no
// faster on the 96-channel share: the routing prologue, not the stream, sets
// its time.)
constexpr int kFusedNW = 8;
constexpr int kFusedCPW = 1;
constexpr int kFusedFill = 256;  // workgroups that keep every CU of the device streaming
constexpr int fused_nch(int Q) { return Q <= 4 ? 3 : 1; }
int fused_nch_for(int Q, int I, int k) {
    constexpr int one = kFusedNW * kFusedCPW;  // channels of one chunk
    return (long long)k * ((I + one - 1) / one) <= kFusedFill ? 1 : fused_nch(Q);
}

template <int Q, int CQ, int NCH, int XG>
hipError_t fused_launch(const PlanArgs& plan, const RouteArgs& route, const float* h, const float* topk_w, int H,
                        int I, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, float* part, int32_t* err,
                        hipStream_t stream) {
    constexpr int range = kFusedNW * kFusedCPW * NCH;
    const int nrange = (I + range - 1) / range;
    const dim3 grid(plan.max_blocks, nrange);
    const dim3 block(kFusedNW * MOE_WAVE);
    if (H == 512 * Q && H == 2048 * CQ)
        MOE_LAUNCH((expert_fused_kernel<Q, CQ, kFusedNW, kFusedCPW, NCH, true, XG>), grid, block, 0, stream,
                   plan, route, h, topk_w, H, I, Wg, Wu, Wd, part, nrange, err);
    else
        MOE_LAUNCH((expert_fused_kernel<Q, CQ, kFusedNW, kFusedCPW, NCH, false, XG>), grid, block, 0, stream,
                   plan, route, h, topk_w, H, I, Wg, Wu, Wd, part, nrange, err);
    return hipGetLastError();
}

template <int Q, int CQ, int XG>
hipError_t fused_q(const PlanArgs& plan, const RouteArgs& route, const float* h, const float* topk_w, int H, int I,
                   const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, float* part, int32_t* err,
                   hipStream_t stream) {
    if constexpr (fused_nch(Q) > 1) {
        if (fused_nch_for(Q, I, plan.k) == 1)
            return fused_launch<Q, CQ, 1, XG>(plan, route, h, topk_w, H, I, Wg, Wu, Wd, part, err, stream);
    }
    return fused_launch<Q, CQ, fused_nch(Q), XG>(plan, route, h, topk_w, H, I, Wg, Wu, Wd, part, err, stream);
}

}  // namespace

bool dense_uses_fused(int M, int H) { return M == 1 && H <= 4096; }

int dense_chunks(int M, int H, int I, int k) {
    if (dense_uses_fused(M, H)) {
        const int range = kFusedNW * kFusedCPW * fused_nch_for((H + 511) / 512 <= 4 ? 4 : 8, I, k);
        return (I + range - 1) / range;
    }
    return down_chunks(I);
}

int down_chunks(int) { return 1; }

hipError_t launch_expert_fused(const PlanArgs& plan, const float* h, const float* topk_w, int H, int I,
                               const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, float* part, int32_t* err,
                               hipStream_t stream) {
    const int Q = (H + 511) / 512;
    const RouteArgs none{};
    if (Q <= 4) return fused_q<4, 1, 0>(plan, none, h, topk_w, H, I, Wg, Wu, Wd, part, err, stream);
    if (Q <= 8) return fused_q<8, 2, 0>(plan, none, h, topk_w, H, I, Wg, Wu, Wd, part, err, stream);
    return hipErrorInvalidValue;  // H > 4096: the register tile would spill; the split schedule is used
}

bool decode_fused_ok(int H, int E, int k, int nslices) {
    return dense_uses_fused(1, H) && E <= kRouteMaxE && k <= MOE_WAVE && nslices >= 1 && nslices <= kRouteSlices;
}

hipError_t launch_decode_fused(const PlanArgs& plan, const RouteArgs& route, const float* h, int H, int I,
                               const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, float* part, int32_t* err,
                               hipStream_t stream) {
    if (!decode_fused_ok(H, plan.E, plan.k, route.nslices) || plan.R != plan.k || plan.max_blocks != plan.k)
        return hipErrorInvalidValue;
    const int Q = (H + 511) / 512;
    // experts in groups of 64: 2 groups up to 128 experts, else 8
    if (plan.E <= 2 * MOE_WAVE)
        return Q <= 4 ? fused_q<4, 1, 2>(plan, route, h, nullptr, H, I, Wg, Wu, Wd, part, err, stream)
                      : fused_q<8, 2, 2>(plan, route, h, nullptr, H, I, Wg, Wu, Wd, part, err, stream);
    return Q <= 4 ? fused_q<4, 1, 8>(plan, route, h, nullptr, H, I, Wg, Wu, Wd, part, err, stream)
                  : fused_q<8, 2, 8>(plan, route, h, nullptr, H, I, Wg, Wu, Wd, part, err, stream);
}

hipError_t launch_gateup_dense(const PlanArgs& plan, const float* h, int H, int I, const uint16_t* Wg,
                               const uint16_t* Wu, float* p, int32_t* err, hipStream_t stream) {
    const int Q = (H + 511) / 512;
    if (Q <= 1) return gateup_q<1, 2>(plan, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 2) return gateup_q<2, 2>(plan, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 4) return gateup_q<4, 2>(plan, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 8) return gateup_q<8, 2>(plan, h, H, I, Wg, Wu, p, err, stream);
    if (Q <= 16) return gateup_q<16, 1>(plan, h, H, I, Wg, Wu, p, err, stream);
    return hipErrorInvalidValue;
}

namespace {
template <int CB, bool MFMA>
hipError_t down_cb(const PlanArgs& plan, int H, int I, const uint16_t* Wd, const float* p, const float* topk_w,
                   float* part, int32_t* err, hipStream_t stream, const VqP* vq, const AlignOut* align) {
    const size_t lds = (size_t)kDownStage * 8 * sizeof(float);
    const dim3 grid((H + CB - 1) / CB, plan.max_blocks);
    const VqP v = vq ? *vq : VqP{};
    const AlignOut a = align ? *align : AlignOut{};
    if (vq && align)
        MOE_LAUNCH((down_kernel<CB, MFMA, true, true>), grid, dim3(kThreads), lds, stream, plan, H, I, Wd, p, topk_w,
                   part, err, v, a);
    else if (vq)
        MOE_LAUNCH((down_kernel<CB, MFMA, true, false>), grid, dim3(kThreads), lds, stream, plan, H, I, Wd, p, topk_w,
                   part, err, v, a);
    else
        MOE_LAUNCH((down_kernel<CB, MFMA, false, false>), grid, dim3(kThreads), lds, stream, plan, H, I, Wd, p,
                   topk_w, part, err, v, a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_down(const PlanArgs& plan, int H, int I, const uint16_t* Wd, const float* p, const float* topk_w,
                       float* part, int32_t* err, hipStream_t stream, const VqP* vq, const AlignOut* align) {
    if ((vq && (!vq->vp || vq->ny < 1)) || (align && (!vq || plan.R > MOE_WAVE || !align->sorted_routes ||
                                                      !align->block_expert || !align->counts)))
        return hipErrorInvalidValue;
    // 256-column blocks on the matrix cores when that still gives two
    // workgroups per CU, else 128-column blocks on the vector ALUs (few
    // experts: there the MFMA pass measured slower, 20.4 vs 19.0 us on four
    // tokens of top-8 over 128 experts, 2048 x 768, while on 21 tokens the
    // 256-column MFMA pass took 46.3 us against 54.4 us)
    if ((size_t)plan.max_blocks * ((H + 255) / 256) >= 512)
        return down_cb<256, true>(plan, H, I, Wd, p, topk_w, part, err, stream, vq, align);
    return down_cb<128, false>(plan, H, I, Wd, p, topk_w, part, err, stream, vq, align);
}

hipError_t launch_combine(const int32_t* topk_ids, int M, int k, int E, int H, int nchunk, const float* part, float* y,
                          hipStream_t stream) {
    const dim3 grid((H / 4 + kCombCG - 1) / kCombCG, M);
    MOE_LAUNCH(combine_kernel, grid, dim3(MOE_WAVE), 0, stream, topk_ids, M, k, E, H, nchunk, part, y,
               FastDiv((uint32_t)nchunk));
    return hipGetLastError();
}

}  // namespace moe

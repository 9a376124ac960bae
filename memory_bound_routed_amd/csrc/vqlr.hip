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
constexpr int kZBatch = 16;

// A code word of D bf16 values (D = 2, 4 or 8), loaded and kept in LDS as one
// 4-, 8- or 16-byte word.
template <int D> struct CodeWord;
template <> struct CodeWord<8> { typedef uint4 T; };
template <> struct CodeWord<4> { typedef uint2 T; };
template <> struct CodeWord<2> { typedef uint32_t T; };
__device__ __forceinline__ void unpack_cw(const uint4 v, float (&f)[8]) { unpack8(v, f); }
__device__ __forceinline__ void unpack_cw(const uint2 v, float (&f)[4]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
}
__device__ __forceinline__ void unpack_cw(const uint32_t v, float (&f)[2]) { f[0] = bf16_lo(v); f[1] = bf16_hi(v); }
__device__ __forceinline__ uint4 zero_cw(uint4) { return make_uint4(0u, 0u, 0u, 0u); }

// RM consecutive low-rank coefficients (bf16) of one lane in (RM + 1) / 2
// 32-bit words, loaded as one 2-, 4-, 8- or 16-byte word.
template <int RM>
struct Coef {
    uint32_t w[(RM + 1) / 2];
    __device__ __forceinline__ void load(const uint16_t* p) {
        if constexpr (RM == 1) {
            w[0] = __builtin_nontemporal_load(p);
        } else if constexpr (RM == 2) {
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
        } else if constexpr (RM == 4) {
            typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
            w[0] = v.x; w[1] = v.y;
        } else {
            const uint4 v = load_stream16(p);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        }
    }
    __device__ __forceinline__ float get(int m) const { return (m & 1) ? bf16_hi(w[m >> 1]) : bf16_lo(w[m >> 1]); }
};
__device__ __forceinline__ uint2 zero_cw(uint2) { return make_uint2(0u, 0u); }
__device__ __forceinline__ uint32_t zero_cw(uint32_t) { return 0u; }

// Overflow workgroups: runs of two or more routes (in block order, the first
// kOverflow of them) share their routes with one more workgroup, which takes
// the odd-numbered routes of the run while the run's own workgroup takes the
// even-numbered ones, so that an expert routed twice ends with the others.
constexpr int kOverflow = 4;

// Per lane: whether plan block bb (< nb) starts a run of at least two routes.
// A well-formed plan fills a run's first block first, so its row 1 is a route
// exactly then (one-row blocks: the next block has the same expert).  Both
// workgroups of a run evaluate this on the same plan, so they agree.
__device__ __forceinline__ bool starts_multi_run(const PlanArgs& plan, int bb, int nb) {
    const int bc = min(max(bb, 0), plan.max_blocks - 1);
    const int e = plan.block_expert[bc];
    const int ep = plan.block_expert[max(bc - 1, 0)];
    const int en = plan.block_expert[min(bc + 1, plan.max_blocks - 1)];
    const int r1 = plan.sorted_routes[(size_t)bc * plan.b + min(1, plan.b - 1)];
    const bool two = plan.b > 1 ? r1 != plan.R : (bc + 1 < nb && en == e);
    return bb >= 0 && bb < nb && (bc == 0 || ep != e) && e >= 0 && e < plan.E && two;
}

// Grid (plan blocks, ceil(I / (4*CPW))): workgroup (blk, cy) owns 4*CPW
// channels of the expert whose run of blocks starts at blk; wave w owns CPW
// of them.  Lane l owns VQ blocks 4*(l + 64*qb) .. +3 of length D (one 4-byte
// index load per channel; h elements 4*D*(l + 64*qb) .. +4D-1) and low-rank
// coordinates rho = RM*l .. RM*l + RM-1 (one load of RM bf16 per channel;
// r % 8 == 0 makes a lane's coordinates all valid or all past r).  The index maps and
// coefficients are kept in registers for every route of the expert; the two
// code books go to LDS.  A route needs its h row and its finished z vectors
// (the slice partials added in slice order) in LDS.
// Loads are ordered by what they wait for: the plan rows come first; then,
// before the index and coefficient stream, the row checks, the code books
// and h and the z partials of row 0 (the expert's first route in a
// well-formed plan, and at small batch usually its only one), since a load
// queued behind the stream would wait for all of it.  Further routes are
// staged rvq at a time.
template <int D, int QB, int RM, int CPW>
__global__ void __launch_bounds__(kThreads)
gateup_vqlr_kernel(PlanArgs plan, VqArgs vq, const float* __restrict__ h, int H, int I, int rvq, float* __restrict__ p,
                   int32_t* __restrict__ err) {
    typedef typename CodeWord<D>::T CW;
    constexpr int HPT = (QB * 64 * D + kThreads - 1) / kThreads;  // float4 of one h row per thread (H <= QB * 256 * D)
    constexpr int ZPT = RM > 2 ? RM / 2 : 1;   // (projection, rho) items of one route per thread
    __shared__ CW book[2][256];
    extern __shared__ __align__(16) float dyn[];
    float* hsm = dyn;                       // [rvq][H]
    float* zsm = dyn + (size_t)rvq * H;     // [kRT][2][r]
    const int b = plan.b;
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const bool ovf = (int)blockIdx.x >= plan.max_blocks;  // an overflow workgroup
    int blk = blockIdx.x;
    if (ovf) {  // find the run: the (x - max_blocks)-th block starting a run of two or more routes
        int nbo = plan.counts[0];
        nbo = nbo < 0 ? 0 : min(nbo, plan.max_blocks);
        int o = (int)blockIdx.x - plan.max_blocks;
        blk = -1;
        for (int c0 = 0; c0 < nbo; c0 += MOE_WAVE) {  // uniform
            const uint64_t m = __ballot(starts_multi_run(plan, c0 + lane, nbo));
            const int c = __popcll(m);
            if (o < c) {
                uint64_t mm = m;
                for (int i = 0; i < o; ++i) mm &= mm - 1;
                blk = c0 + __builtin_ctzll(mm);
                break;
            }
            o -= c;
        }
        if (blk < 0) return;  // fewer such runs than overflow workgroups (uniform)
    }
    const int sp = ovf ? 1 : 0;  // this workgroup's first route of the run

    // Round 1: counts, the previous, this and the next block's expert, the
    // block's rows.
    int nb = plan.counts[0];
    const int e = plan.block_expert[blk];
    const int eprev = blk > 0 ? plan.block_expert[blk - 1] : -1;
    const int enext = plan.block_expert[min(blk + 1, plan.max_blocks - 1)];  // checked against nb below
    int rv = plan.sorted_routes[(size_t)blk * b + min(lane, b - 1)];
    if (lane >= b) rv = plan.R;
    if (nb < 0 || nb > plan.max_blocks) {
        if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) atomicOr(err, DEVERR_BAD_COUNTS);
        nb = nb < 0 ? 0 : plan.max_blocks;
    }
    if (blk >= nb) return;
    if (e < 0 || e >= plan.E) {
        if (!ovf && blockIdx.y == 0 && tid == 0) atomicOr(err, DEVERR_BAD_BLOCK_EXPERT);
        return;
    }
    if (eprev == e) return;  // not the first block of the expert's run (uniform)
    // A run's own workgroup shares it if it is among the first kOverflow runs
    // of two or more routes (rank over the blocks before it).
    bool split = ovf;
    if (!ovf && starts_multi_run(plan, blk, min(max(nb, 0), plan.max_blocks))) {
        int rank = 0;
        for (int c0 = 0; c0 < blk; c0 += MOE_WAVE)  // uniform
            rank += __popcll(__ballot(c0 + lane < blk && starts_multi_run(plan, c0 + lane, nb)));
        split = rank < kOverflow;
    }
    const int nbk = H / D;  // VQ blocks per channel
    const int r = vq.r;
    const int H4 = H / 4;
    const int j0 = (blockIdx.y * kWaves + wave) * CPW;
    const bool active = j0 < I;  // inactive waves still take part in the barriers

    // Round 2 (clamped, always-valid addresses).
    const int idv = plan.topk_ids[min(max(rv, 0), plan.R - 1)];
    // (the argument struct's arrays are indexed by compile-time constants or
    // through a select: a run-time index would load the pointer from the
    // kernel-argument segment with a vector load)
    const int r0 = __builtin_amdgcn_readlane(rv, min(sp, MOE_WAVE - 1));  // row sp: the run's route sp if rows 0..sp are routes
    const int t0 = plan.fk.div(min(max(r0, 0), plan.R - 1));
    CW bk[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + kThreads * u;
        bk[u] = *reinterpret_cast<const CW*>(vq.B[i >> 8] + (size_t)min(i & 255, vq.K - 1) * D);
    }
    float4 h0[HPT];
#pragma unroll
    for (int v = 0; v < HPT; ++v)
        h0[v] = reinterpret_cast<const float4*>(h + (size_t)t0 * H)[min(tid + kThreads * v, H4 - 1)];
    float zx[ZPT][kZBatch];
#pragma unroll
    for (int w = 0; w < ZPT; ++w) {
        const int it = min(tid + kThreads * w, 2 * r - 1);
        const int P = it >= r ? 1 : 0, rho = it - P * r;
#pragma unroll
        for (int u = 0; u < kZBatch; ++u)
            zx[w][u] = (P ? vq.zpart[1] : vq.zpart[0])[((size_t)min(u, vq.zslices - 1) * vq.M + t0) * r + rho];
    }

    __builtin_amdgcn_sched_barrier(0);  // keeps the loads above ahead of the stream below

    // The index and coefficient stream.
    uint32_t jw[2][CPW][QB];
    Coef<RM> cw[2][CPW];  // bf16 patterns, converted (and masked) where used
    const int rl = r / RM;  // lanes holding coefficients (r % 8 == 0, RM <= 8)
#pragma unroll
    for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int j = min(j0 + c, I - 1);
            const uint8_t* jrow = vq.J[P] + ((size_t)e * I + j) * nbk;
            const uint16_t* crow = vq.C[P] + ((size_t)e * I + j) * r;
            // Unconditional loads of clamped addresses, used as loaded: a
            // select here would let the compiler put the load in a branch,
            // which is waited for at the branch's end, one load at a time.
            // Lanes past the last block or coordinate are masked where used.
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int b4 = 4 * (lane + MOE_WAVE * qb);
                jw[P][c][qb] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(jrow + min(b4, nbk - 4)));
            }
            cw[P][c].load(crow + RM * min(lane, rl - 1));
        }

    // Round 2 into LDS (in the stream's basic block, so that nothing moves
    // these loads behind it): the code books, and slot 0 with row 0's h and z.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + kThreads * u;
        book[i >> 8][i & 255] = (i & 255) < vq.K ? bk[u] : zero_cw(bk[u]);
    }
#pragma unroll
    for (int v = 0; v < HPT; ++v)  // unconditional (clamped duplicates store the same value)
        reinterpret_cast<float4*>(hsm)[min(tid + kThreads * v, H4 - 1)] = h0[v];
#pragma unroll
    for (int w = 0; w < ZPT; ++w) {
        const int it = tid + kThreads * w;
        float z = 0.f;
#pragma unroll
        for (int u = 0; u < kZBatch; ++u) z += u < vq.zslices ? zx[w][u] : 0.f;  // slice order
        if (it < 2 * r) {
            const int P = it >= r ? 1 : 0, rho = it - P * r;
            for (int sl = kZBatch; sl < vq.zslices; ++sl) z += (P ? vq.zpart[1] : vq.zpart[0])[((size_t)sl * vq.M + t0) * r + rho];
            zsm[it] = z;
        }
    }
    auto rows_ok = [&](int rvx, int idx) {
        const bool ok = rvx >= 0 && rvx < plan.R && idx == e;
        if (!ok && rvx != plan.R && wave == 0 && !ovf && blockIdx.y == 0) atomicOr(err, DEVERR_BAD_PLAN);
        return __ballot(ok);
    };
    uint64_t todo = rows_ok(rv, idv);
    __syncthreads();

    // One route from LDS slot i: o_P[j] = C_e[j] . z + sum over blocks of the
    // selected code words applied to h's blocks, then p = SiLU(o_gate) * o_up.
    auto compute = [&](int i, int route) {
        float acc[2][CPW];
#pragma unroll
        for (int P = 0; P < 2; ++P)
#pragma unroll
            for (int c = 0; c < CPW; ++c) acc[P][c] = 0.f;
        if (lane < rl) {
#pragma unroll
            for (int P = 0; P < 2; ++P) {
                float z[RM];
                const float* zr = zsm + (i * 2 + P) * r + RM * lane;
#pragma unroll
                for (int m = 0; m < RM; ++m) z[m] = zr[m];
#pragma unroll
                for (int c = 0; c < CPW; ++c)
#pragma unroll
                    for (int m = 0; m < RM; ++m) acc[P][c] = fmaf(cw[P][c].get(m), z[m], acc[P][c]);
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int b4 = 4 * (lane + MOE_WAVE * qb);
            if (b4 >= nbk) continue;
            const float4* hr = reinterpret_cast<const float4*>(hsm + (size_t)i * H + b4 * D);
            float hv[4 * D];
#pragma unroll
            for (int v = 0; v < D; ++v) {
                const float4 x = hr[v];
                hv[4 * v] = x.x; hv[4 * v + 1] = x.y; hv[4 * v + 2] = x.z; hv[4 * v + 3] = x.w;
            }
#pragma unroll
            for (int P = 0; P < 2; ++P)
#pragma unroll
                for (int c = 0; c < CPW; ++c)
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        float cw[D];
                        unpack_cw(book[P][(jw[P][c][qb] >> (8 * x)) & 255u], cw);
#pragma unroll
                        for (int y = 0; y < D; ++y) acc[P][c] = fmaf(cw[y], hv[D * x + y], acc[P][c]);
                    }
        }
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const float og = wave_sum(acc[0][c]);
            const float ou = wave_sum(acc[1][c]);
            if (lane == 0 && j0 + c < I) p[(size_t)route * I + j0 + c] = silu_mul(og, ou);
        }
    };

    // The routes of the run in order (the first block's valid rows, then the
    // following blocks'): all of them, or -- for a shared run -- every other
    // one from sp.  Row sp's h and z are in slot 0 already if rows 0..sp of
    // the first block are routes; other routes are staged rvq at a time.
    const uint64_t lowmask = (2ull << sp) - 1;
    bool pre = sp < b && (todo & lowmask) == lowmask;
    int bb = blk, n = 0;
    for (;;) {
        if (!todo) {
            if (++bb >= nb || (bb == blk + 1 ? enext : plan.block_expert[bb]) != e) break;
            int rv2 = plan.sorted_routes[(size_t)bb * b + min(lane, b - 1)];
            if (lane >= b) rv2 = plan.R;
            todo = rows_ok(rv2, plan.topk_ids[min(max(rv2, 0), plan.R - 1)]);
            rv = rv2;
            continue;
        }
        // the next routes of this workgroup, at most rvq, the first possibly in slot 0
        int rt[kRT], rq[kRT];
        int nr = 0;
#pragma unroll
        for (int i = 0; i < kRT; ++i) {
            rt[i] = -1;
            rq[i] = -1;
        }
        while (todo && nr < rvq) {  // uniform
            const int q = __builtin_ctzll(todo);
            todo &= todo - 1;
            const bool mine = !split || (n & 1) == sp;
            ++n;
            if (!mine) continue;
#pragma unroll
            for (int i = 0; i < kRT; ++i)
                if (i == nr) {
                    rt[i] = __builtin_amdgcn_readlane(rv, q);
                    rq[i] = q;
                }
            ++nr;
        }
        if (nr == 0) continue;
        const bool have0 = pre && bb == blk && rq[0] == sp;  // slot 0 already holds the first
        pre = false;
        if (!have0 || nr > 1) {
            __syncthreads();  // the previous routes' slots are no longer read
#pragma unroll
            for (int i = 0; i < kRT; ++i) {
                if (i >= nr || (i == 0 && have0)) continue;
                const float4* src = reinterpret_cast<const float4*>(h + (size_t)plan.fk.div(rt[i]) * H);
                float4* dst = reinterpret_cast<float4*>(hsm + (size_t)i * H);
                for (int c4 = tid; c4 < H4; c4 += kThreads) dst[c4] = src[c4];
            }
            for (int it = tid; it < nr * 2 * r; it += kThreads) {
                const int i = it / (2 * r), rem = it - i * 2 * r, P = rem / r, rho = rem - P * r;
                if (i == 0 && have0) continue;
                int ti = 0;
#pragma unroll
                for (int ii = 0; ii < kRT; ++ii)
                    if (ii == i) ti = plan.fk.div(rt[ii]);
                float z = 0.f;
                for (int sl0 = 0; sl0 < vq.zslices; sl0 += kZBatch) {
                    float x[kZBatch];
#pragma unroll
                    for (int u = 0; u < kZBatch; ++u)
                        x[u] = (P ? vq.zpart[1] : vq.zpart[0])[((size_t)min(sl0 + u, vq.zslices - 1) * vq.M + ti) * r + rho];
#pragma unroll
                    for (int u = 0; u < kZBatch; ++u) z += sl0 + u < vq.zslices ? x[u] : 0.f;  // slice order
                }
                zsm[it] = z;
            }
            __syncthreads();
        }
        if (!active) continue;
#pragma unroll
        for (int i = 0; i < kRT; ++i) {
            if (i >= nr) break;
            compute(i, rt[i]);
        }
    }
}

template <int D, int QB, int RM, int CPW>
hipError_t vq_launch(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p, int32_t* err,
                     hipStream_t stream) {
    // x: the plan blocks, then the overflow workgroups
    const dim3 grid(plan.max_blocks + kOverflow, (I + kWaves * CPW - 1) / (kWaves * CPW));
    const int rvq = H <= 4096 ? kRT : 2;  // staged h rows: <= 64 KiB
    const size_t lds = ((size_t)rvq * H + (size_t)kRT * 2 * vq.r) * sizeof(float);
    MOE_LAUNCH((gateup_vqlr_kernel<D, QB, RM, CPW>), grid, dim3(kThreads), lds, stream, plan, vq, h, H, I, rvq, p, err);
    return hipGetLastError();
}

// Channels per wave: 8 for the smallest register tile (H <= 2048, r <= 64),
// else 4.
template <int D, int QB>
hipError_t vq_rm(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p, int32_t* err,
                 hipStream_t stream) {
    const int RM = (vq.r + 63) / 64;
    if (RM <= 1) return vq_launch<D, QB, 1, QB == 1 ? 8 : 4>(plan, vq, h, H, I, p, err, stream);
    if (RM <= 2) return vq_launch<D, QB, 2, 4>(plan, vq, h, H, I, p, err, stream);
    if (RM <= 4) return vq_launch<D, QB, 4, 4>(plan, vq, h, H, I, p, err, stream);
    if (RM <= 8) return vq_launch<D, QB, 8, 4>(plan, vq, h, H, I, p, err, stream);
    return hipErrorInvalidValue;
}

// Lane blocks: QB = ceil(H / D / 256) groups of four VQ blocks per lane.
template <int D>
hipError_t vq_qb(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p, int32_t* err,
                 hipStream_t stream) {
    const int QB = (H / D + 255) / 256;
    if (QB <= 1) return vq_rm<D, 1>(plan, vq, h, H, I, p, err, stream);
    if (QB <= 2) return vq_rm<D, 2>(plan, vq, h, H, I, p, err, stream);
    if (QB <= 4) return vq_rm<D, 4>(plan, vq, h, H, I, p, err, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gateup_vqlr(const PlanArgs& plan, const VqArgs& vq, const float* h, int H, int I, float* p,
                              int32_t* err, hipStream_t stream) {
    if (vq.K < 1 || vq.K > 256 || H % (8 * vq.d)) return hipErrorInvalidValue;
    if (vq.d == 8) return vq_qb<8>(plan, vq, h, H, I, p, err, stream);
    if (vq.d == 4) return vq_qb<4>(plan, vq, h, H, I, p, err, stream);
    if (vq.d == 2) return vq_qb<2>(plan, vq, h, H, I, p, err, stream);
    return hipErrorInvalidValue;
}

}  // namespace moe

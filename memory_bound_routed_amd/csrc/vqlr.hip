// VQ + low-rank gate/up projections (page "A Multi-Engine Dataflow for MoE
// Decoding on Scratchpad-Based Tensor Accelerators", Sec. 2.3 blockwise VQ,
// Sec. 3.1 Eq. 1 hybrid representation, Sec. 4.2 shared-projection reuse,
// cross-expert gather batching and joint accumulation).
//
// For projection P of channel j of expert e and token t:
//     o_P[j] = sum_rho C_P,e[j][rho] z_P[t][rho]  +  sum_b T_P[t][b][J_P,e[j][b]]
// with z_P = D_P^T h (computed once per token by the GEMV-partials tiles,
// summed here over their row slices in slice order) and the projection code
// book T_P[t][b][c] = h_b . B_P[c] of the page, h_b the b-th length-d block
// of h.  An fp32 T is 256 KiB per token and projection at H = 2048, more than
// a CU's LDS, and a bf16 T is not accurate enough; so T is cut into slices of
// 64 blocks (64 KiB) and one workgroup owns one (route, projection, slice)
// -- or, when there are more of them than fit on the device at once, a few
// slices of one (route, projection) taken in turn: for each it forms its
// slice of T on the matrix cores and then adds, for every
// channel of the route's expert, T[b][J[j][b]] over its 64 blocks -- one
// 4-byte LDS read and one add per index byte, where applying each code word
// to h directly takes a 4d-byte read and d FMAs.  Each slice workgroup also
// adds the low-rank term of a share of the channels (16-channel chunks dealt
// out over the slices) and stores one partial per (route, projection,
// channel): the sum, in slice order, of the slices it took.  The down
// launch (up to 64 routes) or a finishing kernel (more) adds a route's
// partial rows in row order and forms p = SiLU(o_gate) * o_up (the joint
// accumulation of the page, split across the kernels).
//
// The grid is route-major (one token's use of an expert per workgroup set):
// a route never waits for another route of its expert, and an expert routed
// by two tokens is read twice, the second time mostly from the caches.  All
// slices of one (route, projection) run on one XCD (grid x padded to a
// multiple of 8; workgroups are dealt to the XCDs round robin by linear id),
// so the 128-byte lines of J they share are fetched into one L2.
#include "align_device.h"
#include "device_common.h"
#include "launch.h"
#include "topk_device.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 64;      // VQ blocks per slice of T
constexpr int kCodes = 256;     // code words addressable by a uint8 index (entries >= K are zero)
constexpr int kTRow = kCodes + 4;  // T row stride in floats: the padding puts the four row groups of a
                                   // matrix-core result on different LDS banks
constexpr int kMaxR = 512;      // largest low-rank rank
constexpr int kZBatch = 8;      // z slice partials loaded ahead of the stream

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// fp32 -> bf16 pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// x = hi + lo + O(2^-18 |x|), hi and lo bf16 patterns.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
    hi = bf16_rne(x);
    lo = bf16_rne(x - __uint_as_float(hi << 16));
}

// The index and coefficient streams are read through buffer resources over
// the route's expert (its index rows, its coefficient rows).  A part that is
// not valid is read from the resource's end, which returns zeros without a
// memory access, so no select follows the load: a select on a loaded value
// is placed next to the load, and the compiler waits for the load there.
// Cache policy of the index and coefficient loads: the default (cached), so
// that the second of two slices sharing a 128-byte index line, or a second
// route of the expert on the same XCD, finds it in L2 (non-temporal loads
// measured 24.5 against 22.5 us at 16 tokens, equal at 4 and 8).
constexpr int kStreamAux = 0;

// One lane's quarter of a channel's slice segment: 16 index bytes (blocks
// 16 q .. 16 q + 15 of the slice) as 4 words, at byte offset `off` of the
// index resource `jr` (`end` bytes long); `vb` is the number of valid bytes
// (0, 8 or 16; the rest read as index 0 of a zero row of T).
template <int JW>
__device__ __forceinline__ uint4 load_quarter(__amdgpu_buffer_rsrc_t jr, int off, int end, int vb) {
    if constexpr (JW == 16) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(jr, vb >= 16 ? off : end, 0, kStreamAux);
        return make_uint4(x.x, x.y, x.z, x.w);
    } else {
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(jr, vb >= 8 ? off : end, 0, kStreamAux);
        const u32x2_t b = __builtin_amdgcn_raw_buffer_load_b64(jr, vb >= 16 ? off + 8 : end, 0, kStreamAux);
        return make_uint4(a.x, a.y, b.x, b.y);
    }
}

// 8 low-rank coefficients (16 bytes) at byte offset `off` of the coefficient
// resource `cr` (`end` bytes long), or zeros when !ok.
__device__ __forceinline__ uint4 load_coef(__amdgpu_buffer_rsrc_t cr, int off, int end, bool ok) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(cr, ok ? off : end, 0, kStreamAux);
    return make_uint4(x.x, x.y, x.z, x.w);
}

// The lane's 16 reads T[16 q + i][byte i] of a quarter (gather_issue) and
// their sum in block order (gather_sum); split so that the reads of the next
// pass can go out before this pass is summed.  The words pass through an
// empty asm so that the addresses are formed here, next to their reads (else
// the compiler forms all of them early and holds them in registers, leaving
// none for reads in flight).
__device__ __forceinline__ void gather_issue(const float* T, uint4 win, int q, float (&v)[16]) {
    uint32_t w[4] = {win.x, win.y, win.z, win.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(w[k]));
    const float* Tq = T + q * 16 * kTRow;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = Tq[i * kTRow + ((w[i >> 2] >> (8 * (i & 3))) & 255u)];
}
__device__ __forceinline__ float gather_sum(const float (&v)[16]) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += v[i];
    return acc;
}
__device__ __forceinline__ float gather_quarter(const float* T, uint4 win, int q) {
    float v[16];
    gather_issue(T, win, q, v);
    return gather_sum(v);
}

// x through an empty asm: the compiler cannot see that its value is the
// argument's.
__device__ __forceinline__ int opaque_int(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

constexpr int kVqWaves = 8;                    // waves of a gate/up workgroup (two per SIMD)
constexpr int kVqThreads = kVqWaves * MOE_WAVE;
constexpr int kNTiles = 16 / kVqWaves;         // 16-code tiles of T formed per wave

// Slice workgroup owning the low-rank term of the 16-channel chunk c = kVqWaves p + w
// (pass p, wave w): (p + c) mod nslice, so that a wave's owned passes are
// spread over the slices.
__device__ __forceinline__ int lr_owner(int c, int nslice) { return (c + c / kVqWaves) % nslice; }

constexpr int kPassCh = 16 * kVqWaves;         // channels per pass (16 per wave, 4 lanes each)
constexpr int kRegPasses = 6;                  // passes held in registers (the rest are loaded one at a time)
constexpr int kLrPre = 4;                      // owned low-rank chunks whose coefficients are requested up front
constexpr int kAhead = 2;                      // index passes requested before T, then kept in flight ahead of the gathers
constexpr int kOutPer = (kRegPasses + 3) / 4;  // passes a lane stores (lane q of a quad: passes 4 m + q)
constexpr int kVqResident = 512;               // gate/up workgroups resident at once (2 per CU x 256 CUs)

// Grid (x = 2 * route + projection, padded to a multiple of 8; y = first T
// slice, the workgroup then takes slices y + gridDim.y, ... in turn).  For
// each slice s, workgroup (r, P, y) computes slice s of projection P for
// route r:
//  * T[b][c] = h_b . B_P[c] for the slice's 64 blocks b and the 256 code
//    words c, on the matrix cores: [blocks x (h_hi | h_lo)] times
//    [(B | B) x codes] with bf16 operands (h = h_hi + h_lo to 2^-18, B is
//    bf16), fp32 accumulation; wave w forms codes 32 w .. 32 w + 31;
//  * lane l of wave w, in pass p, takes channel 128 p + 16 w + l / 4 and the
//    16 blocks 16 (l % 4) .. +15 of the slice (its 16 index bytes, one load),
//    sums T over them, and (if the slice owns the channel's chunk) adds its
//    quarter of the low-rank term; the quad's four sums are then added in a
//    fixed order.
// Eight waves (two per SIMD): the gathers are random 4-byte LDS reads, whose
// bank conflicts make them the kernel's largest cost (about 7 cycles per
// 64-lane read on this chip, against about 3 without conflicts), and a
// second wave per SIMD fills the gaps of the first.  Everything that does
// not depend on the route's expert (h, z, the code book) is requested
// together with its id; the index and coefficient stream follows as soon as
// the id has arrived.  ROUTE (the decode step):
// there is no id to read; the workgroup routes its token itself from the
// router's slice partials (route_token: the router's arithmetic, so the
// router's ids bit for bit), and the workgroup of the token's first route,
// gate, slice 0 stores the token's ids, weights and logits.
template <int D, int JW, bool LR, bool ROUTE>
__global__ void __launch_bounds__(kVqThreads)
gateup_vqt_kernel(const int32_t* __restrict__ topk_ids, int R, int k, FastDiv fk, int E, VqArgs vq,
                  const float* __restrict__ h, int H, int I, float* __restrict__ vp, int32_t* __restrict__ err,
                  SelRoute route) {
    static_assert(kNTiles * kVqWaves == 16 && kVqThreads <= 1024, "the 16 code tiles are dealt out evenly");
    __shared__ float T[kSlice * kTRow];
    __shared__ float zsm[kMaxR];
    __shared__ uint4 Aop[4 * MOE_WAVE];  // T's A operand words, M tile m at [m][lane]
    const int r = blockIdx.x >> 1;
    const int P = blockIdx.x & 1;
    const int s0 = blockIdx.y;   // first slice of this workgroup
    const int ny = gridDim.y;    // it takes slices s0, s0 + ny, ... < nslice in turn
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);  // uniform: the pass logic runs on scalars
    const int lane = tid % MOE_WAVE;
    const int g = lane / 16;   // MFMA K group / operand row group
    if (r >= R) return;  // grid padding

    const int nbk = H / D;                              // VQ blocks per channel
    const int nslice = (nbk + kSlice - 1) / kSlice;     // slices of T
    const int rr = vq.r;
    const int t = fk.div(r);
    const uint16_t* Cb = P ? vq.C[1] : vq.C[0];
    const uint16_t* Bb = P ? vq.B[1] : vq.B[0];
    const uint8_t* Jb = P ? vq.J[1] : vq.J[0];
    const float* zp = P ? vq.zpart[1] : vq.zpart[0];

    // Round 1: the route's expert; code-book operands; h operands of the
    // first slice; z partials.
    int e = ROUTE ? 0 : topk_ids[r];
    // (code-book and h operands through buffer resources: the parts a lane
    // does not use read zero from the resource's end)
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const int bend = vq.K * D * 2;
    const __amdgpu_buffer_rsrc_t br =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Bb), (short)0, bend, 0x00020000);
    uint4 bw[kNTiles];  // B operand words of N tiles kNTiles wave + u (code 16 (kNTiles wave + u) + lane % 16)
#pragma unroll
    for (int u = 0; u < kNTiles; ++u) {
        const int c = 16 * (kNTiles * wave + u) + lane % 16;
        if constexpr (D == 8) {
            const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(br, c < vq.K && g < 2 ? c * 16 : bend, 0, 0);
            bw[u] = make_uint4(a.x, a.y, a.z, a.w);
        } else if constexpr (D == 4) {
            const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(br, c < vq.K && g == 0 ? c * 8 : bend, 0, 0);
            bw[u] = make_uint4(a.x, a.y, a.x, a.y);
        } else {
            const uint32_t a = __builtin_amdgcn_raw_buffer_load_b32(br, c < vq.K && g == 0 ? c * 4 : bend, 0, 0);
            bw[u] = make_uint4(a, a, 0u, 0u);
        }
    }
    const int hend = H * 4;
    const __amdgpu_buffer_rsrc_t hr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(h + (size_t)t * H), (short)0, hend, 0x00020000);
    // h of block 16 m + lane % 16 of slice s (zero past the channel's blocks)
    auto load_h = [&](int s, int m, float (&hx)[D]) {
        const int L = min(kSlice, nbk - s * kSlice);
        const int b = 16 * m + lane % 16;
        const bool in = b < L && (D == 8 ? g < 2 : g == 0);
        const int off = (s * kSlice + b) * D * 4;
        if constexpr (D == 2) {
            const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(hr, in ? off : hend, 0, 0);
            hx[0] = __uint_as_float(a.x);
            hx[1] = __uint_as_float(a.y);
        } else {
#pragma unroll
            for (int x = 0; x < D; x += 4) {
                const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(hr, in ? off + 4 * x : hend, 0, 0);
                hx[x] = __uint_as_float(a.x); hx[x + 1] = __uint_as_float(a.y);
                hx[x + 2] = __uint_as_float(a.z); hx[x + 3] = __uint_as_float(a.w);
            }
        }
    };
    // z partials of coordinate rho = tid (the first kZBatch slices; threads
    // past r load nothing)
    // The A operand words of M tile m = wave (waves 0..3) for slice s: h of
    // block 16 m + lane % 16 split into hi + lo bf16, 8 bf16 of K group g,
    // formed once per workgroup and shared through LDS (the caller's barrier
    // publishes them).
    auto make_A = [&](const float (&hx)[D], int ln) {
        const int gg = ln / 16;
        uint32_t hi[D], lo[D];
#pragma unroll
        for (int x = 0; x < D; ++x) split_bf16(hx[x], hi[x], lo[x]);
        uint32_t k8[8];  // K slots 8 g .. 8 g + 7 (zero past 2 D)
        if constexpr (D == 8) {
#pragma unroll
            for (int x = 0; x < 8; ++x) k8[x] = gg == 0 ? hi[x] : lo[x];
        } else if constexpr (D == 4) {
#pragma unroll
            for (int x = 0; x < 4; ++x) { k8[x] = hi[x]; k8[4 + x] = lo[x]; }
        } else {
            k8[0] = hi[0]; k8[1] = hi[1]; k8[2] = lo[0]; k8[3] = lo[1];
            k8[4] = k8[5] = k8[6] = k8[7] = 0u;
        }
        Aop[wave * MOE_WAVE + ln] = make_uint4(k8[0] | (k8[1] << 16), k8[2] | (k8[3] << 16),
                                               k8[4] | (k8[5] << 16), k8[6] | (k8[7] << 16));
    };
    // T on the matrix cores from the A words in LDS; wave w forms codes
    // 16 kNTiles w .. + 16 kNTiles - 1.
    auto make_T = [&](int ln) {
        const int gg = ln / 16;
        uint4 aw[4];  // A operand words of M tile m: 8 bf16 of K group g
#pragma unroll
        for (int m = 0; m < 4; ++m) aw[m] = Aop[m * MOE_WAVE + ln];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int u = 0; u < kNTiles; ++u) {
                const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4_t d4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, aw[m]), __builtin_bit_cast(bf16x8_t, bw[u]), zero, 0, 0, 0);
                // lane holds T[16 m + 4 g + i][16 (kNTiles wave + u) + lane % 16]
                float* dst = T + (16 * m + 4 * gg) * kTRow + 16 * (kNTiles * wave + u) + ln % 16;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * kTRow] = d4[i];
            }
    };

    // h of the first slice, requested before the routing's loads (a wait
    // for it then does not wait for them too).
    float hx0[D];
    if (wave < 4) load_h(s0, wave, hx0);  // uniform
    // z partials of coordinate rho = tid (the first kZBatch slices; threads
    // past r load nothing)
    float zx[kZBatch];
#pragma unroll
    for (int u = 0; u < kZBatch; ++u) zx[u] = 0.f;
    if (LR && wave * MOE_WAVE < rr) {  // uniform: only the waves that hold coordinates load
#pragma unroll
        for (int u = 0; u < kZBatch; ++u)
            zx[u] = zp[((size_t)min(u, vq.zslices - 1) * vq.M + t) * rr + min(tid, rr - 1)];
    }
    RoutePart rp;
    if constexpr (ROUTE) route_token_load(route.part, route.bias, route.nslices, route.M, t, E, rp);
    // T of the first slice does not depend on the route: it is formed while
    // the routing's loads are in flight.
    if (wave < 4) make_A(hx0, lane);  // uniform
    __syncthreads();  // the A words written
    make_T(lane);
    if constexpr (ROUTE) {
        __shared__ RouteLds<kVqThreads> rl;
        const int slot = r - t * k;
        route_token_from<kVqThreads>(rp, route.part, route.bias, route.nslices, route.M, t, E, k,
                                     P == 0 && s0 == 0 && slot == 0, route.logits, route.ids, route.wts, rl, false);
        e = __builtin_amdgcn_readfirstlane(rl.sel_e[slot]);
    }
    if (e < 0 || e >= E) {  // an invalid route has no output (uniform)
        if (P == 0 && s0 == 0 && tid == 0) atomicOr(err, DEVERR_BAD_ROUTE_ID);
        return;
    }
    // The z partials pass through an empty asm here, after the routing: else
    // the compiler starts their sum next to their loads, and the wait for the
    // first of them delays the routing's own loads by a memory round trip.
#pragma unroll
    for (int u = 0; u < kZBatch; ++u) asm volatile("" : "+v"(zx[u]));

    const int npass = (I + kPassCh - 1) / kPassCh;
    const int jend = I * nbk;      // bytes of the expert's index rows
    const int cend = I * rr * 2;   // bytes of its coefficient rows
    const __amdgpu_buffer_rsrc_t jr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(Jb + (size_t)e * jend), (short)0, jend, 0x00020000);
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Cb + (size_t)e * I * rr), (short)0, cend, 0x00020000);
    // The index stream: pass p, lane quarter q of channel 128 p + 16 wave +
    // lane / 4 of slice s (channels past I read past the resource's end).
    auto load_pass = [&](int s, int p, int ln) {
        const int qq = ln % 4;
        const int L = min(kSlice, nbk - s * kSlice);  // valid blocks of slice s (> 0)
        const int vb = min(max(L - 16 * qq, 0), 16);
        const int j = kPassCh * p + 16 * wave + ln / 4;
        return load_quarter<JW>(jr, j * nbk + s * kSlice + 16 * qq, jend, p < npass ? vb : 0);
    };
    // the first slice's first passes go out as soon as the expert is known
    uint4 jq[kRegPasses];
#pragma unroll
    for (int p = 0; p < kAhead; ++p) jq[p] = load_pass(s0, p, lane);
    __builtin_amdgcn_sched_barrier(0);  // keeps the loads above ahead of what follows

    // z (slice partials in slice order) into LDS, read after the first
    // slice's barrier; coordinates past 256 and slices past kZBatch are
    // loaded here.
    if (LR && tid < rr) {
        float z = 0.f;
#pragma unroll
        for (int u = 0; u < kZBatch; ++u) z += u < vq.zslices ? zx[u] : 0.f;
        for (int sl = kZBatch; sl < vq.zslices; ++sl) z += zp[((size_t)sl * vq.M + t) * rr + tid];
        zsm[tid] = z;
    }
    for (int rho = tid + kVqThreads; LR && rho < rr; rho += kVqThreads) {
        float z = 0.f;
        for (int sl = 0; sl < vq.zslices; ++sl) z += zp[((size_t)sl * vq.M + t) * rr + rho];
        zsm[rho] = z;
    }
    for (int rho = rr + tid; rho < kMaxR; rho += kVqThreads) zsm[rho] = 0.f;  // read against zero coefficients

    // The workgroup's slices in turn (a grid of fewer slice rows than
    // slices when the routes would not otherwise fit on the device at
    // once): the routing, code-book, z and LDS set-up above is done once,
    // and a later slice's index, coefficient and h loads go out before the
    // barrier that waits for every wave to finish reading the previous T.
    float osum[kOutPer];  // per lane: the sum over the workgroup's slices of the passes it stores
#pragma unroll
    for (int m = 0; m < kOutPer; ++m) osum[m] = 0.f;
    for (int s = s0; s < nslice; s += ny) {  // uniform
        // The lane id through an empty asm: everything derived from it is
        // formed again per slice instead of being hoisted out of the loop
        // and held in registers across it.
        const int lane_s = opaque_int(lane);
        const int lane = lane_s;
        const int q = lane % 4;   // gather quarter
        const int L = min(kSlice, nbk - s * kSlice);  // valid blocks of this slice (> 0)
        const int vb = min(max(L - 16 * q, 0), 16);
        const bool first = s == s0;

        // Low-rank quarter of the lane's channel in an owned pass: coordinates
        // 64 c0 + 16 q + x, in rho order; the first 64 from the prefetched
        // coefficients, further ones loaded here.
        auto lr_dot = [&](const uint4 (&c)[2], int rho0, float acc) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float f[8];
                unpack8(c[u], f);
                const int rb = min(rho0 + 8 * u, kMaxR - 8);  // coefficients past r are zero
#pragma unroll
                for (int x = 0; x < 8; ++x) acc = fmaf(f[x], zsm[rb + x], acc);
            }
            return acc;
        };
        auto lr_rest = [&](int p, float acc) {  // coordinates 64 .. r - 1
            const int row = (kPassCh * p + 16 * wave + lane / 4) * rr;
            for (int c0 = 64; c0 < rr; c0 += 64) {
                const int rho0 = c0 + 16 * q;
                const uint4 c[2] = {load_coef(cr, (row + rho0) * 2, cend, rho0 < rr),
                                    load_coef(cr, (row + rho0 + 8) * 2, cend, rho0 + 8 < rr)};
                acc = lr_dot(c, rho0, acc);
            }
            return acc;
        };

        if (!first) {
#pragma unroll
            for (int p = 0; p < kAhead; ++p) jq[p] = load_pass(s, p, lane);
        }
        // The passes p < kRegPasses whose 16-channel chunk c = kVqWaves p +
        // wave this slice owns for the low-rank term: lane p of the wave
        // tests pass p, and the ballot is the wave's (uniform) mask.
        uint32_t own = 0;
        if (LR) {
            const int c = kVqWaves * lane + wave;
            own = (uint32_t)__builtin_amdgcn_ballot_w64(lane < min(npass, kRegPasses) && lr_owner(c, nslice) == s);
        }
        // The first kLrPre owned passes, and their coefficients: the lane's 16
        // of the first 64 coordinates, rho = 16 q .. 16 q + 15.
        int po[kLrPre];
        uint32_t own_rest = own;
#pragma unroll
        for (int u = 0; u < kLrPre; ++u) {
            po[u] = own_rest ? __builtin_ctz(own_rest) : -1;
            own_rest &= own_rest - 1;
        }
        uint4 cpre[kLrPre][2];
#pragma unroll
        for (int u = 0; u < kLrPre; ++u) {
            if constexpr (!LR) {
                cpre[u][0] = cpre[u][1] = make_uint4(0u, 0u, 0u, 0u);
                continue;
            }
            const int off = ((kPassCh * max(po[u], 0) + 16 * wave + lane / 4) * rr + 16 * q) * 2;
            const bool use = po[u] >= 0;
            cpre[u][0] = load_coef(cr, off, cend, use && 16 * q < rr);
            cpre[u][1] = load_coef(cr, off + 16, cend, use && 16 * q + 8 < rr);
        }
        __builtin_amdgcn_sched_barrier(0);  // every stream load goes out before the h loads below
        if (!first) {  // T of this slice (the first slice's was formed during the routing)
            if (wave < 4) {  // uniform
                float hx[D];
                load_h(s, wave, hx);
                make_A(hx, lane);
            }
            __syncthreads();  // the previous slice's T is no longer read; the A words written
            make_T(lane);
        }
        __syncthreads();  // T (and, the first time, z) written

        // The gathers, pass by pass as the index words arrive: a workgroup's
        // share of the stream takes about as long as T and the gathers
        // together, so the index request of pass p + kAhead goes out before
        // pass p is gathered (requested all at once, the requests stall the
        // wave until the memory system takes them, and the arithmetic waits
        // behind them).  The low-rank quarter of an owned pass (first 64
        // coordinates, from the prefetched coefficients) follows its gather;
        // coordinates past 64 are added after the loop, whose loads would
        // otherwise sit between the stream's.
        float acc[kRegPasses];
        float vlr[kLrPre];
#pragma unroll
        for (int u = 0; u < kLrPre; ++u) vlr[u] = 0.f;
        float gv[2][16];  // the T reads of passes p and p + 1
        gather_issue(T, jq[0], q, gv[0]);
#pragma unroll
        for (int p = 0; p < kRegPasses; ++p) {
            if (p + kAhead < kRegPasses) jq[p + kAhead] = load_pass(s, p + kAhead, lane);
            if (p + 1 < kRegPasses) gather_issue(T, jq[p + 1], q, gv[(p + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            acc[p] = p < npass ? gather_sum(gv[p & 1]) : 0.f;
#pragma unroll
            for (int u = 0; u < kLrPre; ++u) {
                if (po[u] != p) continue;  // wave-uniform
                vlr[u] = lr_dot(cpre[u], 16 * q, 0.f);
                if (rr <= 64) acc[p] += vlr[u];
            }
        }
        if (rr > 64) {
#pragma unroll
            for (int u = 0; u < kLrPre; ++u) {
                const int p = po[u];  // wave-uniform
                if (p < 0) continue;
                const float v = lr_rest(p, vlr[u]);
#pragma unroll
                for (int pp = 0; pp < kRegPasses; ++pp)
                    if (pp == p) acc[pp] += v;
            }
        }
        for (uint32_t m = own_rest; LR && m; m &= m - 1) {  // owned passes beyond the prefetched ones
            const int p = __builtin_ctz(m);
            const int off = ((kPassCh * p + 16 * wave + lane / 4) * rr + 16 * q) * 2;
            const uint4 c[2] = {load_coef(cr, off, cend, 16 * q < rr),
                                load_coef(cr, off + 16, cend, 16 * q + 8 < rr)};
            float v = lr_dot(c, 16 * q, 0.f);
            if (rr > 64) v = lr_rest(p, v);
#pragma unroll
            for (int pp = 0; pp < kRegPasses; ++pp)
                if (pp == p) acc[pp] += v;
        }
        // quad sums (q0 + q1) + (q2 + q3), in every lane of the quad; lane q of a
        // quad stores passes 4 m + q
#pragma unroll
        for (int p = 0; p < kRegPasses; ++p) {
            acc[p] += dpp<MOE_DPP_QUAD_XOR1>(acc[p]);
            acc[p] += dpp<MOE_DPP_QUAD_XOR2>(acc[p]);
        }
#pragma unroll
        for (int m = 0; m < kOutPer; ++m) {
            float v = acc[4 * m];
#pragma unroll
            for (int x = 1; x < 4; ++x)
                if (4 * m + x < kRegPasses) v = q == x ? acc[4 * m + x] : v;
            osum[m] = first ? v : osum[m] + v;  // the workgroup's slices in ascending order
        }
        for (int p = kRegPasses; p < npass; ++p) {  // further passes: indices loaded here
            const int j = kPassCh * p + 16 * wave + lane / 4;
            const uint4 w = load_quarter<JW>(jr, j * nbk + s * kSlice + 16 * q, jend, vb);
            float a = gather_quarter(T, w, q);
            if (LR && lr_owner(kVqWaves * p + wave, nslice) == s) {
                const int off = (j * rr + 16 * q) * 2;
                const uint4 c[2] = {load_coef(cr, off, cend, 16 * q < rr),
                                    load_coef(cr, off + 16, cend, 16 * q + 8 < rr)};
                float v = lr_dot(c, 16 * q, 0.f);
                if (rr > 64) v = lr_rest(p, v);
                a += v;
            }
            a += dpp<MOE_DPP_QUAD_XOR1>(a);
            a += dpp<MOE_DPP_QUAD_XOR2>(a);
            if (q == 0 && j < I) {  // added to the earlier slices' sum this thread stored
                float* o = vp + ((size_t)(r * ny + s0) * 2 + P) * I + j;
                *o = first ? a : *o + a;
            }
        }
    }
    // lane q of a quad stores passes 4 m + q: the sum over the workgroup's slices
    {
        const int q = lane % 4;
        float* dst = vp + ((size_t)(r * ny + s0) * 2 + P) * I + 16 * wave + lane / 4;
#pragma unroll
        for (int m = 0; m < kOutPer; ++m) {
            const int p = 4 * m + q;
            if (p < min(npass, kRegPasses) && kPassCh * p + 16 * wave + lane / 4 < I) dst[kPassCh * p] = osum[m];
        }
    }
}

template <int D, bool LR, bool ROUTE>
hipError_t vqt_lr(const int32_t* ids, int R, int k, int E, const VqArgs& vq, const float* h, int H, int I, float* vp,
                  int32_t* err, const SelRoute& route, hipStream_t stream) {
    const dim3 grid((2 * R + 7) / 8 * 8, vq_rows(R, H, D));
    // 16-byte index loads when every quarter segment is 16-byte aligned
    if ((H / D) % 16 == 0)
        MOE_LAUNCH((gateup_vqt_kernel<D, 16, LR, ROUTE>), grid, dim3(kVqThreads), 0, stream, ids, R, k,
                   FastDiv((uint32_t)k), E, vq, h, H, I, vp, err, route);
    else
        MOE_LAUNCH((gateup_vqt_kernel<D, 8, LR, ROUTE>), grid, dim3(kVqThreads), 0, stream, ids, R, k,
                   FastDiv((uint32_t)k), E, vq, h, H, I, vp, err, route);
    return hipGetLastError();
}

template <int D>
hipError_t vqt_d(const int32_t* ids, int R, int k, int E, const VqArgs& vq, const float* h, int H, int I, float* vp,
                 int32_t* err, const SelRoute* route, hipStream_t stream) {
    const SelRoute none{};
    if (route) {
        if (vq.r > 0) return vqt_lr<D, true, true>(ids, R, k, E, vq, h, H, I, vp, err, *route, stream);
        return vqt_lr<D, false, true>(ids, R, k, E, vq, h, H, I, vp, err, *route, stream);
    }
    if (vq.r > 0) return vqt_lr<D, true, false>(ids, R, k, E, vq, h, H, I, vp, err, none, stream);
    return vqt_lr<D, false, false>(ids, R, k, E, vq, h, H, I, vp, err, none, stream);
}

// One thread per (route, channel): the partial rows of both projections,
// all loads issued together, added in row order, p = SiLU(o_gate) * o_up.
// With an alignment job (the decode step, whose gate/up launch routed the
// tokens itself), workgroup (0, 0) then aligns the routes from the ids that
// launch stored: the canonical plan of the down projection.
constexpr int kMaxRows = 16;

struct AlignJob {
    const int32_t* ids;  // [R] route ids (null: no alignment)
    int E;
    FastDiv fb;          // division by the block size
    int32_t* sorted_routes;
    int32_t* block_expert;
    int32_t* counts;
    int32_t* err;
};

__global__ void __launch_bounds__(kThreads)
vq_finish_kernel(const float* __restrict__ vp, int R, int I, int ny, float* __restrict__ p, AlignJob aj) {
    extern __shared__ __align__(16) int asm_lds[];
    const int j = blockIdx.x * kThreads + threadIdx.x;
    const int r = blockIdx.y;
    if (j < I) {
        const float* src = vp + (size_t)r * ny * 2 * I + j;
        float g[kMaxRows], u[kMaxRows];
#pragma unroll
        for (int y = 0; y < kMaxRows; ++y) {
            const int yc = min(y, ny - 1);
            g[y] = src[(size_t)(2 * yc) * I];
            u[y] = src[(size_t)(2 * yc + 1) * I];
        }
        float og = 0.f, ou = 0.f;
#pragma unroll
        for (int y = 0; y < kMaxRows; ++y) {
            og += y < ny ? g[y] : 0.f;
            ou += y < ny ? u[y] : 0.f;
        }
        p[(size_t)r * I + j] = silu_mul(og, ou);
    }
    if (aj.ids && blockIdx.x == 0 && blockIdx.y == 0) {  // uniform
        if (R <= MOE_WAVE) {
            if (threadIdx.x < MOE_WAVE)
                align_wave([&](int q) { return aj.ids[q]; }, R, aj.E, aj.fb, aj.sorted_routes, aj.block_expert,
                           aj.counts, aj.err);
        } else {
            align_workgroup([&](int q) { return aj.ids[q]; }, R, aj.E, aj.fb, aj.sorted_routes, aj.block_expert,
                            aj.counts, aj.err, asm_lds);
        }
    }
}

}  // namespace

hipError_t launch_vq_finish(const float* vp, int R, int I, int ny, float* p, hipStream_t stream,
                            const VqPlanJob* plan) {
    if (ny < 1 || ny > kMaxRows || R < 1) return hipErrorInvalidValue;
    AlignJob aj{};
    size_t lds = 0;
    if (plan) {
        static_assert(kThreads == kAlignThreads, "the alignment runs on the finish workgroup's threads");
        if (!plan->ids || plan->E < 1 || plan->b < 1) return hipErrorInvalidValue;
        aj = AlignJob{plan->ids, plan->E, FastDiv((uint32_t)plan->b), plan->sorted_routes, plan->block_expert,
                      plan->counts, plan->err};
        lds = R > MOE_WAVE ? align_lds_bytes(R, plan->E) : 0;
    }
    MOE_LAUNCH(vq_finish_kernel, dim3((I + kThreads - 1) / kThreads, R), dim3(kThreads), lds, stream, vp, R, I, ny,
               p, aj);
    return hipGetLastError();
}

int vq_slices(int H, int d) { return (H / d + kSlice - 1) / kSlice; }

// Slice rows of the gate/up grid, and so the partials per route and
// projection: one per slice while the (route, projection, slice) workgroups
// fit on the device at once (two per CU, the LDS of the kernel's T, on 256
// CUs); beyond that a workgroup takes several slices of its route and
// projection in turn and stores their sum, so no workgroup waits for a
// second round and pays the route, code-book and z set-up again.
int vq_rows(int R, int H, int d) {
    const int nslice = vq_slices(H, d);
    const int per = (2 * R * nslice + kVqResident - 1) / kVqResident;  // slices per workgroup
    return (nslice + per - 1) / per;
}

bool vq_routes_ok(int E, int k) { return E <= kThreads && k <= 32; }

hipError_t launch_gateup_vqlr(const int32_t* topk_ids, int R, int k, int E, const VqArgs& vq, const float* h, int H,
                              int I, float* vp, int32_t* err, hipStream_t stream, const SelRoute* route) {
    if (vq.K < 1 || vq.K > kCodes || H % (8 * vq.d) || vq.r < 0 || vq.r > kMaxR || vq.r % 8 || R < 1 || k < 1)
        return hipErrorInvalidValue;
    if (route && (!vq_routes_ok(E, k) || !route->part || !route->ids || !route->wts || route->M * k != R))
        return hipErrorInvalidValue;
    if (vq.d == 8) return vqt_d<8>(topk_ids, R, k, E, vq, h, H, I, vp, err, route, stream);
    if (vq.d == 4) return vqt_d<4>(topk_ids, R, k, E, vq, h, H, I, vp, err, route, stream);
    if (vq.d == 2) return vqt_d<2>(topk_ids, R, k, E, vq, h, H, I, vp, err, route, stream);
    return hipErrorInvalidValue;
}

}  // namespace moe

// libmoe C ABI: argument validation (fail closed), workspace, launch order.
// The public contract of every function is documented in include/moe.h.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "launch.h"

namespace {

constexpr int kChanChunk = 8;      // kept channels per gather workgroup

struct Rec {
    int kernel;
    hipEvent_t a, b;
};

}  // namespace

// Device buffers of one call sequence (partials, tickets, lists); every
// kernel takes them as arguments.  A context owns one, laid out for its
// max_tokens by workspace_layout.
struct Workspace {
    int32_t* err = nullptr;            // sticky device error flags
    unsigned* ticket = nullptr;        // router last-workgroup tickets (zero between calls)
    float* router_part = nullptr;
    float* zpart[2] = {nullptr, nullptr};
    float* p = nullptr;
    float* down_part = nullptr;
    int32_t* slot_cnt = nullptr;   // channel-sparse: kept channels per (token, slot), int32 [MT][k]
    int32_t* slot_kept = nullptr;  // ... and their channels, int32 [MT][k][I]
    float* chan_part = nullptr;
    // reader: scanned coordinates and values [MT][H/128][80], estimates of
    // the block groups [MT][k][2][nbq][I], kept flags [MT][k][I], recovery
    // partials [MT][k][chunks][rec_rank]
    uint8_t* xsel = nullptr;
    float* xval = nullptr;
    float* est = nullptr;
    uint8_t* kept_flag = nullptr;
    float* rpart = nullptr;
};

struct moe_ctx {
    moe_config cfg;
    moe_weights w;
    int device = 0;
    void* ws_mem = nullptr;
    size_t ws_bytes = 0;
    Workspace ws;
    bool prof = false;
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
};

namespace moe {
LaunchEvents& launch_events() {
    thread_local LaunchEvents ev;
    return ev;
}
}  // namespace moe

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t align_capacity64(int64_t M, int64_t k, int64_t E, int64_t b) {
    const int64_t R = M * k;
    return R + (E < R ? E : R) * (b - 1);
}

constexpr int kMaxTokens = 4096;  // tokens (and routes) of one call at most

// Bytes of the workspace header: the sticky error word and the router's
// last-workgroup tickets, room for the largest token count whatever the
// context's, so that the header and every buffer after it sit at the same
// offsets for calls of any size.  The no-allocation entry point's calls of
// different sizes share one array, and its tickets must stay where earlier
// calls left them (re-armed at zero by their last workgroups) rather than
// land on another call's partials.
size_t workspace_header_bytes() { return 64 + sizeof(unsigned) * (1 + (size_t)moe::router_groups(kMaxTokens)); }

moe_status check_config(const moe_config* c) {
    if (c->H <= 0 || c->I <= 0 || c->E <= 0 || c->top_k <= 0 || c->block_b <= 0 || c->max_tokens <= 0 ||
        c->max_keep < 0)
        return MOE_ERR_INVALID_ARG;
    if (c->H % 8 || c->H < 8 || c->H > 8192) return MOE_ERR_UNSUPPORTED;
    if (c->I > 16384) return MOE_ERR_UNSUPPORTED;
    if (c->E % 8 || c->E < 8 || c->E > 1024) return MOE_ERR_UNSUPPORTED;
    if (c->top_k > 32 || c->top_k > c->E) return MOE_ERR_UNSUPPORTED;
    if (c->block_b > 64) return MOE_ERR_UNSUPPORTED;
    if (c->max_tokens > kMaxTokens || (int64_t)c->max_tokens * c->top_k > kMaxTokens) return MOE_ERR_UNSUPPORTED;
    const int64_t nchunk = ((int64_t)c->max_tokens * c->top_k + 63) / 64;
    if (nchunk * c->E > 6144) return MOE_ERR_UNSUPPORTED;
    if (c->wformat != MOE_WFORMAT_DENSE && c->wformat != MOE_WFORMAT_VQLR) return MOE_ERR_UNSUPPORTED;
    if (c->wformat == MOE_WFORMAT_VQLR) {
        if (c->vq_d != 2 && c->vq_d != 4 && c->vq_d != 8) return MOE_ERR_UNSUPPORTED;
        if (c->vq_K < 1 || c->vq_K > 256 || c->H % (8 * c->vq_d) || c->H / c->vq_d > 1024) return MOE_ERR_UNSUPPORTED;
        if (c->lr_r % 8 || c->lr_r < 0 || c->lr_r > 512) return MOE_ERR_UNSUPPORTED;  // 0: VQ only
    }
    if (c->max_keep > 0) {
        if (c->wformat != MOE_WFORMAT_DENSE) return MOE_ERR_UNSUPPORTED;
        if (c->max_keep > c->top_k * c->I || c->top_k * c->I > 8192) return MOE_ERR_UNSUPPORTED;
    }
    if (c->reader != 0 && c->reader != 1) return MOE_ERR_INVALID_ARG;
    if (c->rec_rank < 0) return MOE_ERR_INVALID_ARG;
    if (c->reader) {
        if (c->max_keep == 0 || c->H % 128) return MOE_ERR_UNSUPPORTED;
        if (c->rec_rank && (c->rec_rank < 8 || c->rec_rank > 32 || c->rec_rank % 8)) return MOE_ERR_UNSUPPORTED;
    } else if (c->rec_rank) {
        return MOE_ERR_UNSUPPORTED;  // the recovery map belongs to the reader
    }
    return MOE_OK;
}

moe_status check_weights(const moe_config* c, const moe_weights* w) {
    if (!w->router_w || !w->w_down) return MOE_ERR_INVALID_ARG;
    if (!aligned(w->router_w, 16) || !aligned(w->w_down, 16)) return MOE_ERR_INVALID_ARG;
    if (w->router_bias && !aligned(w->router_bias, 4)) return MOE_ERR_INVALID_ARG;
    if (c->wformat == MOE_WFORMAT_DENSE) {
        if (!w->w_gate || !w->w_up) return MOE_ERR_INVALID_ARG;
        if (!aligned(w->w_gate, 16) || !aligned(w->w_up, 16)) return MOE_ERR_INVALID_ARG;
    } else {
        for (int P = 0; P < 2; ++P) {
            if (!w->vq_book[P] || !w->vq_idx[P] || !aligned(w->vq_book[P], 16) || !aligned(w->vq_idx[P], 16))
                return MOE_ERR_INVALID_ARG;
            if (c->lr_r == 0) continue;  // VQ only: no low-rank term
            if (!w->lr_basis[P] || !w->lr_coef[P] || !aligned(w->lr_basis[P], 16) || !aligned(w->lr_coef[P], 16))
                return MOE_ERR_INVALID_ARG;
        }
    }
    if (c->max_keep > 0 && !c->reader && (!w->chan_norm || !aligned(w->chan_norm, 16)))
        return MOE_ERR_INVALID_ARG;
    if (c->reader) {
        if (!w->rot_signs || !w->sketch || !aligned(w->sketch, 16) || !w->sketch_scale ||
            !aligned(w->sketch_scale, 4) || !w->down_norm || !aligned(w->down_norm, 16))
            return MOE_ERR_INVALID_ARG;
        if (c->rec_rank &&
            (!w->rec_basis || !aligned(w->rec_basis, 4) || !w->rec_coef || !aligned(w->rec_coef, 16)))
            return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

// Byte size of the workspace of `c` for calls of up to MT tokens; with a
// base address, also the buffer addresses inside it (256-byte aligned).
size_t workspace_layout(const moe_config& c, size_t MT, char* base, Workspace* ws) {
    const size_t R = MT * c.top_k;
    const size_t zsl = c.wformat == MOE_WFORMAT_VQLR && c.lr_r > 0 ? moe::gemv_slices(c.H, c.lr_r) : 0;
    // down partials: one chunk per route on the split path; the fused path
    // (one token) writes dense_chunks of them for each of its top_k routes
    size_t down = R * (size_t)moe::down_chunks(c.I) * c.H;
    if (moe::dense_uses_fused(1, c.H)) {
        const size_t f = (size_t)c.top_k * moe::dense_chunks(1, c.H, c.I, c.top_k) * c.H;
        down = f > down ? f : down;
    }
    const size_t nchan = c.max_keep > 0 ? (c.max_keep + kChanChunk - 1) / kChanChunk : 0;
    const size_t rd = c.reader ? 1 : 0;
    const size_t nscan = rd * MT * (c.H / 128) * 80;  // scanned coordinates of all blocks
    const size_t nkc = rd * R * c.I;                    // candidates
    const size_t nbq = c.reader ? (size_t)moe::reader_groups(c.H / 128, nullptr) : 0;
    constexpr int kBufs = 13;
    const size_t sizes[kBufs] = {
        workspace_header_bytes(),                                       // err flag, router tickets
        sizeof(float) * moe::gemv_slices(c.H, c.E) * MT * c.E,          // router partials
        sizeof(float) * zsl * MT * c.lr_r,                              // z = D^T h partials (gate)
        sizeof(float) * zsl * MT * c.lr_r,                              // z partials (up)
        sizeof(float) * R * c.I * (c.wformat == MOE_WFORMAT_VQLR ? 1 + 2 * (size_t)moe::vq_slices(c.H, c.vq_d) : 1),  // p (+ VQ gate/up partials)
        sizeof(float) * down,                                           // down partials
        c.max_keep > 0 ? sizeof(int32_t) * MT * c.top_k * (1 + (size_t)c.I) : 0,  // per-slot kept lists
        sizeof(float) * MT * nchan * c.H,                               // channel partials
        nscan,                                                          // reader: scanned coordinates
        sizeof(float) * nscan,                                          // ... and their values
        sizeof(float) * 2 * nbq * nkc,                                  // group estimates
        nkc,                                                            // kept flags
        sizeof(float) * R * (c.rec_rank ? (size_t)moe::reader_recover_chunks(c.I) * c.rec_rank : 0),  // recovery
    };
    size_t off[kBufs], total = 0;
    for (int i = 0; i < kBufs; ++i) {
        off[i] = total;
        total += (sizes[i] + 255) & ~(size_t)255;
    }
    if (base && ws) {
        ws->err = reinterpret_cast<int32_t*>(base + off[0]);
        ws->ticket = reinterpret_cast<unsigned*>(base + off[0] + 64);
        ws->router_part = reinterpret_cast<float*>(base + off[1]);
        ws->zpart[0] = reinterpret_cast<float*>(base + off[2]);
        ws->zpart[1] = reinterpret_cast<float*>(base + off[3]);
        ws->p = reinterpret_cast<float*>(base + off[4]);
        ws->down_part = reinterpret_cast<float*>(base + off[5]);
        ws->slot_cnt = reinterpret_cast<int32_t*>(base + off[6]);
        ws->slot_kept = ws->slot_cnt + MT * c.top_k;
        ws->chan_part = reinterpret_cast<float*>(base + off[7]);
        ws->xsel = reinterpret_cast<uint8_t*>(base + off[8]);
        ws->xval = reinterpret_cast<float*>(base + off[9]);
        ws->est = reinterpret_cast<float*>(base + off[10]);
        ws->kept_flag = reinterpret_cast<uint8_t*>(base + off[11]);
        ws->rpart = reinterpret_cast<float*>(base + off[12]);
    }
    return total;
}


hipEvent_t take_event(moe_ctx* ctx) {
    if (!ctx->pool.empty()) {
        hipEvent_t e = ctx->pool.back();
        ctx->pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// While profiling, hands a start/stop event pair to the next launch, which
// stamps them from its own dispatch (see MOE_LAUNCH).  Without a context
// (or with profiling off) it does nothing.
struct Launch {
    moe_ctx* ctx;
    Rec rec{};
    bool on = false;
    Launch(moe_ctx* c, int kernel) : ctx(c) {
        if (ctx && ctx->prof) {
            rec.kernel = kernel;
            rec.a = take_event(ctx);
            rec.b = take_event(ctx);
            on = rec.a && rec.b;
            if (on) moe::launch_events() = moe::LaunchEvents{rec.a, rec.b};
        }
    }
    void done() {
        moe::launch_events() = moe::LaunchEvents{};
        if (on) ctx->recs.push_back(rec);
        on = false;
    }
};

// What one call runs on: the layer (config, weights), the workspace its
// kernels use, and the context that records profiling events (or null).
struct Exec {
    const moe_config& c;
    const moe_weights& w;
    const Workspace& ws;
    moe_ctx* prof;
};

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Channel-sparse mode from the routes (or, with `route`, from the router's
// slice partials): the selection-and-gather launch, then the combine (with
// the recovery map in reader mode when rec_rank > 0).  mode 0: static norms,
// 1: the reader's estimates (already screened).
moe_status sparse_gather_combine(const Exec& x, int mode, const moe::SelRoute* route, const moe::ReaderArgs* ra,
                                 const float* h, int M, int32_t* topk_ids, float* topk_w, int K, int32_t* kept_out,
                                 float* y, hipStream_t s) {
    const moe_config& c = x.c;
    const int nchunks = (K + kChanChunk - 1) / kChanChunk;
    const bool rec = mode == 1 && c.rec_rank > 0;
    hipError_t e;
    {
        Launch l(x.prof, MOE_KERNEL_CHAN_GATHER);
        e = moe::launch_chan_topk_gather(mode, route, topk_ids, topk_w, x.w.chan_norm, ra, M, c.top_k, c.I, c.E, c.H,
                                         K, h, x.w.w_gate, x.w.w_up, x.w.w_down, x.ws.chan_part, kept_out,
                                         rec ? x.ws.kept_flag : nullptr, s);
        l.done();
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    if (!rec) {
        Launch l(x.prof, MOE_KERNEL_CHAN_COMBINE);
        e = moe::launch_chan_combine(M, c.H, nchunks, x.ws.chan_part, y, s);
        l.done();
        return hip_status(e);
    }
    {
        Launch l(x.prof, MOE_KERNEL_READER_RECOVER);
        e = moe::launch_reader_recover(*ra, topk_ids, topk_w, M, s);
        l.done();
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    Launch l(x.prof, MOE_KERNEL_READER_COMBINE);
    e = moe::launch_reader_combine(M, c.H, nchunks, x.ws.chan_part, x.ws.rpart,
                                   c.top_k * moe::reader_recover_chunks(c.I), c.rec_rank, x.w.rec_basis, y, s);
    l.done();
    return hip_status(e);
}

moe::ReaderArgs reader_args(const Exec& x) {
    moe::ReaderArgs ra{};
    ra.sketch = x.w.sketch;
    ra.scale = x.w.sketch_scale;
    ra.xsel = x.ws.xsel;
    ra.xval = x.ws.xval;
    ra.est = x.ws.est;
    ra.dnorm = x.w.down_norm;
    ra.kept_flag = x.ws.kept_flag;
    ra.rec_coef = x.w.rec_coef;
    ra.rpart = x.ws.rpart;
    ra.rank = x.c.rec_rank;
    ra.nblk = x.c.H / 128;
    ra.nbq = moe::reader_groups(ra.nblk, &ra.bpw);
    ra.rowb = moe::reader_row_bytes(x.c.I);
    ra.I = x.c.I;
    ra.k = x.c.top_k;
    ra.E = x.c.E;
    return ra;
}

// Reader, from the routes on: rotation (unless already done), screening,
// then selection-and-gather and the combine (with the recovery map when
// rec_rank > 0).
moe_status reader_forward(const Exec& x, bool rotated, const moe::SelRoute* route, const float* h, int M,
                          const int32_t* topk_ids, const float* topk_w, int K, int32_t* kept_out, float* y,
                          hipStream_t s) {
    const moe_config& c = x.c;
    const moe::ReaderArgs ra = reader_args(x);
    hipError_t e;
    if (!rotated) {
        Launch l(x.prof, MOE_KERNEL_READER_ROTATE);
        e = moe::launch_reader_rotate(h, M, c.H, x.w.rot_signs, x.ws.xsel, x.ws.xval, s);
        l.done();
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    {
        Launch l(x.prof, MOE_KERNEL_READER_SCREEN);
        e = moe::launch_reader_screen(ra, route, topk_ids, M, s);
        l.done();
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return sparse_gather_combine(x, 1, nullptr, &ra, h, M, const_cast<int32_t*>(topk_ids),
                                 const_cast<float*>(topk_w), K, kept_out, y, s);
}

moe_status route_topk_impl(const Exec& x, const float* h, int32_t M, int32_t* topk_ids, float* topk_w,
                           float* logits_out, hipStream_t s) {
    if (M == 0) return MOE_OK;
    if (!h || !topk_ids || !topk_w || !aligned(h, 16)) return MOE_ERR_INVALID_ARG;
    const moe_config& c = x.c;
    Launch l(x.prof, MOE_KERNEL_ROUTER);
    hipError_t e = moe::launch_router(h, M, c.H, x.w.router_w, c.E, x.w.router_bias, c.top_k, x.ws.router_part,
                                      x.ws.ticket, topk_ids, topk_w, logits_out, s);
    l.done();
    return hip_status(e);
}

moe_status align_impl(const Exec& x, const int32_t* topk_ids, int32_t M, int32_t* sorted_routes,
                      int32_t* block_expert, int32_t* counts, hipStream_t s) {
    if (!counts) return MOE_ERR_INVALID_ARG;
    // M == 0: the kernel runs with no routes and only writes counts = {0, 0}
    if (M > 0 && (!topk_ids || !sorted_routes || !block_expert)) return MOE_ERR_INVALID_ARG;
    const moe_config& c = x.c;
    Launch l(x.prof, MOE_KERNEL_ALIGN);
    hipError_t e = moe::launch_align(topk_ids, M * c.top_k, c.E, c.block_b, sorted_routes, block_expert, counts,
                                     x.ws.err, s);
    l.done();
    return hip_status(e);
}

moe_status route_align_impl(const Exec& x, bool with_z, const float* h, int32_t M, int32_t* topk_ids,
                            float* topk_w, float* logits_out, int32_t* sorted_routes, int32_t* block_expert,
                            int32_t* counts, hipStream_t s) {
    if (!counts) return MOE_ERR_INVALID_ARG;
    if (M == 0) return align_impl(x, nullptr, 0, nullptr, nullptr, counts, s);
    if (!h || !topk_ids || !topk_w || !sorted_routes || !block_expert || !aligned(h, 16)) return MOE_ERR_INVALID_ARG;
    const moe_config& c = x.c;
    // with_z: the VQ + low-rank shared projections z = D^T h ride along as
    // extra workgroups of the same launch
    const moe::GemvJob jobs[2] = {{x.w.lr_basis[0], c.lr_r, x.ws.zpart[0]},
                                  {x.w.lr_basis[1], c.lr_r, x.ws.zpart[1]}};
    Launch l(x.prof, MOE_KERNEL_ROUTER_ALIGN);
    hipError_t e = moe::launch_router_align(h, M, c.H, x.w.router_w, c.E, x.w.router_bias, c.top_k,
                                            x.ws.router_part, x.ws.ticket, topk_ids, topk_w, logits_out, c.block_b,
                                            sorted_routes, block_expert, counts, x.ws.err, s,
                                            with_z ? jobs : nullptr, with_z ? 2 : 0);
    l.done();
    return hip_status(e);
}

// vq_route / vq_plan (VQ + low rank, the decode step): the gate/up launch
// routes the tokens itself (storing ids, weights and logits) and the finish
// launch aligns the routes into sorted_routes / block_expert / counts.
moe_status expert_forward_impl(const Exec& x, bool z_ready, const float* h, int32_t M, const int32_t* topk_ids,
                               const float* topk_w, const int32_t* sorted_routes, const int32_t* block_expert,
                               const int32_t* counts, int32_t keep_channels, int32_t* kept_out, float* y,
                               hipStream_t s, const moe::SelRoute* vq_route = nullptr,
                               const moe::AlignOut* vq_plan = nullptr) {
    const moe_config& c = x.c;
    if (M == 0) return MOE_OK;
    if (!h || !topk_ids || !topk_w || !y || !aligned(h, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
    hipError_t e;

    if (keep_channels > 0) {
        if (c.max_keep == 0 || c.wformat != MOE_WFORMAT_DENSE) return MOE_ERR_UNSUPPORTED;
        if (keep_channels > c.max_keep) return MOE_ERR_CAPACITY;
        if (c.reader) return reader_forward(x, false, nullptr, h, M, topk_ids, topk_w, keep_channels, kept_out, y, s);
        return sparse_gather_combine(x, 0, nullptr, nullptr, h, M, const_cast<int32_t*>(topk_ids),
                                     const_cast<float*>(topk_w), keep_channels, kept_out, y, s);
    }

    if (!sorted_routes || !block_expert || !counts) return MOE_ERR_INVALID_ARG;
    moe::PlanArgs plan{};
    plan.topk_ids = topk_ids;
    plan.sorted_routes = sorted_routes;
    plan.block_expert = block_expert;
    plan.counts = counts;
    plan.R = M * c.top_k;
    plan.k = c.top_k;
    plan.fk = FastDiv((uint32_t)c.top_k);
    plan.b = c.block_b;
    plan.fb = FastDiv((uint32_t)c.block_b);
    plan.max_blocks = (int)(align_capacity64(M, c.top_k, c.E, c.block_b) / c.block_b);
    plan.E = c.E;

    int nchunk = moe::down_chunks(c.I);
    if (c.wformat == MOE_WFORMAT_DENSE && moe::dense_uses_fused(M, c.H)) {
        nchunk = moe::dense_chunks(M, c.H, c.I, c.top_k);
        Launch l(x.prof, MOE_KERNEL_EXPERT_FUSED);
        e = moe::launch_expert_fused(plan, h, topk_w, c.H, c.I, x.w.w_gate, x.w.w_up, x.w.w_down, x.ws.down_part,
                                     x.ws.err, s);
        l.done();
        if (e != hipSuccess) return MOE_ERR_HIP;
    } else {
        if (c.wformat == MOE_WFORMAT_DENSE) {
            Launch l(x.prof, MOE_KERNEL_GATEUP);
            e = moe::launch_gateup_dense(plan, h, c.H, c.I, x.w.w_gate, x.w.w_up, x.ws.p, x.ws.err, s);
            l.done();
            if (e != hipSuccess) return MOE_ERR_HIP;
            Launch ld(x.prof, MOE_KERNEL_DOWN);
            e = moe::launch_down(plan, c.H, c.I, x.w.w_down, x.ws.p, topk_w, x.ws.down_part, x.ws.err, s);
            ld.done();
            if (e != hipSuccess) return MOE_ERR_HIP;
        } else {
            moe::GemvJob jobs[2] = {{x.w.lr_basis[0], c.lr_r, x.ws.zpart[0]},
                                    {x.w.lr_basis[1], c.lr_r, x.ws.zpart[1]}};
            if (!z_ready && c.lr_r > 0) {  // else computed by the routing launch of this step (or no low rank)
                Launch l(x.prof, MOE_KERNEL_VQ_SHARED);
                e = moe::launch_gemv_partials(h, M, c.H, jobs, 2, s);
                l.done();
                if (e != hipSuccess) return MOE_ERR_HIP;
            }
            moe::VqArgs vq{};
            for (int P = 0; P < 2; ++P) {
                vq.C[P] = x.w.lr_coef[P];
                vq.B[P] = x.w.vq_book[P];
                vq.J[P] = x.w.vq_idx[P];
                vq.zpart[P] = x.ws.zpart[P];
            }
            vq.zslices = c.lr_r > 0 ? moe::gemv_slices(c.H, c.lr_r) : 0;
            vq.M = M;
            vq.r = c.lr_r;
            vq.K = c.vq_K;
            vq.d = c.vq_d;
            // the gate/up partials after p in the same buffer
            float* const vpart = x.ws.p + (size_t)plan.R * c.I;
            const moe::VqP vqp{vpart, moe::vq_rows(plan.R, c.H, c.vq_d)};
            {
                Launch l(x.prof, MOE_KERNEL_GATEUP_VQLR);
                e = moe::launch_gateup_vqlr(topk_ids, plan.R, c.top_k, c.E, vq, h, c.H, c.I, vpart, x.ws.err, s,
                                            vq_route);
                l.done();
                if (e != hipSuccess) return MOE_ERR_HIP;
            }
            // Up to 64 routes the down launch adds the partials itself (and in
            // the decode step aligns the routes); above, a finishing launch
            // forms p (and aligns), then the down launch reads p.  Both form
            // p = SiLU(o_gate) * o_up with the same sums, bit for bit.
            const bool in_down = plan.R <= MOE_WAVE;
            if (!in_down) {
                const moe::VqPlanJob pj = vq_plan ? moe::VqPlanJob{topk_ids, c.E, c.block_b, vq_plan->sorted_routes,
                                                                   vq_plan->block_expert, vq_plan->counts, x.ws.err}
                                                  : moe::VqPlanJob{};
                Launch l(x.prof, MOE_KERNEL_VQ_FINISH);
                e = moe::launch_vq_finish(vqp.vp, plan.R, c.I, vqp.ny, x.ws.p, s, vq_plan ? &pj : nullptr);
                l.done();
                if (e != hipSuccess) return MOE_ERR_HIP;
            }
            Launch l(x.prof, MOE_KERNEL_DOWN);
            e = moe::launch_down(plan, c.H, c.I, x.w.w_down, x.ws.p, topk_w, x.ws.down_part, x.ws.err, s,
                                 in_down ? &vqp : nullptr, in_down && vq_plan ? vq_plan : nullptr);
            l.done();
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
    }
    Launch l(x.prof, MOE_KERNEL_COMBINE);
    e = moe::launch_combine(topk_ids, M, c.top_k, c.E, c.H, nchunk, x.ws.down_part, y, s);
    l.done();
    return hip_status(e);
}

moe_status decode_step_impl(const Exec& x, const float* h, int32_t M, int32_t* topk_ids, float* topk_w,
                            float* logits_out, int32_t* sorted_routes, int32_t* block_expert, int32_t* counts,
                            int32_t keep_channels, int32_t* kept_out, float* y, hipStream_t s) {
    const moe_config& c = x.c;
    if (keep_channels > 0) {
        // router GEMV partials, then a channel selection whose workgroups
        // route their tokens, then gather and combine
        if (c.max_keep == 0 || c.wformat != MOE_WFORMAT_DENSE) return MOE_ERR_UNSUPPORTED;
        if (keep_channels > c.max_keep) return MOE_ERR_CAPACITY;
        if (M == 0) return MOE_OK;
        if (!h || !topk_ids || !topk_w || !y || !aligned(h, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
        hipError_t e;
        if (c.reader && c.E > 256) {  // routing as moe_route_topk, then the reader from the routes
            moe_status st = route_topk_impl(x, h, M, topk_ids, topk_w, logits_out, s);
            if (st != MOE_OK) return st;
            return reader_forward(x, false, nullptr, h, M, topk_ids, topk_w, keep_channels, kept_out, y, s);
        }
        {
            // the reader's rotation rides along in workgroups of its own
            const moe::RotJob rot{x.w.rot_signs, x.ws.xsel, x.ws.xval};
            Launch l(x.prof, MOE_KERNEL_ROUTER_GEMV);
            e = moe::launch_router_partials(h, M, c.H, x.w.router_w, c.E, x.ws.router_part, s,
                                            c.reader ? &rot : nullptr);
            l.done();
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
        moe::SelRoute route{};
        route.part = x.ws.router_part;
        route.bias = x.w.router_bias;
        route.nslices = moe::router_slices(c.H, c.E);
        route.M = M;
        route.ids = topk_ids;
        route.wts = topk_w;
        route.logits = logits_out;
        if (c.reader) return reader_forward(x, true, &route, h, M, topk_ids, topk_w, keep_channels, kept_out, y, s);
        return sparse_gather_combine(x, 0, &route, nullptr, h, M, topk_ids, topk_w, keep_channels, kept_out, y, s);
    }
    const int nsl = moe::router_slices(c.H, c.E);
    if (c.wformat == MOE_WFORMAT_VQLR && M > 0 && moe::vq_routes_ok(c.E, c.top_k)) {
        // router GEMV partials (and z = D^T h in workgroups of their own),
        // then a gate/up launch whose workgroups route their tokens, a down
        // launch that adds the gate/up partials (and aligns the routes), and
        // the combine
        if (!h || !topk_ids || !topk_w || !sorted_routes || !block_expert || !counts || !y || !aligned(h, 16) ||
            !aligned(y, 16))
            return MOE_ERR_INVALID_ARG;
        const moe::GemvJob jobs[2] = {{x.w.lr_basis[0], c.lr_r, x.ws.zpart[0]},
                                      {x.w.lr_basis[1], c.lr_r, x.ws.zpart[1]}};
        {
            Launch l(x.prof, MOE_KERNEL_ROUTER_GEMV);
            const hipError_t e = moe::launch_router_partials(h, M, c.H, x.w.router_w, c.E, x.ws.router_part, s,
                                                             nullptr, c.lr_r > 0 ? jobs : nullptr,
                                                             c.lr_r > 0 ? 2 : 0);
            l.done();
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
        moe::SelRoute route{};
        route.part = x.ws.router_part;
        route.bias = x.w.router_bias;
        route.nslices = nsl;
        route.M = M;
        route.ids = topk_ids;
        route.wts = topk_w;
        route.logits = logits_out;
        const moe::AlignOut pj{sorted_routes, block_expert, counts};
        return expert_forward_impl(x, true, h, M, topk_ids, topk_w, sorted_routes, block_expert, counts, 0, nullptr,
                                   y, s, &route, &pj);
    }
    if (M != 1 || c.wformat != MOE_WFORMAT_DENSE || !moe::decode_fused_ok(c.H, c.E, c.top_k, nsl)) {
        const bool vq = c.wformat == MOE_WFORMAT_VQLR;  // z = D^T h in the routing launch
        moe_status st = route_align_impl(x, vq && c.lr_r > 0, h, M, topk_ids, topk_w, logits_out, sorted_routes,
                                         block_expert, counts, s);
        if (st != MOE_OK) return st;
        return expert_forward_impl(x, vq, h, M, topk_ids, topk_w, sorted_routes, block_expert, counts, 0, nullptr,
                                   y, s);
    }
    if (!h || !topk_ids || !topk_w || !sorted_routes || !block_expert || !counts || !y || !aligned(h, 16) ||
        !aligned(y, 16))
        return MOE_ERR_INVALID_ARG;
    hipError_t e;
    {
        Launch l(x.prof, MOE_KERNEL_ROUTER_GEMV);
        e = moe::launch_router_partials(h, 1, c.H, x.w.router_w, c.E, x.ws.router_part, s);
        l.done();
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    moe::PlanArgs plan{};
    plan.R = c.top_k;
    plan.k = c.top_k;
    plan.fk = FastDiv((uint32_t)c.top_k);
    plan.b = c.block_b;
    plan.fb = FastDiv((uint32_t)c.block_b);
    plan.max_blocks = c.top_k;
    plan.E = c.E;
    moe::RouteArgs route{};
    route.part = x.ws.router_part;
    route.bias = x.w.router_bias;
    route.nslices = nsl;
    route.ids = topk_ids;
    route.wts = topk_w;
    route.logits = logits_out;
    route.sorted_routes = sorted_routes;
    route.block_expert = block_expert;
    route.counts = counts;
    {
        Launch l(x.prof, MOE_KERNEL_DECODE_FUSED);
        e = moe::launch_decode_fused(plan, route, h, c.H, c.I, x.w.w_gate, x.w.w_up, x.w.w_down, x.ws.down_part,
                                     x.ws.err, s);
        l.done();
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    Launch l(x.prof, MOE_KERNEL_COMBINE);
    e = moe::launch_combine(topk_ids, 1, c.top_k, c.E, c.H, moe::dense_chunks(1, c.H, c.I, c.top_k),
                            x.ws.down_part, y, s);
    l.done();
    return hip_status(e);
}

Exec exec_of(moe_ctx* ctx) { return Exec{ctx->cfg, ctx->w, ctx->ws, ctx}; }

// Workspace of moe_decode_step_noalloc: one array per device, zeroed when the
// code object is loaded (so its error word and tickets start at zero; every
// kernel that takes a ticket re-arms it) and kept until the process ends.
// In host code `scratch` names a host-side stand-in: its device address on
// each GPU comes from hipGetSymbolAddress and is kept per device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
moe_status scratch_address(char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
        g_scratch_dev[dev] = static_cast<char*>(ptr);
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_align_capacity(int32_t M, int32_t k, int32_t E, int32_t b) {
    if (M < 0 || k <= 0 || E <= 0 || b <= 0) return -1;
    const int64_t c = align_capacity64(M, k, E, b);
    return c > INT32_MAX ? -1 : (int32_t)c;
}

int64_t moe_workspace_bytes(const moe_config* cfg, int32_t max_tokens) {
    if (!cfg || max_tokens < 1) return -1;
    moe_config c = *cfg;
    c.max_tokens = max_tokens;
    if (check_config(&c) != MOE_OK) return -1;
    return (int64_t)workspace_layout(c, (size_t)max_tokens, nullptr, nullptr);
}

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
        case MOE_ERR_CAPACITY: return "capacity exceeded";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_DEVICE: return "device error flag set";
    }
    return "unknown status";
}

const char* moe_kernel_name(int32_t k) {
    static const char* names[MOE_KERNEL_COUNT] = {"router",      "vq_shared",   "align",        "gateup",
                                                  "gateup_vqlr", "down",        "combine",      "chan_select",
                                                  "chan_gather", "chan_combine", "expert_fused", "router_align",
                                                  "router_gemv", "decode_fused", "vq_finish",   "reader_rotate",
                                                  "reader_screen", "reader_select", "reader_recover",
                                                  "reader_combine"};
    return (k >= 0 && k < MOE_KERNEL_COUNT) ? names[k] : nullptr;
}

moe_status moe_create(const moe_config* cfg, const moe_weights* w, moe_ctx** out) {
    if (!out) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg || !w) return MOE_ERR_INVALID_ARG;
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    st = check_weights(cfg, w);
    if (st != MOE_OK) return st;

    moe_ctx* ctx = new (std::nothrow) moe_ctx();
    if (!ctx) return MOE_ERR_HIP;
    ctx->cfg = *cfg;
    ctx->w = *w;
    if (hipGetDevice(&ctx->device) != hipSuccess) {
        delete ctx;
        return MOE_ERR_HIP;
    }
    const size_t MT = cfg->max_tokens;
    const size_t total = workspace_layout(*cfg, MT, nullptr, nullptr);
    if (hipMalloc(&ctx->ws_mem, total) != hipSuccess) {
        delete ctx;
        return MOE_ERR_HIP;
    }
    ctx->ws_bytes = total;
    workspace_layout(*cfg, MT, static_cast<char*>(ctx->ws_mem), &ctx->ws);
    if (hipMemset(ctx->ws_mem, 0, workspace_header_bytes()) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        hipFree(ctx->ws_mem);
        delete ctx;
        return MOE_ERR_HIP;
    }
    *out = ctx;
    return MOE_OK;
}

void moe_destroy(moe_ctx* ctx) {
    if (!ctx) return;
    hipDeviceSynchronize();
    for (auto& r : ctx->recs) {
        hipEventDestroy(r.a);
        hipEventDestroy(r.b);
    }
    for (auto e : ctx->pool) hipEventDestroy(e);
    if (ctx->ws_mem) hipFree(ctx->ws_mem);
    delete ctx;
}

moe_status moe_route_topk(moe_ctx* ctx, const float* h, int32_t M, int32_t* topk_ids, float* topk_w,
                          float* logits_out, void* stream) {
    if (!ctx || M < 0) return MOE_ERR_INVALID_ARG;
    if (M > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    return route_topk_impl(exec_of(ctx), h, M, topk_ids, topk_w, logits_out, static_cast<hipStream_t>(stream));
}

moe_status moe_route_align(moe_ctx* ctx, const float* h, int32_t M, int32_t* topk_ids, float* topk_w,
                           float* logits_out, int32_t* sorted_routes, int32_t* block_expert, int32_t* counts,
                           void* stream) {
    if (!ctx || M < 0) return MOE_ERR_INVALID_ARG;
    if (M > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    return route_align_impl(exec_of(ctx), false, h, M, topk_ids, topk_w, logits_out, sorted_routes, block_expert,
                            counts, static_cast<hipStream_t>(stream));
}

moe_status moe_align_blocks(moe_ctx* ctx, const int32_t* topk_ids, int32_t M, int32_t* sorted_routes,
                            int32_t* block_expert, int32_t* counts, void* stream) {
    if (!ctx || M < 0) return MOE_ERR_INVALID_ARG;
    if (M > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    return align_impl(exec_of(ctx), topk_ids, M, sorted_routes, block_expert, counts,
                      static_cast<hipStream_t>(stream));
}

moe_status moe_expert_forward(moe_ctx* ctx, const float* h, int32_t M, const int32_t* topk_ids, const float* topk_w,
                              const int32_t* sorted_routes, const int32_t* block_expert, const int32_t* counts,
                              int32_t keep_channels, int32_t* kept_out, float* y, void* stream) {
    if (!ctx || M < 0 || keep_channels < 0) return MOE_ERR_INVALID_ARG;
    if (M > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    return expert_forward_impl(exec_of(ctx), false, h, M, topk_ids, topk_w, sorted_routes, block_expert, counts,
                               keep_channels, kept_out, y, static_cast<hipStream_t>(stream));
}

moe_status moe_decode_step(moe_ctx* ctx, const float* h, int32_t M, int32_t* topk_ids, float* topk_w,
                           float* logits_out, int32_t* sorted_routes, int32_t* block_expert, int32_t* counts,
                           int32_t keep_channels, int32_t* kept_out, float* y, void* stream) {
    if (!ctx || M < 0 || keep_channels < 0) return MOE_ERR_INVALID_ARG;
    if (M > ctx->cfg.max_tokens) return MOE_ERR_CAPACITY;
    return decode_step_impl(exec_of(ctx), h, M, topk_ids, topk_w, logits_out, sorted_routes, block_expert, counts,
                            keep_channels, kept_out, y, static_cast<hipStream_t>(stream));
}

moe_status moe_decode_step_noalloc(const moe_config* cfg, const moe_weights* w, const float* h, int32_t M,
                                   int32_t* topk_ids, float* topk_w, float* logits_out, int32_t* sorted_routes,
                                   int32_t* block_expert, int32_t* counts, int32_t keep_channels, int32_t* kept_out,
                                   float* y, void* stream) {
    if (!cfg || !w || M < 0 || keep_channels < 0) return MOE_ERR_INVALID_ARG;
    moe_status st = check_config(cfg);
    if (st != MOE_OK) return st;
    st = check_weights(cfg, w);
    if (st != MOE_OK) return st;
    if (M > cfg->max_tokens) return MOE_ERR_CAPACITY;
    // the workspace of exactly this call's M must fit the array
    const size_t MT = M > 0 ? (size_t)M : 1;
    if (workspace_layout(*cfg, MT, nullptr, nullptr) > kScratchBytes) return MOE_ERR_CAPACITY;
    char* base = nullptr;
    st = scratch_address(&base);
    if (st != MOE_OK) return st;
    Workspace ws;
    workspace_layout(*cfg, MT, base, &ws);
    const Exec x{*cfg, *w, ws, nullptr};
    return decode_step_impl(x, h, M, topk_ids, topk_w, logits_out, sorted_routes, block_expert, counts,
                            keep_channels, kept_out, y, static_cast<hipStream_t>(stream));
}

moe_status moe_reader_inspect(moe_ctx* ctx, const float* h, int32_t M, const int32_t* topk_ids,
                              const float* topk_w, int32_t K, uint8_t* xsel, float* xval, float* est, float* score,
                              int32_t* kept, void* stream) {
    if (!ctx || M < 0) return MOE_ERR_INVALID_ARG;
    const moe_config& c = ctx->cfg;
    if (!c.reader) return MOE_ERR_UNSUPPORTED;
    if (M > c.max_tokens || K > c.max_keep) return MOE_ERR_CAPACITY;
    if (K < 1) return MOE_ERR_INVALID_ARG;
    if (M == 0) return MOE_OK;
    if (!h || !topk_ids || !topk_w || !aligned(h, 16)) return MOE_ERR_INVALID_ARG;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const Exec x = exec_of(ctx);
    const moe::ReaderArgs ra = reader_args(x);
    hipError_t e = moe::launch_reader_rotate(h, M, c.H, x.w.rot_signs, x.ws.xsel, x.ws.xval, s);
    if (e == hipSuccess) e = moe::launch_reader_screen(ra, nullptr, topk_ids, M, s);
    if (e == hipSuccess)
        e = moe::launch_reader_select(ra, topk_ids, topk_w, M, K, x.ws.slot_cnt, x.ws.slot_kept, kept, est, score, s);
    const size_t nscan = (size_t)M * (c.H / 128) * 80;
    if (e == hipSuccess && xsel) e = hipMemcpyAsync(xsel, x.ws.xsel, nscan, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && xval) e = hipMemcpyAsync(xval, x.ws.xval, 4 * nscan, hipMemcpyDeviceToDevice, s);
    return hip_status(e);
}

int32_t moe_sketch_row_bytes(int32_t I) {
    if (I < 1 || I > 16384) return -1;
    return moe::reader_row_bytes(I);
}

namespace {
moe_status check_load_shape(const moe_config* cfg) {
    if (!cfg || cfg->H <= 0 || cfg->I <= 0 || cfg->E <= 0) return MOE_ERR_INVALID_ARG;
    if (cfg->H % 8 || cfg->H > 8192 || cfg->I > 16384 || cfg->E > 8192) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}
}  // namespace

moe_status moe_reader_sketch(const moe_config* cfg, const uint16_t* w_gate, const uint16_t* w_up,
                             const int8_t* rot_signs, uint8_t* sketch, float* sketch_scale, void* stream) {
    moe_status st = check_load_shape(cfg);
    if (st != MOE_OK) return st;
    if (cfg->H % 128) return MOE_ERR_UNSUPPORTED;
    if (!w_gate || !w_up || !rot_signs || !sketch || !sketch_scale) return MOE_ERR_INVALID_ARG;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(sketch_scale, 4)) return MOE_ERR_INVALID_ARG;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t bytes = (size_t)cfg->E * 2 * cfg->H * moe::reader_row_bytes(cfg->I);
    if (hipMemsetAsync(sketch, 0, bytes, s) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(
        moe::launch_reader_sketch(cfg->E, cfg->I, cfg->H, w_gate, w_up, rot_signs, sketch, sketch_scale, s));
}

moe_status moe_down_norms(const moe_config* cfg, const uint16_t* w_down, float* down_norm, void* stream) {
    moe_status st = check_load_shape(cfg);
    if (st != MOE_OK) return st;
    if (!w_down || !down_norm || !aligned(w_down, 16) || !aligned(down_norm, 4)) return MOE_ERR_INVALID_ARG;
    return hip_status(
        moe::launch_down_norms(cfg->E, cfg->I, cfg->H, w_down, down_norm, static_cast<hipStream_t>(stream)));
}

moe_status moe_recovery_basis(const moe_config* cfg, const uint16_t* w_down, int32_t rank, int32_t iters,
                              float* basis, void* stream) {
    moe_status st = check_load_shape(cfg);
    if (st != MOE_OK) return st;
    if (rank < 1 || rank > 32 || iters < 1 || iters > 1000) return MOE_ERR_INVALID_ARG;
    if (cfg->H % 64) return MOE_ERR_UNSUPPORTED;
    if (!w_down || !basis || !aligned(w_down, 16) || !aligned(basis, 4)) return MOE_ERR_INVALID_ARG;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void* scratch_mem = nullptr;
    if (hipMalloc(&scratch_mem, moe::recovery_basis_scratch(cfg->H, rank)) != hipSuccess) return MOE_ERR_HIP;
    hipError_t e = moe::launch_recovery_basis(cfg->E, cfg->I, cfg->H, w_down, rank, iters, basis, scratch_mem, s);
    const hipError_t e2 = hipStreamSynchronize(s);
    hipFree(scratch_mem);
    return hip_status(e != hipSuccess ? e : e2);
}

moe_status moe_recovery_coefs(const moe_config* cfg, const float* basis, int32_t rank, const uint16_t* w_down,
                              uint16_t* coef, void* stream) {
    moe_status st = check_load_shape(cfg);
    if (st != MOE_OK) return st;
    if (rank < 8 || rank > 32 || rank % 8) return MOE_ERR_INVALID_ARG;
    if (!basis || !w_down || !coef || !aligned(basis, 4) || !aligned(w_down, 16) || !aligned(coef, 16))
        return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_recovery_coefs(cfg->E, cfg->I, cfg->H, basis, rank, w_down, coef,
                                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_read_device_error(moe_ctx* ctx, int32_t* flags, int32_t clear) {
    if (!ctx || !flags) return MOE_ERR_INVALID_ARG;
    if (hipDeviceSynchronize() != hipSuccess) return MOE_ERR_HIP;
    int32_t v = 0;
    if (hipMemcpy(&v, ctx->ws.err, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
    if (clear && v && hipMemset(ctx->ws.err, 0, sizeof(int32_t)) != hipSuccess) return MOE_ERR_HIP;
    *flags = v;
    return v ? MOE_ERR_DEVICE : MOE_OK;
}

moe_status moe_channel_norms(const moe_config* cfg, const uint16_t* w_gate, const uint16_t* w_up,
                             const uint16_t* w_down, float* norms, void* stream) {
    if (!cfg || !w_gate || !w_up || !w_down || !norms) return MOE_ERR_INVALID_ARG;
    if (cfg->H <= 0 || cfg->I <= 0 || cfg->E <= 0) return MOE_ERR_INVALID_ARG;
    if (cfg->H % 8 || (int64_t)cfg->E * cfg->I > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(norms, 4))
        return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_channel_norms(cfg->E, cfg->I, cfg->H, w_gate, w_up, w_down, norms,
                                                static_cast<hipStream_t>(stream)));
}

moe_status moe_validate_plan(const int32_t* ids, int32_t M, int32_t k, int32_t E, int32_t b, const int32_t* rows,
                             const int32_t* blocks, const int32_t* counts, int32_t* reason) {
    auto fail = [&](int code) {
        if (reason) *reason = code;
        return MOE_ERR_INVALID_ARG;
    };
    if (reason) *reason = 0;
    if (M < 0 || k <= 0 || E <= 0 || b <= 0) return MOE_ERR_INVALID_ARG;
    if (M > 0 && (!ids || !counts)) return MOE_ERR_INVALID_ARG;
    if (M == 0) return MOE_OK;
    const int64_t R = (int64_t)M * k;
    const int64_t cap = align_capacity64(M, k, E, b);
    const int64_t nb = counts[0], np = counts[1];
    if (nb < 0 || np != nb * b || np > cap) return fail(1);
    if (nb > 0 && (!rows || !blocks)) return MOE_ERR_INVALID_ARG;
    std::vector<int> seen((size_t)R, 0);
    int prev_e = -1;
    for (int64_t blk = 0; blk < nb; ++blk) {
        const int e = blocks[blk];
        if (e < 0 || e >= E) return fail(6);
        if (e < prev_e) return fail(6);
        prev_e = e;
        bool pad_seen = false;
        int nvalid = 0;
        for (int q = 0; q < b; ++q) {
            const int64_t r = rows[blk * b + q];
            if (r == R) {
                pad_seen = true;
                continue;
            }
            if (r < 0 || r > R) return fail(8);
            if (pad_seen) return fail(5);
            const int id = ids[r];
            if (id < 0 || id >= E) return fail(7);
            if (id != e) return fail(4);
            if (seen[(size_t)r]++) return fail(3);
            ++nvalid;
        }
        if (nvalid == 0) return fail(5);
    }
    for (int64_t r = 0; r < R; ++r)
        if (ids[r] >= 0 && ids[r] < E && !seen[(size_t)r]) return fail(2);
    return MOE_OK;
}

moe_status moe_profile_enable(moe_ctx* ctx, int32_t enable) {
    if (!ctx) return MOE_ERR_INVALID_ARG;
    ctx->prof = enable != 0;
    return MOE_OK;
}

moe_status moe_profile_read(moe_ctx* ctx, double* ms, int64_t* launches) {
    if (!ctx || !ms || !launches) return MOE_ERR_INVALID_ARG;
    moe_status st = MOE_OK;
    for (auto& r : ctx->recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
            st = MOE_ERR_HIP;
        } else {
            ms[r.kernel] += t;
            launches[r.kernel] += 1;
        }
        ctx->pool.push_back(r.a);
        ctx->pool.push_back(r.b);
    }
    ctx->recs.clear();
    return st;
}

}  // extern "C"

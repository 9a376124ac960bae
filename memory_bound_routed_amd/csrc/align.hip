// Canonical alignment of routes into padded expert blocks (page "Route-Block
// Membership Selects Packed-AWQ Arithmetic", Sec. 2.1 alignment and padded
// blocks, Sec. 3.1 Eq. 1 route-block membership, Sec. 5.3 stable (expert id,
// route id) construction).
//
// One workgroup; the bodies (align_wave for up to 64 routes, else
// align_workgroup) are shared with the router's last workgroup and documented
// in align_device.h.
#include "align_device.h"
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

__global__ void __launch_bounds__(kAlignThreads)
align_kernel(const int32_t* __restrict__ topk_ids, int R, int E, int b, int32_t* __restrict__ sorted_routes,
             int32_t* __restrict__ block_expert, int32_t* __restrict__ counts, int32_t* __restrict__ err, FastDiv fb) {
    extern __shared__ int smem[];
    if (R <= MOE_WAVE) {
        if (threadIdx.x < MOE_WAVE)
            align_wave([&](int r) { return topk_ids[r]; }, R, E, fb, sorted_routes, block_expert, counts, err);
        return;
    }
    align_workgroup([&](int r) { return topk_ids[r]; }, R, E, fb, sorted_routes, block_expert, counts, err, smem);
}

}  // namespace

size_t align_lds_bytes(int R, int E) { return align_lds_bytes_inline(R, E); }

hipError_t launch_align(const int32_t* topk_ids, int R, int E, int b, int32_t* sorted_routes,
                        int32_t* block_expert, int32_t* counts, int32_t* err, hipStream_t stream) {
    MOE_LAUNCH(align_kernel, dim3(1), dim3(kAlignThreads), align_lds_bytes(R, E), stream, topk_ids, R, E, b,
                       sorted_routes, block_expert, counts, err, FastDiv((uint32_t)b));
    return hipGetLastError();
}

}  // namespace moe

// Top-k by rank counting under a total order of (logit, expert), shared by
// the router and by the expert kernel that routes its own token (page
// "Route-Block Membership Selects Packed-AWQ Arithmetic", Sec. 2.1: the
// router's M x k expert-id array; ties go to the lower expert id).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Total-order key of (logit, expert): a larger key ranks first.  The high
// word maps the fp32 logit monotonically onto uint32 (-0 is first turned into
// +0, so equal logits give equal words), the low word is ~e, so that equal
// logits order by ascending expert id.  Keys are distinct within a token.
__device__ __forceinline__ uint64_t order_key(float l, int e) {
    uint32_t u = __float_as_uint(l + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}

// The logit and the expert a key was made from (-0 comes back as +0).
__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t hi = (uint32_t)(key >> 32);
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }

// c + (kv < o): the borrow out of the 64-bit difference kv - o, taken by a
// chain of 32-bit subtract-with-borrow operations and added as a carry.  The
// compiler turns the plain comparison into 64-bit compares and selects,
// which take several times longer on this path.
__device__ __forceinline__ int add_if_less(int c, uint64_t kv, uint64_t o) {
    uint32_t t;
    asm("v_sub_co_u32 %1, vcc, %2, %4\n\t"
        "v_subb_co_u32 %1, vcc, %3, %5, vcc\n\t"
        "v_addc_co_u32 %0, vcc, 0, %0, vcc"
        : "+v"(c), "=&v"(t)
        : "v"((uint32_t)kv), "v"((uint32_t)(kv >> 32)), "v"((uint32_t)o), "v"((uint32_t)(o >> 32))
        : "vcc");
    return c;
}

// # keys in row[j0 .. j0+n) greater than kv (n and j0 even: 16-byte pairs).
__device__ __forceinline__ int count_greater(const uint64_t* row, int j0, int n, uint64_t kv) {
    const ulonglong2* r2 = reinterpret_cast<const ulonglong2*>(row + j0);
    int c = 0;
    int q = 0;
    for (; q + 8 <= n / 2; q += 8) {  // eight 16-byte reads in flight
        ulonglong2 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = r2[q + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) c = add_if_less(add_if_less(c, kv, o[u].x), kv, o[u].y);
    }
    for (; q < n / 2; ++q) {
        const ulonglong2 o = r2[q];
        c = add_if_less(add_if_less(c, kv, o.x), kv, o.y);
    }
    return c;
}

// Renormalised softmax over the selected logits of one token, on one wave:
// lane s < k holds the logit of slot s (slot 0 the largest); returns
// exp(l_s - l_0) / sum_{s' < k} exp(l_s' - l_0), the denominator added in slot
// order.  Lanes s >= k return an unspecified value.
__device__ __forceinline__ float topk_softmax(float l, int lane, int k) {
    const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 0));
    const float x = lane < k ? expf(l - l0) : 0.f;
    float den = 0.f;
    for (int s = 0; s < k; ++s) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), s));
    return x / den;
}

}  // namespace moe

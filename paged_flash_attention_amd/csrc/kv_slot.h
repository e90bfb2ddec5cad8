// Helpers shared by the kernels that write new tokens into the page pool (the KV
// write and the fused attention input): the sequence of a token, the absmax of a
// head vector spread over D/8 lanes, and the INT8 quantiser of 8 elements.
//
// Quantiser (TileInfer.jl performance page, "INT8 KV cache": one scale per cached
// vector): scale = absmax/127 in IEEE fp32; code = clamp(rint(x/scale), +-127),
// ties to even; a zero vector gets scale 0 and codes 0.
#pragma once

#include "pfa_device.h"

namespace pfa {

// largest s with cu[s] <= tok (cu nondecreasing, cu[0] = 0)
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int batch, int tok) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (__ldg(cu + mid) <= tok) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// max over the D/8 lanes that hold one head vector
template <int D>
__device__ __forceinline__ float group_absmax(float m) {
    constexpr int L = D / 8;
    if constexpr (L >= 16) m = xor_max<8>(m);
    if constexpr (L >= 8) m = xor_max<4>(m);
    m = xor_max<2>(m);
    m = xor_max<1>(m);
    return m;
}

// The 8 codes of x at `scale`, packed into two dwords.
__device__ __forceinline__ uint2 quantise8(const float (&x)[8], float scale) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float c = 0.0f;
        if (scale > 0.0f) {
            c = __builtin_rintf(x[i] / scale);
            c = fminf(fmaxf(c, -127.0f), 127.0f);
        }
        uint32_t b = (uint32_t)((int32_t)c) & 0xffu;
        w[i >> 2] |= b << (8 * (i & 3));
    }
    return make_uint2(w[0], w[1]);
}

}  // namespace pfa

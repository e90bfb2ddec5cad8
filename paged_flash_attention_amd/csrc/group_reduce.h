// Cross-lane helpers of the split-KV decode kernels (BF16/INT8 and 3-bit): the
// transposed butterfly that reduces the G heads' partial dots of a key over the
// lanes that hold the key, and a wave-uniform read of one lane's value.
#pragma once

#include "pfa_device.h"

namespace pfa {

// Transposed butterfly over the LPK lanes of a key group.  On entry, slot j of
// this lane holds its partial sum for head (j ^ myhead).  On return, slot 0 holds
// this lane's head's full sum over all D dims.
template <int LPK, int G>
__device__ __forceinline__ float transpose_reduce(float (&acc)[G]) {
    if constexpr (G >= 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += xor_lane<LPK / 2>(acc[j + 8]);
    }
    constexpr int M8 = (G >= 16) ? LPK / 4 : LPK / 2;
    if constexpr (G >= 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += xor_lane<M8>(acc[j + 4]);
    }
    constexpr int M4 = (G >= 8) ? M8 / 2 : LPK / 2;
    if constexpr (G >= 4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] += xor_lane<M4>(acc[j + 2]);
    }
    constexpr int M2 = (G >= 4) ? M4 / 2 : LPK / 2;
    if constexpr (G >= 2) acc[0] += xor_lane<M2>(acc[1]);
    constexpr int R = (G >= 2) ? M2 / 2 : LPK / 2;
    float s = acc[0];
    if constexpr (R >= 8) s += xor_lane<8>(s);
    if constexpr (R >= 4) s += xor_lane<4>(s);
    if constexpr (R >= 2) s += xor_lane<2>(s);
    if constexpr (R >= 1) s += xor_lane<1>(s);
    return s;
}

__device__ __forceinline__ float lane_read(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

}  // namespace pfa

// Cross-lane helpers of the split-KV decode kernels (BF16/INT8 and 3-bit): the
// transposed butterfly that reduces the G heads' partial dots of a key over the
// lanes that hold the key, and a wave-uniform read of one lane's value.
#pragma once

#include "pfa_device.h"

namespace pfa {

// Transposed butterfly over the LPK lanes of a key group (LPK = 16 or 8), on the
// VALU only (DPP moves, no LDS).  On entry, slot j of this lane holds its partial
// sum for head (j ^ myhead), myhead = (lane % LPK) / (LPK / G).  On return, slot 0
// holds this lane's head's full sum over the group.  (A "head" is any of G sums
// the group shares: G = LPK, two keys of 8 heads each, leaves every lane a sum of
// its own.)
//
// Each stage adds the partner's slot j ^ delta to slot j for the lower half of the
// live slots.  The partner is lane ^ m, with m = 15 (row mirror), 7 (half-row
// mirror), 2, 1 (quad permutes) for LPK = 16, and 7, 2, 1 for LPK = 8; its head is
// myhead ^ delta with delta = m / (LPK / G).  In that order delta's top bit is
// always the upper half of the live slots (or delta = 0 once one slot is left),
// and the masks span the whole group.
template <int M>
__device__ __forceinline__ float dpp_xor(float x) {
    // row_mirror: i <- 15 - i; row_half_mirror: i <- 7 - i; quad_perm [2,3,0,1]; [1,0,3,2]
    constexpr int ctrl = M == 15 ? 0x140 : M == 7 ? 0x141 : M == 2 ? 0x4E : 0xB1;
    static_assert(M == 15 || M == 7 || M == 2 || M == 1, "DPP partner");
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, true));
}

template <int LPK, int G, int M, int N>
__device__ __forceinline__ void mirror_stage(float (&acc)[G]) {
    constexpr int HG = LPK / G;
    constexpr int delta = M / HG;
    if constexpr (N > 1) {
        static_assert(delta >= N / 2 && delta < N, "stage order");
#pragma unroll
        for (int j = 0; j < N / 2; ++j) acc[j] += dpp_xor<M>(acc[j ^ delta]);
    } else {
        static_assert(delta == 0, "stage order");
        acc[0] += dpp_xor<M>(acc[0]);
    }
}

template <int LPK, int G>
__device__ __forceinline__ float transpose_reduce(float (&acc)[G]) {
    static_assert(LPK == 16 || LPK == 8, "lanes per key");
    static_assert(G >= 1 && G <= LPK, "group size");
    constexpr int N1 = G, N2 = N1 > 1 ? N1 / 2 : 1, N3 = N2 > 1 ? N2 / 2 : 1, N4 = N3 > 1 ? N3 / 2 : 1;
    if constexpr (LPK == 16) {
        mirror_stage<LPK, G, 15, N1>(acc);
        mirror_stage<LPK, G, 7, N2>(acc);
        mirror_stage<LPK, G, 2, N3>(acc);
        mirror_stage<LPK, G, 1, N4>(acc);
    } else {
        mirror_stage<LPK, G, 7, N1>(acc);
        mirror_stage<LPK, G, 2, N2>(acc);
        mirror_stage<LPK, G, 1, N3>(acc);
    }
    return acc[0];
}

__device__ __forceinline__ float lane_read(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

}  // namespace pfa

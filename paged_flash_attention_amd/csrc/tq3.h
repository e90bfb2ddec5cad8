// 3-bit rotated KV cache: the device side of the format.
//
// The qengine README's feature list names a 3-bit KV cache made of a
// Walsh-Hadamard rotation and a Lloyd-Max scalar quantiser.  The format here:
//  * each cached K or V vector x (D elements) is rotated, y = H_D x (Sylvester
//    order, unnormalised; the inverse is H_D / D);
//  * one fp32 scale per vector, s = sqrt(sum(y^2) / D) (the RMS of y, = ||x||);
//  * each t = y/s is coded by the symmetric 8-level Lloyd-Max quantiser of the unit
//    normal: levels +-M[0..3], thresholds 0, +-T[0..2].  Code bits 0-1 are the
//    magnitude index m = #{k : |t| >= T[k]}, bit 2 is 1 when t >= 0 (a zero vector
//    takes t = 0);
//  * the codes of a vector are packed as D/8 little-endian 24-bit fields of 3
//    bytes: field j holds elements 8j .. 8j+7, element 8j+i in bits 3i .. 3i+2
//    (3D/8 bytes per vector), so a lane's 8 codes are its own 3 bytes;
//  * the cache holds x^ = H_D (s * c) / D with c = +-M[m].
// The code decisions are made in fp32 in one fixed order (butterflies by stride 1,
// 2, ..., D/2; squares summed by 8 in order, then the groups in a pairwise tree;
// correctly rounded sqrt and divide), so that they are reproducible bit for bit.
//
// A lane owns 8 consecutive elements (group g = elements 8g .. 8g+7), and the
// L = D/8 lanes of one vector are consecutive lanes of a wave.
#pragma once

#include "pfa_device.h"

namespace pfa {

// y = H_D x over the L lanes of a vector, in place: butterflies of stride 1, 2, 4
// inside the lane, then 8, 16, ... across lanes.  At each butterfly the element
// with the stride bit clear (a) and its partner (b) become a + b and a - b.
template <int L>
__device__ __forceinline__ void fwht_lanes(float (&x)[8], int g) {
#pragma unroll
    for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!(e & h)) {
                const float a = x[e], b = x[e + h];
                x[e] = a + b;
                x[e + h] = a - b;
            }
    auto stage = [&](auto mc) __attribute__((always_inline)) {
        constexpr int M = decltype(mc)::value;
        const bool upper = (g & M) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = xor_lane<M>(x[i]);
            x[i] = upper ? p - x[i] : x[i] + p;
        }
    };
    if constexpr (L >= 2) stage(std::integral_constant<int, 1>{});
    if constexpr (L >= 4) stage(std::integral_constant<int, 2>{});
    if constexpr (L >= 8) stage(std::integral_constant<int, 4>{});
    if constexpr (L >= 16) stage(std::integral_constant<int, 8>{});
}

// sum of y^2 over the vector: the lane's 8 squares in order, then the lane sums
// in a pairwise tree (partner g ^ 1, then g ^ 2, ...).  Every lane gets the total.
template <int L>
__device__ __forceinline__ float sum_squares_lanes(const float (&y)[8]) {
#pragma clang fp contract(off)
    float s = y[0] * y[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) s = s + y[i] * y[i];
    if constexpr (L >= 2) s = s + xor_lane<1>(s);
    if constexpr (L >= 4) s = s + xor_lane<2>(s);
    if constexpr (L >= 8) s = s + xor_lane<4>(s);
    if constexpr (L >= 16) s = s + xor_lane<8>(s);
    return s;
}

// Quantise the lane's 8 rotated elements at scale s; returns their 24-bit field.
__device__ __forceinline__ uint32_t tq3_codes8(const float (&y)[8], float s, const Tq3Book& bk) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = s == 0.0f ? 0.0f : y[i] / s;
        const float a = fabsf(t);
        const uint32_t m = (uint32_t)(a >= bk.t[0]) + (uint32_t)(a >= bk.t[1]) + (uint32_t)(a >= bk.t[2]);
        const uint32_t pos = t >= 0.0f ? 1u : 0u;
        w |= (m | (pos << 2)) << (3 * i);
    }
    return w;
}

// The level of a code: codes 0..3 are -M[0..3], codes 4..7 are +M[0..3].
__device__ __forceinline__ float tq3_level_of(int code, const Tq3Book& bk) {
    const float lo = (code & 1) ? bk.m[1] : bk.m[0];
    const float hi = (code & 1) ? bk.m[3] : bk.m[2];
    const float mag = (code & 2) ? hi : lo;
    return (code & 4) ? mag : -mag;
}

// The 8 levels of a field, looked up in a level table in LDS.
__device__ __forceinline__ void tq3_levels8(uint32_t w, const float* table, float (&c)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = table[(w >> (3 * i)) & 7u];
}

}  // namespace pfa

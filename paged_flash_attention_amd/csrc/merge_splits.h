// Merge of one (row, query head)'s split partials into its output row, by one
// 64-lane wave.  This is the combine of the TileInfer.jl performance page ("Fused
// kernels, FlashAttention and PagedAttention"):
//   M   = max(max_i lse_i, sink)
//   out = sum_i e^(lse_i - M) o_i / (sum_i e^(lse_i - M) + e^(sink - M))
// with the sink terms only when a sink is given.  Both the combine kernel and the
// fused decode (the last split of a KV head merges its query heads one by one)
// call this, so the two paths give the same bits.  (Merging the G heads of a KV
// head at once, 64/G lanes each, measured slower in the fused decode.)
//  * The lanes read the lse values in parallel for the max and the weight sum,
//    and put the weights in LDS, CHUNK splits at a time.
//  * Every lane owns D/64 consecutive elements and walks the splits in order,
//    8 rows in flight, each split's o row read as one coalesced D*4-byte access.
//  * Splits with lse = -inf weigh 0.  The leading run of them (the splits a
//    window hides) is skipped without reading their o rows, which decode leaves
//    unwritten.
#pragma once

#include "pfa_device.h"

namespace pfa {

// COHERENT: read lse and o with agent-scope atomic loads (coherent across the
// XCDs' L2 caches with no cache maintenance), for partials other workgroups wrote
// during the same kernel.
template <bool COHERENT>
__device__ __forceinline__ float load_part(const float* p) {
    if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}

template <int D, int CHUNK, bool COHERENT = false>
__device__ __forceinline__ void merge_splits(const float* lse, const float* op, int ns, const float* sink_p,
                                             float* w_lds, float* out) {
    const int lane = (int)__lane_id();
    float m = -INFINITY;
    float first = (float)ns;
    for (int i = lane; i < ns; i += kWave) {
        const float l = load_part<COHERENT>(lse + i);
        m = fmaxf(m, l);
        if (l != -INFINITY) first = fminf(first, (float)i);
    }
    m = stride_max<1>(m);
    const int i_first = (int)-stride_max<1>(-first);
    const bool has_sink = sink_p != nullptr;
    const float sink = has_sink ? __ldg(sink_p) : -INFINITY;
    if (has_sink) m = fmaxf(m, sink);
    const float ms = (m == -INFINITY) ? 0.0f : m;

    constexpr int E = D / kWave;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    float wsum = 0.0f;
    for (int base = i_first; base < ns; base += CHUNK) {
        const int cnt = min(ns - base, CHUNK);
        for (int i = lane; i < cnt; i += kWave) {
            const float w = __expf(load_part<COHERENT>(lse + base + i) - ms);   // 0 for lse = -inf
            w_lds[i] = w;
            wsum += w;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const float* row = op + (int64_t)base * D + lane * E;
        int i = 0;
        for (; i + 8 <= cnt; i += 8) {
            float v[8][E];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e) v[u][e] = load_part<COHERENT>(row + (int64_t)(i + u) * D + e);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float w = w_lds[i + u];
#pragma unroll
                for (int e = 0; e < E; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
            }
        }
        for (; i < cnt; ++i) {
            const float w = w_lds[i];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(w, load_part<COHERENT>(row + (int64_t)i * D + e), acc[e]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    wsum = stride_sum<1>(wsum);
    const float z = wsum + (has_sink ? __expf(sink - ms) : 0.0f);
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
    float* o = out + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = acc[e] * inv;
}

}  // namespace pfa

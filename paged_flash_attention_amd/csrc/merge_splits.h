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

// The same merge for E * 64 elements of D (a lane per E consecutive elements: one
// 64-element slice, or E = D/64 for a whole row) and a split count known to be
// at most NS <= 128, with every load issued before the loads' first use: the lse
// values (NS/64 per lane), then the lane's elements of every o row.  The loads go
// through buffer resources that end at row ns, so rows past the count read 0
// with no memory access and no branch.  The arithmetic is merge_splits' in the
// same order, so the two give the same bits: split i's weight e^(lse_i - M) is
// broadcast for the fma of row i; lane L sums the weights of splits i_first + L
// and i_first + L + 64, as the chunked loop does; rows outside [i_first, ns)
// take no fma (the window-hidden ones were never written).  op and out point at
// the lane group's first element in row 0; rows are D floats apart.
template <int D, int NS, int E = 1, bool COHERENT = false>
__device__ __forceinline__ void merge_splits_short(const float* lse, const float* op, int ns, const float* sink_p,
                                                   float* out) {
    static_assert(NS >= 1 && NS <= 2 * kWave, "at most two lse per lane");
    static_assert((E == 1 || E == 2) && NS * E <= 128, "registers");
    constexpr int K = NS > kWave ? 2 : 1;                // lse values per lane
    constexpr int kAux = COHERENT ? 16 : 0;              // sc1: agent-coherent load
    const int lane = (int)__lane_id();
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)lse, 0, ns * 4, 0x00020000);
    const int o_bytes = ns > 0 ? ((ns - 1) * D + kWave * E) * 4 : 0;    // through row ns-1's elements
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)op, 0, o_bytes, 0x00020000);
    float l[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        l[k] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (k * kWave + lane) * 4, 0, kAux));
    float v[NS][E];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int off = (u * D + lane * E) * 4;
        if constexpr (E == 2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(ro, off, 0, kAux);
            v[u][0] = __uint_as_float(x[0]);
            v[u][1] = __uint_as_float(x[1]);
        } else {
            v[u][0] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, off, 0, kAux));
        }
    }

    float m = -INFINITY, first = (float)ns;
#pragma unroll
    for (int k = K - 1; k >= 0; --k) {
        if (k * kWave + lane >= ns) l[k] = -INFINITY;
        m = fmaxf(m, l[k]);
        if (l[k] != -INFINITY) first = (float)(k * kWave + lane);
    }
    m = stride_max<1>(m);
    const int i_first = __builtin_amdgcn_readfirstlane((int)-stride_max<1>(-first));   // same in every lane
    const bool has_sink = sink_p != nullptr;
    const float sink = has_sink ? __ldg(sink_p) : -INFINITY;
    if (has_sink) m = fmaxf(m, sink);
    const float ms = (m == -INFINITY) ? 0.0f : m;
    float w[K];
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = __expf(l[k] - ms);   // 0 past the count and for lse = -inf
    // lane L: w(j) + w(j + 64) for j = i_first + L, each term only below ns
    const int j = i_first + lane;
    const int src = (j & (kWave - 1)) * 4;
    const float a0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(w[0])));
    float part = j < ns ? a0 : 0.0f;
    if constexpr (K == 2) {
        const float a1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(w[1])));
        const float wa = j < kWave ? a0 : a1;
        part = (j < ns ? wa : 0.0f) + (j + kWave < ns ? a1 : 0.0f);
    }
    const float wsum = stride_sum<1>(part);

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        // a select, not a branch: a branch lets the compiler sink row i's load
        // into it, and the rows would then arrive one round trip at a time
        const bool take = i >= i_first && i < ns;
        const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[i / kWave]), i % kWave));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = take ? fmaf(wi, v[i][e], acc[e]) : acc[e];
    }
    const float z = wsum + (has_sink ? __expf(sink - ms) : 0.0f);
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) out[lane * E + e] = acc[e] * inv;
}

// merge_splits_short at the smallest depth of NS, NS/2, ..., 8 that holds this
// row's ns (the branch is uniform and comes before any load).
template <int D, int NS, int E = 1, bool COHERENT = false>
__device__ __forceinline__ void merge_splits_short_any(const float* lse, const float* op, int ns, const float* sink_p,
                                                       float* out) {
    if constexpr (NS > 8) {
        if (ns <= NS / 2) {
            merge_splits_short_any<D, NS / 2, E, COHERENT>(lse, op, ns, sink_p, out);
            return;
        }
    }
    merge_splits_short<D, NS, E, COHERENT>(lse, op, ns, sink_p, out);
}

}  // namespace pfa

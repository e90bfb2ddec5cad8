// Combine: merge split-KV partials into the final output.
//
// The TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") keeps this merge as a separate kernel after the split-KV decode.
// It measured the variant that fuses it into the split kernel, through an
// acquire-release counter, as 2% slower.  For each (row r, query head h):
//   M   = max(max_i lse_i, sink_h)
//   out = sum_i e^(lse_i - M) o_i / (sum_i e^(lse_i - M) + e^(sink_h - M))
// The sink terms appear only when sinks are given.  For decode a row is a
// sequence, and its ceil(len/S) splits are merged.  For split prefill a row is a
// query token, located through cu_rows, and all max_splits are merged; splits with
// no visible key carry lse = -inf and weigh 0.  The leading run of such splits
// is skipped without reading its o rows.
//
// One 64-lane wave per (row, h):
//  * the lanes take the splits' lse values in parallel for the max and the weight
//    sum, and put the weights in LDS;
//  * then every lane owns D/64 consecutive elements and walks the splits, 8 rows
//    in flight, each split's o_part row read as one coalesced D*4-byte access.
// The work is tiny: rows*Hq*splits*(D+1)*4 bytes read.
#include "pfa_device.h"

namespace pfa {
namespace {

constexpr int kMaxLdsSplits = 1024;

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
    __shared__ float w_lds[kMaxLdsSplits];
    const int h = blockIdx.x % a.num_q_heads;
    const int r = blockIdx.x / a.num_q_heads;
    const int lane = threadIdx.x;
    int row = r;
    int ns = a.max_splits;
    if (a.cu_rows) {
        const int s = r / a.rows_per_seq, t = r % a.rows_per_seq;
        const int c0 = __ldg(a.cu_rows + s);
        if (t >= __ldg(a.cu_rows + s + 1) - c0) return;
        row = c0 + t;
    } else if (a.seq_lens) {
        const int len = __ldg(a.seq_lens + r);
        ns = min((len + a.split_keys - 1) / a.split_keys, a.max_splits);
    }
    const int64_t bh = (int64_t)row * a.num_q_heads + h;
    const float* lse = a.lse_part + (int64_t)bh * a.max_splits;
    const float* op = a.o_part + (int64_t)bh * a.max_splits * D;

    // max, and the first split with a visible key: decode leaves the o rows of the
    // splits a window hides (always a prefix) unwritten, so they are never read
    float m = -INFINITY;
    float first = (float)ns;
    for (int i = lane; i < ns; i += kWave) {
        const float l = lse[i];
        m = fmaxf(m, l);
        if (l != -INFINITY) first = fminf(first, (float)i);
    }
    m = stride_max<1>(m);
    const int i_first = (int)-stride_max<1>(-first);
    const bool has_sink = a.sinks != nullptr;
    const float sink = has_sink ? __ldg(a.sinks + h) : -INFINITY;
    m = fmaxf(m, sink);
    const float ms = (m == -INFINITY) ? 0.0f : m;

    constexpr int E = D / kWave;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    float wsum = 0.0f;
    for (int base = i_first; base < ns; base += kMaxLdsSplits) {
        const int cnt = min(ns - base, kMaxLdsSplits);
        for (int i = lane; i < cnt; i += kWave) {
            const float w = __expf(lse[base + i] - ms);      // 0 for lse = -inf
            w_lds[i] = w;
            wsum += w;
        }
        __syncthreads();
        const float* row = op + (int64_t)base * D + lane * E;
        int i = 0;
        for (; i + 8 <= cnt; i += 8) {
            float v[8][E];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e) v[u][e] = row[(int64_t)(i + u) * D + e];
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
            for (int e = 0; e < E; ++e) acc[e] = fmaf(w, row[(int64_t)i * D + e], acc[e]);
        }
        __syncthreads();
    }
    wsum = stride_sum<1>(wsum);
    const float z = wsum + (has_sink ? __expf(sink - ms) : 0.0f);
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
    float* o = a.out + (int64_t)bh * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = acc[e] * inv;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s) {
    const int64_t rows = a.cu_rows ? (int64_t)a.batch * a.rows_per_seq : a.batch;
    const unsigned grid = (unsigned)(rows * a.num_q_heads);
    if (grid == 0) return hipSuccess;
    if (head_dim == 128)
        hipLaunchKernelGGL((combine_kernel<128>), dim3(grid), dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((combine_kernel<64>), dim3(grid), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace pfa

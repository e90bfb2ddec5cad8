// Combine: merge split-KV decode partials into the final output.
//
// The TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") keeps this merge as a separate kernel after the split-KV decode.
// It measured the variant that fuses it into the split kernel, through an
// acquire-release counter, as 2% slower.  For each (sequence b, query head h):
//   M   = max(max_i lse_i, sink_h)
//   out = sum_i e^(lse_i - M) o_i / (sum_i e^(lse_i - M) + e^(sink_h - M))
// over the ceil(len/S) splits of b.  The sink terms appear only when sinks are
// given.
//
// One 64-lane wave per (b, h).  Lanes stride over the splits' lse values for the
// max; then every lane owns D/64 consecutive elements and walks the splits, so each
// split's o_part row is read as one coalesced D*4-byte access.  Work is tiny:
// B*Hq*splits*(D+1)*4 bytes read.
#include "pfa_device.h"

namespace pfa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
    const int bh = blockIdx.x;
    const int b = bh / a.num_q_heads;
    const int h = bh % a.num_q_heads;
    const int lane = threadIdx.x;
    const int len = __ldg(a.seq_lens + b);
    int ns = (len + a.split_keys - 1) / a.split_keys;
    ns = ns < a.max_splits ? ns : a.max_splits;
    const float* lse = a.lse_part + (int64_t)bh * a.max_splits;
    const float* op = a.o_part + (int64_t)bh * a.max_splits * D;

    float m = -INFINITY;
    for (int i = lane; i < ns; i += kWave) m = fmaxf(m, lse[i]);
    m = stride_max<1>(m);
    const bool has_sink = a.sinks != nullptr;
    const float sink = has_sink ? __ldg(a.sinks + h) : -INFINITY;
    m = fmaxf(m, sink);
    const float ms = (m == -INFINITY) ? 0.0f : m;

    // each lane owns D/64 elements
    constexpr int E = D / kWave;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    float wsum = 0.0f;
    for (int i = 0; i < ns; ++i) {
        const float l = lse[i];
        const float w = (l == -INFINITY) ? 0.0f : __expf(l - ms);
        wsum += w;
        if (w != 0.0f) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += w * op[(int64_t)i * D + lane * E + e];
        }
    }
    float z = wsum + (has_sink ? __expf(sink - ms) : 0.0f);
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
    float* o = a.out + (int64_t)bh * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = acc[e] * inv;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s) {
    const unsigned grid = (unsigned)a.batch * (unsigned)a.num_q_heads;
    if (grid == 0) return hipSuccess;
    if (head_dim == 128)
        hipLaunchKernelGGL((combine_kernel<128>), dim3(grid), dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((combine_kernel<64>), dim3(grid), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace pfa

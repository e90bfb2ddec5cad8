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
// One 64-lane wave per (row, h) runs merge_splits (merge_splits.h).
// The work is tiny: rows*Hq*splits*(D+1)*4 bytes read.
#include "merge_splits.h"

namespace pfa {
namespace {

constexpr int kMaxLdsSplits = 1024;

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
    __shared__ float w_lds[kMaxLdsSplits];
    const int h = blockIdx.x % a.num_q_heads;
    const int r = blockIdx.x / a.num_q_heads;
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
    merge_splits<D, kMaxLdsSplits>(a.lse_part + bh * a.max_splits, a.o_part + bh * a.max_splits * D, ns,
                                   a.sinks ? a.sinks + h : nullptr, w_lds, a.out + bh * D);
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

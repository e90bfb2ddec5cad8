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
// Up to 128 splits, merge_splits_short has all the row's partials in flight at
// once, at the smallest depth of 8, 16, 32, 64 and 128 that holds the row's split
// count; one 64-lane wave takes a 64-element slice of D where (row, h) items are
// fewer than 8192, else the whole row.  Above 128 splits, one wave per (row, h)
// runs the chunked merge_splits (merge_splits.h).  All give the same bits.
// The work is tiny: rows*Hq*splits*(D+1)*4 bytes read, so the time is latency.
#include "merge_splits.h"

namespace pfa {
namespace {

constexpr int kMaxLdsSplits = 1024;

// NS > 0: every row has at most NS <= 128 splits, merged by merge_splits_short at
// the depth the row needs; a wave takes one 64-element slice of D (SLICE) or the
// whole row.  NS = 0: any count, a wave per (row, head) through the chunked merge.
template <int D, int NS, bool SLICE>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
    __shared__ float w_lds[NS > 0 ? 1 : kMaxLdsSplits];
    constexpr int kSlices = (NS > 0 && SLICE) ? D / kWave : 1;
    constexpr int E = D / (kWave * kSlices);     // elements per lane: D/64 for a whole row
    const int slice = blockIdx.x % kSlices;
    const int bh_id = blockIdx.x / kSlices;
    const int h = bh_id % a.num_q_heads;
    const int r = bh_id / a.num_q_heads;
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
    const float* lse = a.lse_part + bh * a.max_splits;
    const float* op = a.o_part + bh * a.max_splits * D;
    const float* sink = a.sinks ? a.sinks + h : nullptr;
    if constexpr (NS > 0)
        merge_splits_short_any<D, NS, E>(lse, op + slice * kWave, max(ns, 0), sink, a.out + bh * D + slice * kWave);
    else
        merge_splits<D, kMaxLdsSplits>(lse, op, ns, sink, w_lds, a.out + bh * D);
}

// Slices pay where (row, head) items are few: the headline decode's 1024 items
// run as 2048 waves.  Where items are many (a 1024-token prefill chunk: 32768)
// a second wave per item only repeats the prologue, and the whole row goes to
// one wave (at D = 128 and up to 64 splits, whose 2 x 64 row registers fit).
constexpr int64_t kSliceBelow = 8192;

template <int D, bool SLICE>
hipError_t launch_ds(const CombineArgs& a, unsigned bh, hipStream_t s) {
    const int n = a.max_splits;
    const dim3 g(bh * (SLICE ? D / kWave : 1)), b(64);
    if (n <= 8) hipLaunchKernelGGL((combine_kernel<D, 8, SLICE>), g, b, 0, s, a);
    else if (n <= 16) hipLaunchKernelGGL((combine_kernel<D, 16, SLICE>), g, b, 0, s, a);
    else if (n <= 32) hipLaunchKernelGGL((combine_kernel<D, 32, SLICE>), g, b, 0, s, a);
    else if (n <= 64) hipLaunchKernelGGL((combine_kernel<D, 64, SLICE>), g, b, 0, s, a);
    else if (n <= 128 && SLICE) hipLaunchKernelGGL((combine_kernel<D, 128, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<D, 0, false>), dim3(bh), b, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const CombineArgs& a, unsigned bh, hipStream_t s) {
    if constexpr (D == 64) {
        return launch_ds<D, true>(a, bh, s);   // one slice is the whole row
    } else {
        const bool slice = (int64_t)bh < kSliceBelow || a.max_splits > 64;
        return slice ? launch_ds<D, true>(a, bh, s) : launch_ds<D, false>(a, bh, s);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s) {
    const int64_t rows = a.cu_rows ? (int64_t)a.batch * a.rows_per_seq : a.batch;
    const int64_t n = rows * a.num_q_heads;
    if (n == 0) return hipSuccess;
    if (n * (head_dim / kWave) > 0x7fffffff) return hipErrorInvalidValue;
    const unsigned bh = (unsigned)n;
    return head_dim == 128 ? launch_d<128>(a, bh, s) : launch_d<64>(a, bh, s);
}

}  // namespace pfa

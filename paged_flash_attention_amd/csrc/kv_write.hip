// KV write: scatter new tokens' K/V rows into their pages.
//
// The TileInfer.jl performance page lists the KV cache write among the engine's
// per-op kernels ("Fused kernels, FlashAttention and PagedAttention").  Its
// "INT8 KV cache" section stores one scale per cached vector.  For BF16 pools this
// kernel copies the bits.  For INT8 pools it quantises each (token, KV head) vector:
//   scale = absmax/127 in IEEE fp32;
//   code  = clamp(rint(x/scale), +-127), ties to even;
//   a zero vector gets scale 0.
// With a key smoothing vector s (same section: keys smoothed by the key norm's
// weight), a key vector is divided by s per channel (IEEE fp32) before that.
//
// For 3-bit rotated pools (tq3.h) it rotates each vector by the Walsh-Hadamard
// transform, takes its RMS as the scale and writes the 3-bit codes in 24-bit
// fields, with the decisions in fp32 in the fixed order tq3.h gives.
//
// Each thread owns 8 consecutive elements (16 B of bf16 input) of one vector for
// both K and V, so D/8 lanes share a vector.  The absmax is a max over those lanes
// with DPP/swizzle moves.  Loads and stores are 16 B (codes: 8 B) per lane and are
// contiguous across the lanes of a vector.  The kernel is HBM-bound: it reads
// 2*D*2 B and writes 2*D*b B (+8 B scales) per (token, head).
#include "kv_slot.h"
#include "tq3.h"

namespace pfa {
namespace {

template <int D, bool INT8>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
    constexpr int L = D / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t vec = t / L;
    const int chunk = (int)(t % L);
    const int64_t nvec = (int64_t)a.num_tokens * a.num_kv_heads;
    bool ok = vec < nvec;
    int tok = 0, head = 0;
    int64_t dst = 0;  // element index of this lane's chunk in the pool
    int64_t sdst = 0; // scale index
    if (ok) {
        tok = (int)(vec / a.num_kv_heads);
        head = (int)(vec % a.num_kv_heads);
        const int s = find_seq(a.cu_new, a.batch, tok);
        const int c0 = __ldg(a.cu_new + s), c1 = __ldg(a.cu_new + s + 1);
        const int pos = __ldg(a.seq_lens + s) - (c1 - c0) + (tok - c0);
        const int pidx = pos / kPage;
        report(a.err, pos < 0, PFA_BOUNDS_Q_LEN);
        report(a.err, pos >= 0 && pidx >= a.bt_stride, PFA_BOUNDS_SEQ_LEN);
        ok = tok < c1 && pos >= 0 && pidx < a.bt_stride;
        if (ok) {
            const int page = __ldg(a.block_table + (int64_t)s * a.bt_stride + pidx);
            ok = page >= 0 && page < a.num_pages;
            report(a.err, !ok, PFA_BOUNDS_PAGE);
            sdst = ((int64_t)page * a.num_kv_heads + head) * kPage + (pos % kPage);
            dst = sdst * D + chunk * 8;
        }
    }
    const int64_t src = vec * D + chunk * 8;
    uint4 kin = make_uint4(0, 0, 0, 0), vin = make_uint4(0, 0, 0, 0);
    if (vec < nvec) {
        kin = *reinterpret_cast<const uint4*>(a.k_new + src);
        vin = *reinterpret_cast<const uint4*>(a.v_new + src);
    }
    if constexpr (!INT8) {
        if (ok) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.k_pool) + dst) = kin;
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.v_pool) + dst) = vin;
        }
    } else {
        float kx[8], vx[8];
        const uint32_t kw[4] = {kin.x, kin.y, kin.z, kin.w};
        const uint32_t vw[4] = {vin.x, vin.y, vin.z, vin.w};
        float km = 0.0f, vm = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kx[2 * i] = bf16_lo(kw[i]);
            kx[2 * i + 1] = bf16_hi(kw[i]);
            vx[2 * i] = bf16_lo(vw[i]);
            vx[2 * i + 1] = bf16_hi(vw[i]);
        }
        if (a.k_smooth) {   // keys smoothed per channel: quantise k / s, s a power of two (exact)
            const float4* sp = reinterpret_cast<const float4*>(a.k_smooth + chunk * 8);
            const float4 s0 = __ldg(sp), s1 = __ldg(sp + 1);
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) kx[i] = kx[i] / smooth_pow2(sv[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            km = fmaxf(km, fabsf(kx[i]));
            vm = fmaxf(vm, fabsf(vx[i]));
        }
        km = group_absmax<D>(km);
        vm = group_absmax<D>(vm);
        const float ks = km / 127.0f;
        const float vs = vm / 127.0f;
        const uint2 kc = quantise8(kx, ks);
        const uint2 vc = quantise8(vx, vs);
        if (ok) {
            *reinterpret_cast<uint2*>(static_cast<int8_t*>(a.k_pool) + dst) = kc;
            *reinterpret_cast<uint2*>(static_cast<int8_t*>(a.v_pool) + dst) = vc;
            if (chunk == 0) {
                a.k_scale[sdst] = ks;
                a.v_scale[sdst] = vs;
            }
        }
    }
}

// 3-bit rotated pools: same lane layout as above.  A vector's codes are 3D/8
// bytes; lane g writes its 24-bit field, bytes 3g .. 3g+2.
template <int D>
__global__ __launch_bounds__(256) void kv_write_tq3_kernel(KvWriteArgs a) {
    constexpr int L = D / 8;
    constexpr int VB = 3 * D / 8;           // bytes per vector
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t vec = t / L;
    const int g = (int)(t % L);
    const int64_t nvec = (int64_t)a.num_tokens * a.num_kv_heads;
    bool ok = vec < nvec;
    int64_t sdst = 0;   // slot index: (page, head, offset)
    if (ok) {
        const int tok = (int)(vec / a.num_kv_heads);
        const int head = (int)(vec % a.num_kv_heads);
        const int s = find_seq(a.cu_new, a.batch, tok);
        const int c0 = __ldg(a.cu_new + s), c1 = __ldg(a.cu_new + s + 1);
        const int pos = __ldg(a.seq_lens + s) - (c1 - c0) + (tok - c0);
        const int pidx = pos / kPage;
        report(a.err, pos < 0, PFA_BOUNDS_Q_LEN);
        report(a.err, pos >= 0 && pidx >= a.bt_stride, PFA_BOUNDS_SEQ_LEN);
        ok = tok < c1 && pos >= 0 && pidx < a.bt_stride;
        if (ok) {
            const int page = __ldg(a.block_table + (int64_t)s * a.bt_stride + pidx);
            ok = page >= 0 && page < a.num_pages;
            report(a.err, !ok, PFA_BOUNDS_PAGE);
            sdst = ((int64_t)page * a.num_kv_heads + head) * kPage + (pos % kPage);
        }
    }
    // every lane of a vector takes part in the cross-lane steps, so a lane past the
    // last vector computes on zeros and stores nothing
    const int64_t src = min(vec, nvec - 1) * D + g * 8;
    const uint4 kin = *reinterpret_cast<const uint4*>(a.k_new + src);
    const uint4 vin = *reinterpret_cast<const uint4*>(a.v_new + src);
    auto encode = [&](const uint4& in, uint8_t* pool, float* scale) __attribute__((always_inline)) {
        const uint32_t w[4] = {in.x, in.y, in.z, in.w};
        float y[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[2 * i] = bf16_lo(w[i]);
            y[2 * i + 1] = bf16_hi(w[i]);
        }
        fwht_lanes<L>(y, g);
        const float sc = __builtin_sqrtf(sum_squares_lanes<L>(y) / (float)D);
        const uint32_t field = tq3_codes8(y, sc, a.book);
        if (ok) {
            uint8_t* dst = pool + sdst * VB + 3 * g;
            dst[0] = (uint8_t)field;
            dst[1] = (uint8_t)(field >> 8);
            dst[2] = (uint8_t)(field >> 16);
            if (g == 0) scale[sdst] = sc;
        }
    };
    encode(kin, static_cast<uint8_t*>(a.k_pool), a.k_scale);
    encode(vin, static_cast<uint8_t*>(a.v_pool), a.v_scale);
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs& a, int kv_dtype, hipStream_t s) {
    const int64_t threads = (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / 8);
    if (threads == 0) return hipSuccess;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (a.head_dim == 128) {
        if (kv_dtype == 2) hipLaunchKernelGGL((kv_write_tq3_kernel<128>), dim3(grid), dim3(256), 0, s, a);
        else if (kv_dtype == 1) hipLaunchKernelGGL((kv_write_kernel<128, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((kv_write_kernel<128, false>), dim3(grid), dim3(256), 0, s, a);
    } else {
        if (kv_dtype == 2) hipLaunchKernelGGL((kv_write_tq3_kernel<64>), dim3(grid), dim3(256), 0, s, a);
        else if (kv_dtype == 1) hipLaunchKernelGGL((kv_write_kernel<64, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((kv_write_kernel<64, false>), dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace pfa

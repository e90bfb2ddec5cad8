// Fused attention input: q/k RMSNorm, RoPE and the KV-cache write, straight from
// the fused q/k/v projection output.
//
// The TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") fuses these into the engine's attention-input kernels,
// bit-identical to the chain of per-op kernels they replace (copies, two norms,
// two RoPEs, one KV write).  The chain here is: each op reads bf16 and writes
// bf16; inside an op the arithmetic is IEEE fp32 with every product and sum
// rounded on its own (no contraction), in this order:
//   RMSNorm of a head vector x (weight w):
//     g_j = x_8j^2 + x_(8j+1)^2 + ... + x_(8j+7)^2, left to right (lane j's 8)
//     ss  = the D/8 lane sums added pairwise, partner lane j xor m, for
//           m = D/16, ..., 1 (the xor butterfly; every lane ends with the same bits)
//     r   = 1 / sqrt(ss / D + eps);  y = bf16((x * r) * w)
//   RoPE, rotate-half, (c, s) = table[pos][i] for i < D/2:
//     out_i = bf16(a*c - b*s),  out_(i+D/2) = bf16(b*c + a*s),  a = y_i, b = y_(i+D/2)
// q heads get RMSNorm(q_norm_w) + RoPE and go to q_out; k heads get
// RMSNorm(k_norm_w) + RoPE and go to the pool; v heads go to the pool unchanged.
// INT8 pools quantise the final k and v vectors as the KV write does (keys
// divided by the pool's smoothing vector first, when it has one).
//
// MI355X layout: one wave per token.  The token's sequence (a lane-parallel count
// over cu_new), position, pool slot, RoPE row and both weight vectors are read
// once; then the wave walks the token's head vectors, 64/(D/8) at a time, four
// such passes with their 16-byte loads in flight together.  A lane owns 8
// consecutive elements of a head vector, so D/8 lanes hold one; the sum of
// squares, the absmax and the rotate-half partner exchange (lane j xor D/16) are
// DPP/swizzle moves within those lanes.  Every lane runs the same instructions
// whatever kind its head is (the kind only picks the store), so the cross-lane
// moves never run under a partial mask.  The kernel is HBM-bound: it reads the
// qkv row once and writes q, k and v once.
#include "kv_slot.h"

namespace pfa {
namespace {

// The sequence holding token `tok`: the number of s >= 1 with cu[s] <= tok, counted
// 64 sequences per load round by the lanes of the wave.
__device__ __forceinline__ int wave_find_seq(const int32_t* __restrict__ cu, int batch, int tok) {
    const int lane = (int)__lane_id();
    int s = 0;
    for (int base = 1; base < batch; base += kWave) {
        const int i = base + lane;
        const bool le = i < batch && __ldg(cu + i) <= tok;
        const int n = __builtin_popcountll(__ballot(le));
        s += n;
        if (n < kWave) break;
    }
    return s;
}

template <int D, bool INT8>
__global__ __launch_bounds__(256) void attn_input_kernel(AttnInputArgs a) {
#pragma clang fp contract(off)
    constexpr int L = D / 8;        // lanes per head vector
    constexpr int HPW = kWave / L;  // head vectors per wave pass
    constexpr int HALF = L / 2;     // rotate-half partner: lane j xor HALF
    const int lane = threadIdx.x % kWave;
    const int tok = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave);
    if (tok >= a.num_tokens) return;                     // the whole wave
    const int slot = lane / L;      // head within a pass
    const int chunk = lane % L;
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
    const int heads = Hq + 2 * Hkv;

    // ---- per token, once: sequence, position, pool slot, RoPE row, weights ----
    const int s = __builtin_amdgcn_readfirstlane(wave_find_seq(a.cu_new, a.batch, tok));
    const int c0 = __ldg(a.cu_new + s), c1 = __ldg(a.cu_new + s + 1);
    const int pos = __ldg(a.seq_lens + s) - (c1 - c0) + (tok - c0);
    report(a.err, pos < 0, PFA_BOUNDS_Q_LEN);
    report(a.err, pos >= 0 && pos / kPage >= a.bt_stride, PFA_BOUNDS_SEQ_LEN);
    bool slot_ok = tok < c1 && pos >= 0 && pos / kPage < a.bt_stride;
    int64_t slot0 = 0;              // (page * Hkv) * P + offset: add kvh * P
    if (slot_ok) {
        const int page = __ldg(a.block_table + (int64_t)s * a.bt_stride + pos / kPage);
        slot_ok = page >= 0 && page < a.num_pages;
        report(a.err, !slot_ok, PFA_BOUNDS_PAGE);
        slot0 = (int64_t)page * Hkv * kPage + (pos % kPage);
    }
    const int prow = min(max(pos, 0), a.rope_max_pos - 1);
    const float4* cs = reinterpret_cast<const float4*>(a.rope + ((int64_t)prow * (D / 2) + (chunk % HALF) * 8) * 2);
    float cosv[8], sinv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = __ldg(cs + i);
        cosv[2 * i] = v.x; sinv[2 * i] = v.y;
        cosv[2 * i + 1] = v.z; sinv[2 * i + 1] = v.w;
    }
    float qw[8], kw[8];
    {
        const uint4 q4 = *reinterpret_cast<const uint4*>(a.q_norm_w + chunk * 8);
        const uint4 k4 = *reinterpret_cast<const uint4*>(a.k_norm_w + chunk * 8);
        const uint32_t qa[4] = {q4.x, q4.y, q4.z, q4.w}, ka[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qw[2 * i] = bf16_lo(qa[i]); qw[2 * i + 1] = bf16_hi(qa[i]);
            kw[2 * i] = bf16_lo(ka[i]); kw[2 * i + 1] = bf16_hi(ka[i]);
        }
    }
    float ks[8];                    // INT8 key smoothing of the lane's 8 channels, powers of two (1 = none)
#pragma unroll
    for (int e = 0; e < 8; ++e) ks[e] = 1.0f;
    const bool smooth = INT8 && a.k_smooth != nullptr;
    if (smooth) {
        const float4* sp = reinterpret_cast<const float4*>(a.k_smooth + chunk * 8);
        const float4 s0 = __ldg(sp), s1 = __ldg(sp + 1);
        ks[0] = s0.x; ks[1] = s0.y; ks[2] = s0.z; ks[3] = s0.w;
        ks[4] = s1.x; ks[5] = s1.y; ks[6] = s1.z; ks[7] = s1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) ks[e] = smooth_pow2(ks[e]);
    }
    const uint16_t* row = a.qkv + (int64_t)tok * heads * D + chunk * 8;
    const bool lower = chunk < HALF;

    // one head vector: RMSNorm + RoPE for q and k, then its store
    auto process = [&](int h, const uint4& xin) __attribute__((always_inline)) {
        const bool live = h < heads;
        const bool is_q = h < Hq, is_k = !is_q && h < Hq + Hkv, is_v = h >= Hq + Hkv;
        float x[8];
        const uint32_t xw[4] = {xin.x, xin.y, xin.z, xin.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(xw[i]); x[2 * i + 1] = bf16_hi(xw[i]); }
        // RMSNorm
        float g = x[0] * x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) g = g + x[e] * x[e];
        if constexpr (L >= 16) g = g + xor_lane<8>(g);
        if constexpr (L >= 8) g = g + xor_lane<4>(g);
        g = g + xor_lane<2>(g);
        g = g + xor_lane<1>(g);
        const float r = 1.0f / __builtin_sqrtf(g / (float)D + a.eps);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = bf16_lo(pack_bf16_rne((x[e] * r) * (is_q ? qw[e] : kw[e]), 0.0f));
        // RoPE: the lane of the other half holds the partner elements
        float rot[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pv = xor_lane<HALF>(y[e]);
            const float ya = lower ? y[e] : pv;     // element i
            const float yb = lower ? pv : y[e];     // element i + D/2
            rot[e] = lower ? (ya * cosv[e] - yb * sinv[e]) : (yb * cosv[e] + ya * sinv[e]);
        }
        uint32_t ow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ow[i] = pack_bf16_rne(rot[2 * i], rot[2 * i + 1]);
        const uint4 out = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        const int64_t sdst = slot0 + (int64_t)(is_k ? h - Hq : h - Hq - Hkv) * kPage;
        if (live && is_q) *reinterpret_cast<uint4*>(a.q_out + ((int64_t)tok * Hq + h) * D + chunk * 8) = out;
        if constexpr (!INT8) {
            if (live && slot_ok && !is_q) {
                uint16_t* pool = static_cast<uint16_t*>(is_k ? a.k_pool : a.v_pool);
                // select the words, not the objects (an object select goes through scratch)
                const uint4 kv = make_uint4(is_k ? out.x : xin.x, is_k ? out.y : xin.y,
                                            is_k ? out.z : xin.z, is_k ? out.w : xin.w);
                *reinterpret_cast<uint4*>(pool + sdst * D + chunk * 8) = kv;
            }
        } else {
            float qv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qv[2 * i] = is_v ? x[2 * i] : bf16_lo(ow[i]);
                qv[2 * i + 1] = is_v ? x[2 * i + 1] : bf16_hi(ow[i]);
            }
            if (smooth && is_k) {   // keys smoothed per channel: quantise k / s (exact)
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[e] = qv[e] / ks[e];
            }
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(qv[e]));
            m = group_absmax<D>(m);
            const float scale = m / 127.0f;
            const uint2 codes = quantise8(qv, scale);
            if (live && slot_ok && !is_q) {
                int8_t* pool = static_cast<int8_t*>(is_k ? a.k_pool : a.v_pool);
                *reinterpret_cast<uint2*>(pool + sdst * D + chunk * 8) = codes;
                if (chunk == 0) (is_k ? a.k_scale : a.v_scale)[sdst] = scale;
            }
        }
    };

    // the token's head vectors, four passes of HPW heads with their loads in flight
    // together (named registers: an array here is not unrolled and goes to scratch)
    auto load = [&](int h) __attribute__((always_inline)) {
        return h < heads ? *reinterpret_cast<const uint4*>(row + (int64_t)h * D) : make_uint4(0, 0, 0, 0);
    };
    for (int h0 = slot; h0 < heads; h0 += 4 * HPW) {
        const uint4 x0 = load(h0), x1 = load(h0 + HPW), x2 = load(h0 + 2 * HPW), x3 = load(h0 + 3 * HPW);
        process(h0, x0);
        process(h0 + HPW, x1);
        process(h0 + 2 * HPW, x2);
        process(h0 + 3 * HPW, x3);
    }
}

}  // namespace

hipError_t launch_attn_input(const AttnInputArgs& a, int head_dim, bool int8, hipStream_t s) {
    if (a.num_tokens == 0) return hipSuccess;
    const unsigned grid = (unsigned)(((int64_t)a.num_tokens + 3) / 4);   // 4 waves (tokens) per workgroup
    if (head_dim == 128) {
        if (int8) hipLaunchKernelGGL((attn_input_kernel<128, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((attn_input_kernel<128, false>), dim3(grid), dim3(256), 0, s, a);
    } else {
        if (int8) hipLaunchKernelGGL((attn_input_kernel<64, true>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((attn_input_kernel<64, false>), dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace pfa

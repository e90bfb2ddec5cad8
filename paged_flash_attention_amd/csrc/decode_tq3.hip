// Split-KV paged decode over the 3-bit rotated cache (format in tq3.h).
//
// The TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") gives the split-KV decode: an online softmax over the pages in
// place, one partial per key range, merged by a separate combine.  The qengine
// README's feature list gives the cache: a Walsh-Hadamard rotation and a 3-bit
// Lloyd-Max quantiser.  As H_D H_D = D I, attention over the dequantised cache
// x^_j = H_D (s_j c_j) / D works in the rotated domain:
//   q . x^_j          = s_j * ((H_D q / D) . c_j)
//   sum_j p_j x^_j    = H_D (sum_j p_j s_j c_j) / D
// so q is rotated once per split, a key costs a dot of its levels with the rotated
// q, and the split's output is rotated back once at its end.  The partials (o/l,
// natural lse) have the layout of the BF16/INT8 decode, so the same combine
// merges them.
//
// One wave per (split, KV head, sequence), in the BF16/INT8 decode's 1-D grid
// order (KV head fastest, then split, then sequence).  A lane owns 8 elements
// (group g) of one key: L = D/8 lanes cover a key, and one step handles
// R = 64/L keys of a page (NS = 16/R steps per page).  Every lane keeps the rotated
// q of its 8 elements for all G heads, so a key's G scores come from one 8-term
// dot per head and a butterfly over its L lanes.  The softmax max is taken per
// step and the rescale is lazy (only when some head's max grows).  The next page's
// plane bytes and scales are loaded step by step into the registers the current
// step has just unpacked.  Unwritten slots may hold a NaN scale: masked keys are
// removed by selects, never by a multiplication by zero.
#include "tq3.h"

namespace pfa {
namespace {

template <int D, int G, bool FINAL>
__global__ __launch_bounds__(kWave) void decode_tq3_kernel(DecodeArgs a, Tq3Book bk) {
    constexpr int L = D / 8;          // lanes per key
    constexpr int R = kWave / L;      // keys per step
    constexpr int NS = kPage / R;     // steps per page
    constexpr int PB = D / 8;         // bytes per plane
    constexpr int VB = 3 * PB;        // bytes per vector
    constexpr float kInvD = 1.0f / D;

    const int lane = threadIdx.x;
    const int g = lane % L;
    const int kr = lane / L;
    const int Hq = a.num_q_heads;
    const int Hkv = a.num_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int sp = FINAL ? 0 : (blockIdx.x / Hkv) % a.max_splits;
    const int b = FINAL ? blockIdx.x / Hkv : blockIdx.x / (Hkv * a.max_splits);
    const int head0 = kvh * G;
    const int64_t row0 = (int64_t)b * Hq + head0;

    int len = __ldg(a.seq_lens + b);
    len = min(max(len, 0), a.bt_stride * kPage);
    int lo = a.window > 0 ? max(0, len - a.window) : 0;
    int hi = len;
    if constexpr (FINAL) {
        if (lo >= hi) {   // no keys: output 0
            for (int e = lane; e < G * D; e += kWave) a.out[row0 * D + e] = 0.0f;
            return;
        }
    } else {
        const int s0 = sp * a.split_keys;
        if (s0 >= len) return;
        if (s0 + a.split_keys <= lo) {   // the window hides the whole split
            if (lane < G) a.lse_part[(row0 + lane) * a.max_splits + sp] = -INFINITY;
            return;
        }
        lo = max(lo, s0);
        hi = min(hi, s0 + a.split_keys);
    }

    // rotated query: qr[j] = (H_D q_j / D), elements 8g .. 8g+7
    float qr[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(a.q + (row0 + j) * D + g * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qr[j][2 * i] = bf16_lo(w[i]);
            qr[j][2 * i + 1] = bf16_hi(w[i]);
        }
        fwht_lanes<L>(qr[j], g);
#pragma unroll
        for (int i = 0; i < 8; ++i) qr[j][i] *= kInvD;
    }
    const float c2 = a.sm_scale * kLog2e;      // scores in log2 units

    const int p0 = lo / kPage, p1 = (hi - 1) / kPage;
    const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool);
    const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool);

    // raw plane bytes and scales of one page, by step
    uint32_t kb[NS][3], vb[NS][3];
    float ks[NS], vs[NS];
    auto page_block = [&](int p) __attribute__((always_inline)) {
        const int id = min(max(__ldg(bt + p), 0), a.num_pages - 1);
        return ((int64_t)id * Hkv + kvh) * kPage;          // first vector of the (page, head) block
    };
    auto load_step = [&](int64_t blk, int r) __attribute__((always_inline)) {
        const int64_t vec = blk + r * R + kr;
        const uint8_t* kp = kpool + vec * VB + g;
        const uint8_t* vp = vpool + vec * VB + g;
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) {
            kb[r][pl] = kp[pl * PB];
            vb[r][pl] = vp[pl * PB];
        }
        ks[r] = __ldg(a.k_scale + vec);
        vs[r] = __ldg(a.v_scale + vec);
    };

    float o[G][8];
    float m_run[G], l_run[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[j][i] = 0.0f;
    }

    {
        const int64_t blk = page_block(p0);
#pragma unroll
        for (int r = 0; r < NS; ++r) load_step(blk, r);
    }
    for (int p = p0; p <= p1; ++p) {
        const bool more = p < p1;
        const int64_t nblk = more ? page_block(p + 1) : 0;
#pragma unroll
        for (int r = 0; r < NS; ++r) {
            const uint32_t kw = kb[r][0] | (kb[r][1] << 8) | (kb[r][2] << 16);
            const uint32_t vw = vb[r][0] | (vb[r][1] << 8) | (vb[r][2] << 16);
            const float ksr = ks[r], vsr = vs[r];
            if (more) load_step(nblk, r);

            const int key = p * kPage + r * R + kr;
            const bool valid = key >= lo && key < hi;
            float c[8];
            tq3_levels8(kw, bk, c);
            float s[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float d = qr[j][0] * c[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) d = fmaf(qr[j][i], c[i], d);
                if constexpr (L >= 2) d = xor_sum<1>(d);
                if constexpr (L >= 4) d = xor_sum<2>(d);
                if constexpr (L >= 8) d = xor_sum<4>(d);
                if constexpr (L >= 16) d = xor_sum<8>(d);
                s[j] = valid ? d * (ksr * c2) : -INFINITY;
            }
            // the step's max over its R keys; lazy rescale
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float mt = stride_max<L>(s[j]);
                if (mt > m_run[j]) {          // uniform: every lane holds the same mt and m_run
                    const float alpha = fast_exp2(m_run[j] - mt);   // 0 when m_run is -inf
                    l_run[j] *= alpha;
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[j][i] *= alpha;
                    m_run[j] = mt;
                }
            }
            float cv[8];
            tq3_levels8(vw, bk, cv);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float mu = m_run[j] == -INFINITY ? 0.0f : m_run[j];
                const float pj = fast_exp2(s[j] - mu);            // 0 for masked keys
                l_run[j] += pj;
                const float w = valid ? pj * vsr : 0.0f;          // vsr may be NaN when masked
#pragma unroll
                for (int i = 0; i < 8; ++i) o[j][i] = fmaf(w, cv[i], o[j][i]);
            }
        }
    }

    // sum over the key rows of a step, rotate back, normalise, write
#pragma unroll
    for (int j = 0; j < G; ++j) {
        // l_run counts each key once per lane of its row: sum over rows only
        l_run[j] = stride_sum<L>(l_run[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[j][i] = stride_sum<L>(o[j][i]);
        fwht_lanes<L>(o[j], g);
    }
    if (kr != 0) return;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float mu = m_run[j] == -INFINITY ? 0.0f : m_run[j];
        float* dst;
        float inv;
        if constexpr (FINAL) {
            float z = l_run[j];
            if (a.sinks) z += fast_exp2(__ldg(a.sinks + head0 + j) * kLog2e - mu);
            inv = z > 0.0f ? 1.0f / z : 0.0f;
            dst = a.out + (row0 + j) * D + g * 8;
        } else {
            const int64_t pr = (row0 + j) * a.max_splits + sp;
            inv = l_run[j] > 0.0f ? 1.0f / l_run[j] : 0.0f;
            if (g == 0) a.lse_part[pr] = l_run[j] > 0.0f ? (m_run[j] + fast_log2(l_run[j])) * kLn2 : -INFINITY;
            dst = a.o_part + pr * D + g * 8;
        }
        const float f = inv * kInvD;
        *reinterpret_cast<float4*>(dst) = make_float4(o[j][0] * f, o[j][1] * f, o[j][2] * f, o[j][3] * f);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[j][4] * f, o[j][5] * f, o[j][6] * f, o[j][7] * f);
    }
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, const Tq3Book& bk, hipStream_t s) {
    const int rows = a.batch * a.num_kv_heads;
    if (a.max_splits == 1)
        hipLaunchKernelGGL((decode_tq3_kernel<D, G, true>), dim3(rows), dim3(kWave), 0, s, a, bk);
    else
        hipLaunchKernelGGL((decode_tq3_kernel<D, G, false>), dim3(a.max_splits * rows), dim3(kWave), 0, s, a, bk);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, const Tq3Book& bk, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_dg<D, 1>(a, bk, s);
        case 2: return launch_dg<D, 2>(a, bk, s);
        case 4: return launch_dg<D, 4>(a, bk, s);
        case 8: return launch_dg<D, 8>(a, bk, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_tq3(const DecodeArgs& a, int head_dim, const Tq3Book& bk, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    return head_dim == 128 ? launch_d<128>(a, bk, s) : launch_d<64>(a, bk, s);
}

}  // namespace pfa

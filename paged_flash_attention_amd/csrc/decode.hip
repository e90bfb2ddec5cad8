// Split-KV paged decode: one query token per sequence, over its cached pages.
//
// The TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") does decode this way.  It runs an online softmax over the pages
// in place, reading each page once through the block table, and splits the keys of
// a sequence so that many workgroups share one sequence.  A separate combine then
// merges the splits.  Its "INT8 KV cache" section keeps one scale per cached
// vector.  At 32k positions it also loads 32-key tiles and each half of the head
// dimension separately, so the INT8 kernel stays spill-free.
//
// MI355X design.  The kernel is HBM-bound, and each K/V element is used by exactly
// one lane group, so nothing is staged in LDS for reuse:
//  * One 64-lane wave per (split, KV head, sequence).  The G = Hq/Hkv query heads of
//    the group share every page read (GQA packing).
//  * Page-head block = 16 keys x D.  A lane loads 8 consecutive elements of one key
//    per load (16 B for bf16, 8 B for int8).  LPK = D/8 lanes cover a key, and one
//    load instruction covers 64/LPK keys in one contiguous 512*elem-byte run.  The
//    next page's K/V is prefetched while the current one is consumed.
//  * q.k: v_dot2_f32_bf16 on (q, k) bf16 pairs.  INT8 codes are exact in bf16.
//    Each lane's partial dots for the G heads go through a transposed butterfly
//    over the LPK lanes (DPP / swizzle moves).  Slot j of a lane holds head
//    (j ^ myhead), so every stage adds a partner's upper half to its own lower half
//    with no selects, and ends with the lane holding its own head's full score.
//  * The softmax max is taken per page and the rescale is lazy: o and l are
//    rescaled only when some head's running max grows.  The weights p are shared
//    through a 2-slot LDS buffer, so each lane reads the G weights of its own key.
//  * p.v: fp32 FMAs on the lane's 8 elements for all G heads.  For INT8 the value
//    scale is folded into p.
//  * At the end, the partial o is reduced across the lanes that held different keys.
//    The kernel writes o/l and lse = ln(sum e^s) (split mode), or the final output
//    with the sink applied (unsplit mode).
#include "pfa_device.h"

namespace pfa {
namespace {

template <bool INT8> struct Chunk;
template <> struct Chunk<false> { typedef uint4 T; };   // 8 bf16
template <> struct Chunk<true> { typedef uint2 T; };    // 8 int8

__device__ __forceinline__ void unpack_bf16x8(const uint4& c, float (&x)[8]) {
    x[0] = bf16_lo(c.x); x[1] = bf16_hi(c.x);
    x[2] = bf16_lo(c.y); x[3] = bf16_hi(c.y);
    x[4] = bf16_lo(c.z); x[5] = bf16_hi(c.z);
    x[6] = bf16_lo(c.w); x[7] = bf16_hi(c.w);
}

__device__ __forceinline__ void unpack_i8x8(const uint2& c, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = (float)(int)(int8_t)(c.x >> (8 * i));
        x[4 + i] = (float)(int)(int8_t)(c.y >> (8 * i));
    }
}

// The 8 K elements as four bf16 pairs.
__device__ __forceinline__ void k_pairs(const uint4& c, uint32_t (&k)[4]) {
    k[0] = c.x; k[1] = c.y; k[2] = c.z; k[3] = c.w;
}
__device__ __forceinline__ void k_pairs(const uint2& c, uint32_t (&k)[4]) {
    float x[8];
    unpack_i8x8(c, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = pack_hi16(x[2 * j], x[2 * j + 1]);
}
__device__ __forceinline__ void v_floats(const uint4& c, float (&x)[8]) { unpack_bf16x8(c, x); }
__device__ __forceinline__ void v_floats(const uint2& c, float (&x)[8]) { unpack_i8x8(c, x); }

// Transposed butterfly over the LPK lanes of a key group.  On entry, slot j of
// this lane holds its partial dot for head (j ^ myhead).  On return, slot 0 holds
// this lane's head's full dot over all D dims.
template <int LPK, int G>
__device__ __forceinline__ float transpose_reduce(float (&acc)[G]) {
    if constexpr (G >= 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += xor_lane<LPK / 2>(acc[j + 8]);
    }
    constexpr int M8 = (G >= 16) ? LPK / 4 : LPK / 2;
    if constexpr (G >= 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += xor_lane<M8>(acc[j + 4]);
    }
    constexpr int M4 = (G >= 8) ? M8 / 2 : LPK / 2;
    if constexpr (G >= 4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] += xor_lane<M4>(acc[j + 2]);
    }
    constexpr int M2 = (G >= 4) ? M4 / 2 : LPK / 2;
    if constexpr (G >= 2) acc[0] += xor_lane<M2>(acc[1]);
    // remaining masks: full sums
    constexpr int R = (G >= 2) ? M2 / 2 : LPK / 2;
    float s = acc[0];
    if constexpr (R >= 8) s += xor_lane<8>(s);
    if constexpr (R >= 4) s += xor_lane<4>(s);
    if constexpr (R >= 2) s += xor_lane<2>(s);
    if constexpr (R >= 1) s += xor_lane<1>(s);
    return s;
}

template <int D, int G, bool INT8, bool FINAL>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
    constexpr int EB = INT8 ? 1 : 2;           // bytes per element
    constexpr int LPK = D / 8;                 // lanes per key
    constexpr int KPL = kWave / LPK;           // keys per load instruction
    constexpr int NLOAD = kPage / KPL;         // loads per page per tensor
    constexpr int HG = LPK / G;                // lanes holding each head after the reduce
    static_assert(G <= LPK, "group size");
    typedef typename Chunk<INT8>::T CT;

    __shared__ float p_buf[2][kPage][G];

    const int lane = threadIdx.x;
    const int sub = lane % LPK;
    const int kg = lane / LPK;
    const int myhead = sub / HG;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int Hq = a.num_q_heads;
    const int head0 = kvh * G;

    int len = __ldg(a.seq_lens + b);
    len = min(len, a.bt_stride * kPage);
    int lo = 0, hi = len;
    if (a.window > 0) lo = max(0, len - a.window);
    if constexpr (!FINAL) {
        const int s0 = split * a.split_keys;
        if (s0 >= len || split >= a.max_splits) return;
        lo = max(lo, s0);
        hi = min(hi, s0 + a.split_keys);
    }
    const int64_t part_row = ((int64_t)b * Hq + head0) * a.max_splits + split;  // (b, head0, split)

    if (lo >= hi) {
        if constexpr (!FINAL) {
            // whole split hidden by the window: empty partial
            for (int e = lane; e < G * D; e += kWave) {
                const int g = e / D, d = e % D;
                a.o_part[(part_row + (int64_t)g * a.max_splits) * D + d] = 0.0f;
            }
            if (lane < G) a.lse_part[part_row + (int64_t)lane * a.max_splits] = -INFINITY;
        }
        return;
    }

    // q: slot j holds head (j ^ myhead), dims sub*8 .. sub*8+7, as bf16 pairs
    uint32_t q[G][4];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint16_t* qp = a.q + ((int64_t)b * Hq + head0 + (j ^ myhead)) * D + sub * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(qp);
        q[j][0] = v.x; q[j][1] = v.y; q[j][2] = v.z; q[j][3] = v.w;
    }
    const float c2 = a.sm_scale * kLog2e;      // scores kept in log2 units

    const int p0 = lo / kPage, p1 = (hi - 1) / kPage;
    const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
    const int64_t head_stride = (int64_t)kPage * D;              // elements per page-head block
    const char* kbase = static_cast<const char*>(a.k_pool);
    const char* vbase = static_cast<const char*>(a.v_pool);
    const int lane_off = lane * 8 * EB;

    auto page_id = [&](int p) -> int {
        int id = __ldg(bt + p);
        id = min(max(id, 0), a.num_pages - 1);
        return id;
    };

    CT kc[NLOAD], vc[NLOAD];
    float ksc[NLOAD], vsc[NLOAD];
    auto load_page = [&](int p, CT (&kk)[NLOAD], CT (&vv)[NLOAD], float (&ks)[NLOAD], float (&vs)[NLOAD]) {
        const int id = page_id(p);
        const int64_t blk = (int64_t)id * a.num_kv_heads + kvh;
        const char* kp = kbase + blk * head_stride * EB + lane_off;
        const char* vp = vbase + blk * head_stride * EB + lane_off;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            kk[i] = *reinterpret_cast<const CT*>(kp + i * 512 * EB);
            vv[i] = *reinterpret_cast<const CT*>(vp + i * 512 * EB);
        }
        if constexpr (INT8) {
#pragma unroll
            for (int i = 0; i < NLOAD; ++i) {
                ks[i] = __ldg(a.k_scale + blk * kPage + i * KPL + kg);
                vs[i] = __ldg(a.v_scale + blk * kPage + i * KPL + kg);
            }
        }
    };

    float o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = 0.0f;
    float m_run = -INFINITY;   // running max (log2 units) of this lane's head
    float l_run = 0.0f;        // this lane's share of sum 2^(s - m_run) (its keys, its head)

    load_page(p0, kc, vc, ksc, vsc);
    for (int p = p0; p <= p1; ++p) {
        CT kcur[NLOAD], vcur[NLOAD];
        float kscur[NLOAD], vscur[NLOAD];
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            kcur[i] = kc[i]; vcur[i] = vc[i];
            kscur[i] = ksc[i]; vscur[i] = vsc[i];
        }
        if (p < p1) load_page(p + 1, kc, vc, ksc, vsc);

        const int kbase_pos = p * kPage;
        const bool full = kbase_pos >= lo && kbase_pos + kPage <= hi;

        // ---- scores ----
        float s[NLOAD];
        bool valid[NLOAD];
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            uint32_t kp[4];
            k_pairs(kcur[i], kp);
            float acc[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float t = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[j][w]), as_bf16x2(kp[w]), t, false);
                acc[j] = t;
            }
            float dot = transpose_reduce<LPK, G>(acc);
            const int key = kbase_pos + i * KPL + kg;
            valid[i] = key >= lo && key < hi;
            float sc = INT8 ? c2 * kscur[i] : c2;
            s[i] = valid[i] ? dot * sc : -INFINITY;
        }
        // ---- running max, lazy rescale ----
        float pm = s[0];
#pragma unroll
        for (int i = 1; i < NLOAD; ++i) pm = fmaxf(pm, s[i]);
        pm = stride_max<LPK>(pm);
        const float m_new = fmaxf(m_run, pm);
        if (__any(m_new > m_run)) {
            const float alpha = fast_exp2(m_run - m_new);   // 0 on the first page
            l_run *= alpha;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float ag = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), g * HG));
#pragma unroll
                for (int j = 0; j < 8; ++j) o[g][j] *= ag;
            }
            m_run = m_new;
        }
        // ---- weights ----
        const int pb = p & 1;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const float pw = fast_exp2(s[i] - m_run);      // 0 for masked keys
            l_run += pw;
            float pv = pw;
            if constexpr (INT8) pv = valid[i] ? pw * vscur[i] : 0.0f;
            if (sub % HG == 0) p_buf[pb][i * KPL + kg][myhead] = pv;
        }
        __syncthreads();
        // ---- p.v ----
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            float pw[G];
#pragma unroll
            for (int g = 0; g < G; ++g) pw[g] = p_buf[pb][i * KPL + kg][g];
            float x[8];
            v_floats(vcur[i], x);
            if constexpr (!INT8) {
                if (!full) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) x[j] = valid[i] ? x[j] : 0.0f;
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pw[g], x[j], o[g][j]);
        }
    }

    // ---- reduce across key groups ----
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = stride_sum<LPK>(o[g][j]);
    const float l_tot = stride_sum<LPK>(l_run);

#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g % KPL != kg) continue;
        const float lg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_tot), g * HG));
        const float mg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), g * HG));
        float inv;
        float* dst;
        if constexpr (FINAL) {
            float z = lg;
            if (a.sinks) z += fast_exp2(__ldg(a.sinks + head0 + g) * kLog2e - mg);
            inv = 1.0f / z;
            dst = a.out + ((int64_t)b * Hq + head0 + g) * D + sub * 8;
        } else {
            inv = 1.0f / lg;
            dst = a.o_part + (part_row + (int64_t)g * a.max_splits) * D + sub * 8;
            if (sub == 0) a.lse_part[part_row + (int64_t)g * a.max_splits] = (mg + fast_log2(lg)) * kLn2;
        }
        float4 w0 = make_float4(o[g][0] * inv, o[g][1] * inv, o[g][2] * inv, o[g][3] * inv);
        float4 w1 = make_float4(o[g][4] * inv, o[g][5] * inv, o[g][6] * inv, o[g][7] * inv);
        reinterpret_cast<float4*>(dst)[0] = w0;
        reinterpret_cast<float4*>(dst)[1] = w1;
    }
}

template <int D, int G, bool INT8>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t s) {
    if (a.max_splits == 1) {
        hipLaunchKernelGGL((decode_kernel<D, G, INT8, true>), dim3(1, a.num_kv_heads, a.batch),
                           dim3(kWave), 0, s, a);
    } else {
        hipLaunchKernelGGL((decode_kernel<D, G, INT8, false>),
                           dim3(a.max_splits, a.num_kv_heads, a.batch), dim3(kWave), 0, s, a);
    }
    return hipGetLastError();
}

template <int D, bool INT8>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_dg<D, 1, INT8>(a, s);
        case 2: return launch_dg<D, 2, INT8>(a, s);
        case 4: return launch_dg<D, 4, INT8>(a, s);
        case 8: return launch_dg<D, 8, INT8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool int8, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    if (head_dim == 128) return int8 ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
    return int8 ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace pfa

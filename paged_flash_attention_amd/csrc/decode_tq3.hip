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
// order (KV head fastest, then split, then sequence), and with its lane layout: a
// lane owns 8 elements (group sub) of one key, L = D/8 lanes cover a key, and one
// step handles R = 64/L keys of a page (NS = 16/R steps per page).  q is rotated
// in head order (the rotation runs across the L lanes of one head), then re-read
// through LDS so that slot j of a lane holds head j ^ myhead: one transposed
// butterfly then leaves each lane with its own head's score (myhead = sub/(L/G)).
// The softmax max is taken per page, the rescale is lazy (only when some head's
// max grows), and the weights of a page's keys are shared through LDS for p.v,
// which accumulates all G heads in every lane.  A code's level is one bit-field
// extract and one read of an 8-entry level table in LDS.  The next page's code
// bytes and scales are loaded step by step into the registers the current step
// has just unpacked.  Unwritten slots may hold a NaN scale: masked keys are removed by
// selects, never by a multiplication by zero.
#include "group_reduce.h"
#include "tq3.h"

namespace pfa {
namespace {

template <int D, int G, bool FINAL>
// (the block table is a __restrict__ argument of its own, so that page ids are
// scalar loads, counted apart from the K/V loads)
__global__ __launch_bounds__(kWave) void decode_tq3_kernel(DecodeArgs a, Tq3Book bk,
                                                           const int32_t* __restrict__ block_table) {
    constexpr int L = D / 8;          // lanes per key
    constexpr int R = kWave / L;      // keys per step
    constexpr int NS = kPage / R;     // steps per page
    constexpr int HG = L / G;         // lanes holding each head after the reduce
    constexpr int VB = 3 * D / 8;     // bytes per vector
    constexpr float kInvD = 1.0f / D;
    static_assert(G <= L, "group size");

    __shared__ __attribute__((aligned(16))) float q_lds[G][D];
    __shared__ __attribute__((aligned(16))) float p_buf[NS][R][G];
    __shared__ float lv[8];                    // level of each 3-bit code

    const int lane = threadIdx.x;
    const int sub = lane % L;
    const int kr = lane / L;
    const int myhead = sub / HG;
    const int Hq = a.num_q_heads;
    const int Hkv = a.num_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int sp = FINAL ? 0 : (blockIdx.x / Hkv) % a.max_splits;
    const int b = FINAL ? blockIdx.x / Hkv : blockIdx.x / (Hkv * a.max_splits);
    const int head0 = kvh * G;
    const int64_t row0 = (int64_t)b * Hq + head0;

    int len = __ldg(a.seq_lens + b);
    report(a.err, len < 0 || len > a.bt_stride * kPage ||
                      (!FINAL && sp == 0 && (int64_t)a.max_splits * a.split_keys < len),
           PFA_BOUNDS_SEQ_LEN);
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

    const int p0 = lo / kPage, p1 = (hi - 1) / kPage;
    const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool);
    const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool);

    // raw code bytes and scales of one page, by step
    uint32_t kb[NS][3], vb[NS][3];
    float ks[NS], vs[NS];
    auto page_block = [&](int p) __attribute__((always_inline)) {
        const int raw = __ldg(bt + p);
        report(a.err, raw < 0 || raw >= a.num_pages, PFA_BOUNDS_PAGE);
        const int id = min(max(raw, 0), a.num_pages - 1);
        return ((int64_t)id * Hkv + kvh) * kPage;          // first vector of the (page, head) block
    };
    auto load_step = [&](int64_t blk, int r) __attribute__((always_inline)) {
        const int64_t vec = blk + r * R + kr;
        const uint8_t* kp = kpool + vec * VB + 3 * sub;
        const uint8_t* vp = vpool + vec * VB + 3 * sub;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            kb[r][k] = kp[k];
            vb[r][k] = vp[k];
        }
        ks[r] = __ldg(a.k_scale + vec);
        vs[r] = __ldg(a.v_scale + vec);
    };

    // rotated query H_D q / D.  The R key rows of the wave would each rotate the
    // same G heads, so row r rotates heads r, r + R, ... (in head order, across its
    // L lanes) and the wave shares them through LDS; each lane then reads its slots
    // (slot j = head j ^ myhead).  The first page's loads go out before, so the
    // rotation runs while they are in flight.
    {
        const int64_t blk = page_block(p0);
#pragma unroll
        for (int r = 0; r < NS; ++r) load_step(blk, r);
    }
    float qr[G][8];
    constexpr int HPR = (G + R - 1) / R;      // heads per key row
#pragma unroll
    for (int e = 0; e < HPR; ++e) {
        const int h = e * R + kr;
        if (h < G) {   // (uniform within a key row, whose L lanes run the rotation together)
            const uint4 v = *reinterpret_cast<const uint4*>(a.q + (row0 + h) * D + sub * 8);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = bf16_lo(w[i]);
                x[2 * i + 1] = bf16_hi(w[i]);
            }
            fwht_lanes<L>(x, sub);
            float4* d = reinterpret_cast<float4*>(&q_lds[h][sub * 8]);
            d[0] = make_float4(x[0] * kInvD, x[1] * kInvD, x[2] * kInvD, x[3] * kInvD);
            d[1] = make_float4(x[4] * kInvD, x[5] * kInvD, x[6] * kInvD, x[7] * kInvD);
        }
    }
    if (lane < 8) lv[lane] = tq3_level_of(lane, bk);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float4* s4 = reinterpret_cast<const float4*>(&q_lds[j ^ myhead][sub * 8]);
        const float4 x0 = s4[0], x1 = s4[1];
        qr[j][0] = x0.x; qr[j][1] = x0.y; qr[j][2] = x0.z; qr[j][3] = x0.w;
        qr[j][4] = x1.x; qr[j][5] = x1.y; qr[j][6] = x1.z; qr[j][7] = x1.w;
    }
    const float c2 = a.sm_scale * kLog2e;      // scores in log2 units

    float o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = 0.0f;
    float m_run = -INFINITY;   // running max (log2 units) of this lane's head
    float l_run = 0.0f;        // this lane's share of sum 2^(s - m_run) (its row's keys, its head)

    for (int p = p0; p <= p1; ++p) {
        const bool more = p < p1;
        const int64_t nblk = more ? page_block(p + 1) : 0;
        // ---- scores of the page: one per lane and step (this lane's head) ----
        float s[NS];
        uint32_t vw[NS];
        float vsc[NS];
#pragma unroll
        for (int r = 0; r < NS; ++r) {
            const uint32_t kw = kb[r][0] | (kb[r][1] << 8) | (kb[r][2] << 16);
            vw[r] = vb[r][0] | (vb[r][1] << 8) | (vb[r][2] << 16);
            const float ksr = ks[r];
            vsc[r] = vs[r];
            if (more) load_step(nblk, r);
            float c[8];
            tq3_levels8(kw, lv, c);
            float acc[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float d = qr[j][0] * c[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) d = fmaf(qr[j][i], c[i], d);
                acc[j] = d;
            }
            const float dot = transpose_reduce<L, G>(acc);
            s[r] = dot * (ksr * c2);
        }
        // masks on the pages that cross [lo, hi) only: the scores of keys outside
        // become -inf by a select (their scales may be poison) and their value
        // scales 0, so the weight is 0 rather than 0 * NaN
        if (!(p * kPage >= lo && p * kPage + kPage <= hi)) {
#pragma unroll
            for (int r = 0; r < NS; ++r) {
                const int key = p * kPage + r * R + kr;
                const bool out = key < lo || key >= hi;
                s[r] = out ? -INFINITY : s[r];
                vsc[r] = out ? 0.0f : vsc[r];
            }
        }
        // ---- running max, lazy rescale with headroom: the reference max moves only
        // when a head's max exceeds it by more than 8, so every weight is <= 2^8
        // (no overflow in fp32 or bf16) and the rescale, G*8 multiplies, runs on
        // few pages.  o and l share the reference, so o/l and m + log2(l) hold. ----
        float pm = s[0];
#pragma unroll
        for (int r = 1; r < NS; ++r) pm = fmaxf(pm, s[r]);
        pm = stride_max<L>(pm);
        const float m_new = fmaxf(m_run, pm);
        if (__any(m_new > m_run + 8.0f)) {
            const float alpha = fast_exp2(m_run - m_new);   // 0 on the first page
            l_run *= alpha;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float ag = lane_read(alpha, g * HG);
#pragma unroll
                for (int i = 0; i < 8; ++i) o[g][i] *= ag;
            }
            m_run = m_new;
        }
        // ---- weights, shared within the wave ----
#pragma unroll
        for (int r = 0; r < NS; ++r) {
            const float pw = fast_exp2(s[r] - m_run);      // 0 for masked keys
            l_run += pw;
            const float pv = pw * vsc[r];
            if (sub % HG == 0) p_buf[r][kr][myhead] = pv;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- p.v in the rotated domain, all G heads ----
#pragma unroll
        for (int r = 0; r < NS; ++r) {
            float cv[8];
            tq3_levels8(vw[r], lv, cv);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float w = p_buf[r][kr][g];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[g][i] = fmaf(w, cv[i], o[g][i]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // sum over the key rows, rotate back, normalise, write
    const float l_tot = stride_sum<L>(l_run);
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = stride_sum<L>(o[g][i]);
        fwht_lanes<L>(o[g], sub);
    }
    if (kr != 0) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mg = lane_read(m_run, g * HG);
        const float lg = lane_read(l_tot, g * HG);
        const float mu = mg == -INFINITY ? 0.0f : mg;
        float* dst;
        float inv;
        if constexpr (FINAL) {
            float z = lg;
            if (a.sinks) z += fast_exp2(__ldg(a.sinks + head0 + g) * kLog2e - mu);
            inv = z > 0.0f ? 1.0f / z : 0.0f;
            dst = a.out + (row0 + g) * D + sub * 8;
        } else {
            const int64_t pr = (row0 + g) * a.max_splits + sp;
            inv = lg > 0.0f ? 1.0f / lg : 0.0f;
            if (sub == 0) a.lse_part[pr] = lg > 0.0f ? (mg + fast_log2(lg)) * kLn2 : -INFINITY;
            dst = a.o_part + pr * D + sub * 8;
        }
        const float f = inv * kInvD;
        *reinterpret_cast<float4*>(dst) = make_float4(o[g][0] * f, o[g][1] * f, o[g][2] * f, o[g][3] * f);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[g][4] * f, o[g][5] * f, o[g][6] * f, o[g][7] * f);
    }
}

template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, const Tq3Book& bk, hipStream_t s) {
    const int rows = a.batch * a.num_kv_heads;
    if (a.max_splits == 1)
        hipLaunchKernelGGL((decode_tq3_kernel<D, G, true>), dim3(rows), dim3(kWave), 0, s, a, bk, a.block_table);
    else
        hipLaunchKernelGGL((decode_tq3_kernel<D, G, false>), dim3(a.max_splits * rows), dim3(kWave), 0, s, a, bk,
                           a.block_table);
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

// Paged flash-attention prefill: causal attention of a chunk of new tokens over
// their sequence's paged K/V.  That K/V is the restored prefix plus the chunk.
//
// Sources: the TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") runs an online softmax over the pages in place, so it never
// writes the q x k score matrix.  The Qml-engine announcement says a session turn
// restores the conversation's KV from a store and prefills only the new turn.
//
// MI355X design (gfx950, v_mfma_f32_32x32x16_bf16):
//  * A workgroup is 4 waves and owns 128 query rows of one (sequence, KV head).
//    A row is one (token, head-of-group) pair, so the G query heads sharing a KV
//    head share every K/V tile (GQA packing).  Each wave owns 32 rows.
//  * Each iteration takes 64 keys (4 pages).  Their page ids come from the block
//    table.  The K tile is staged in LDS row-major; the V tile is staged
//    transposed (V^T, keys contiguous per dim) through register permutes.  Both
//    are double-buffered, with the next tile's global loads in flight during
//    the current tile's math.
//  * Scores are computed transposed: S^T = K Q^T.  Then every lane of the MFMA
//    output holds one query row (lane % 32) and 16 of the keys, with the other
//    16 in lane ^ 32.  The row max and row sum take one cross-lane step, and
//    P^T is already in the B-operand layout of O^T = V^T P^T.  The O^T
//    accumulator of a lane also belongs to its one row, so the online-softmax
//    rescale is a per-lane scalar, skipped when no row's max grew.
//  * Scores are kept in log2 units (sm_scale*log2 e folded in), and
//    exp2 -> v_exp_f32.  P is rounded to bf16 (RNE) for the PV MFMA.
//  * Causal/window masking costs nothing on tiles that are fully visible.  A wave
//    skips the MFMAs of tiles that lie entirely outside its rows' ranges.
//  * Workgroups map to XCDs so that each XCD's L2 holds the K/V of the heads it
//    serves.  Within an XCD the longest (latest) query tiles go first.
//  * Split mode covers a short chunk on a long prefix, such as 130 new tokens on
//    8192.  Such a chunk has too few query tiles to fill 256 CUs, so the key
//    range is cut into max_splits ranges of split_keys keys, a multiple of 64.
//    Each workgroup writes a softmax-normalised partial with its natural
//    log-sum-exp, and the combine kernel then merges them with the sink.
#include "pfa_device.h"

namespace pfa {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBN = 64;           // keys per iteration
constexpr int kXcds = 8;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct Tile {
    static constexpr int KP = D + 8;          // K row pitch (elements): 16 lanes reading one
                                              // column of 16 rows hit 16 distinct bank quads
    uint16_t k[2][kBN][KP];
    uint16_t vt[2][D][kBN];                   // V^T rows of 64 keys, 16-byte chunks swizzled
};

// position of key-quad q (0..15) of a 64-key tile inside a V^T row: within each
// 16-key group the middle two quads swap, so that the 8 keys one MFMA lane needs
// (k-slots 8*(lane/32)..+8) are contiguous.
__device__ __forceinline__ int vt_quad_pos(int q) {
    return (q & ~3) | ((q & 1) << 1) | ((q & 2) >> 1);
}

// Element offset of (row d, 16-byte chunk c, element e in chunk) in a V^T buffer.
// A row is 128 B, half the banks; chunk c of row d sits at c ^ ((d >> 1) & 7), so
// the 16 rows one 16-lane read touches fall on 16 distinct bank quads.
__device__ __forceinline__ int vt_off(int d, int c, int e) {
    return d * kBN + ((c ^ ((d >> 1) & 7)) << 3) + e;
}

template <int D, int G, bool SPLIT>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
    constexpr int TPW = kRowsPerWave / G;               // tokens per wave
    constexpr int TPB = TPW * kWaves;                   // tokens per workgroup
    constexpr int KK = D / 16;                          // MFMA k-steps over D
    constexpr int DB = D / 32;                          // 32-row blocks of O^T
    constexpr int CPR = D / 8;                          // 16-byte chunks per K row
    constexpr int KLOADS = kBN * CPR / 256;             // K chunks per thread
    static_assert(KLOADS * 256 == kBN * CPR, "K tile split");

    __shared__ Tile<D> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int lane = tid % kWave;
    const int r32 = lane % 32;
    const int half = lane / 32;

    // ---- work item (XCD-aware, heaviest tiles first) ----
    // items run (b, kvh, split, tile) with tile fastest; each XCD takes a
    // contiguous range, so the tiles that share a (b, kvh, split) K/V range share
    // one L2.
    const int n_tiles = (a.max_q_len + TPB - 1) / TPB;
    const int nsplit = SPLIT ? a.max_splits : 1;
    const int n_items = a.batch * a.num_kv_heads * nsplit * n_tiles;
    const int per_xcd = (n_items + kXcds - 1) / kXcds;
    const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (item >= n_items) return;
    const int tile = n_tiles - 1 - item % n_tiles;
    const int split = (item / n_tiles) % nsplit;
    const int kvh = (item / (n_tiles * nsplit)) % a.num_kv_heads;
    const int b = item / (n_tiles * nsplit * a.num_kv_heads);

    const int cq0 = __ldg(a.cu_q + b);
    const int q_len = __ldg(a.cu_q + b + 1) - cq0;
    const int tok0 = tile * TPB;
    if (tok0 >= q_len) return;
    const int n = min(__ldg(a.seq_lens + b), a.bt_stride * kPage);
    const int prefix = n - q_len;
    const int Hq = a.num_q_heads;
    const int W = a.window;

    // this lane's query row
    const int tok_l = tok0 + wave * TPW + r32 / G;
    const int h_l = kvh * G + r32 % G;
    const bool row_ok = tok_l < q_len;
    const int pos_l = prefix + tok_l;

    // key ranges: workgroup (within this split) and wave
    const int wg_last = min(tok0 + TPB, q_len) - 1;
    int hi = prefix + wg_last + 1;
    int lo = W > 0 ? max(0, prefix + tok0 - W + 1) : 0;
    if constexpr (SPLIT) {
        lo = max(lo, split * a.split_keys);
        hi = min(hi, (split + 1) * a.split_keys);
        if (lo >= hi) {
            // no key of this split is visible to any row of the tile
            if (row_ok) {
                const int64_t pr = ((int64_t)(cq0 + tok_l) * Hq + h_l) * a.max_splits + split;
                float* op = a.o_part + pr * D + half * (D / 2);
                for (int d = 0; d < D / 2; d += 4)
                    *reinterpret_cast<float4*>(op + d) = make_float4(0.f, 0.f, 0.f, 0.f);
                if (half == 0) a.lse_part[pr] = -INFINITY;
            }
            return;
        }
    }
    const int w_first = tok0 + wave * TPW;
    const int w_last = min(tok0 + (wave + 1) * TPW, q_len) - 1;
    const bool wave_live = w_first < q_len;
    const int w_hi = prefix + w_last + 1;
    const int w_lo = W > 0 ? max(0, prefix + w_first - W + 1) : 0;

    // ---- Q fragment (B operand of S^T = K Q^T) ----
    bf16x8 qf[KK];
    {
        const uint16_t* qp = a.q + ((int64_t)(cq0 + tok_l) * Hq + h_l) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_ok) v = *reinterpret_cast<const uint4*>(qp + 16 * kk);
            qf[kk] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
    const int64_t hblk = (int64_t)kPage * D;             // elements per page-head block

    // ---- tile loads: global -> registers ----
    // A 64-key tile is 4 pages.  Its page ids are wave-uniform loads; pages past the
    // sequence end are never read (their rows are zero-filled).
    uint4 kreg[KLOADS];
    uint4 vreg[4];
    const int vq = tid % 16;                              // key quad of this thread (V)
    const int vc = tid / 16;                              // 8-dim chunk of this thread (V)
    auto sel4 = [](int j, const uint16_t* p0, const uint16_t* p1, const uint16_t* p2,
                   const uint16_t* p3) { return j == 0 ? p0 : j == 1 ? p1 : j == 2 ? p2 : p3; };
    auto load_tile = [&](int kb) {
        const int key0 = kb * kBN;
        const uint16_t* kp[4];
        const uint16_t* vp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pi = kb * 4 + j;
            int pg = 0;
            if (pi * kPage < n) pg = min(max(__ldg(bt + pi), 0), a.num_pages - 1);
            const int64_t off = ((int64_t)pg * a.num_kv_heads + kvh) * hblk;
            kp[j] = a.k_pool + off;
            vp[j] = a.v_pool + off;
        }
#pragma unroll
        for (int e = 0; e < KLOADS; ++e) {
            const int c = tid + 256 * e;
            const int key = c / CPR, col = c % CPR;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (key0 + key < n)
                v = *reinterpret_cast<const uint4*>(sel4(key / kPage, kp[0], kp[1], kp[2], kp[3]) +
                                                    (key % kPage) * D + col * 8);
            kreg[e] = v;
        }
        if (vc < CPR) {
            const uint16_t* vbase = sel4(vq / 4, vp[0], vp[1], vp[2], vp[3]) + (4 * (vq % 4)) * D + vc * 8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (key0 + 4 * vq + e < n) v = *reinterpret_cast<const uint4*>(vbase + e * D);
                vreg[e] = v;
            }
        }
    };
    // ---- registers -> LDS (K row-major, V transposed and swizzled) ----
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int e = 0; e < KLOADS; ++e) {
            const int c = tid + 256 * e;
            const int key = c / CPR, col = c % CPR;
            *reinterpret_cast<uint4*>(&sm.k[buf][key][col * 8]) = kreg[e];
        }
        if (vc < CPR) {
            const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
            const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
            const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
            const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
            const int kpos = 4 * vt_quad_pos(vq);
            uint16_t* vt = &sm.vt[buf][0][0];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const int w = j >> 1;
                uint2 t;
                t.x = __builtin_amdgcn_perm(w1[w], w0[w], sel);
                t.y = __builtin_amdgcn_perm(w3[w], w2[w], sel);
                *reinterpret_cast<uint2*>(vt + vt_off(vc * 8 + j, kpos >> 3, kpos & 7)) = t;
            }
        }
    };

    // ---- accumulators ----
    f32x16 acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.0f;
    float m_run = -INFINITY;   // log2 units
    float l_run = 0.0f;        // this lane's share (its 16 keys of each 32)
    const float c2 = a.sm_scale * kLog2e;

    const int kb0 = lo / kBN;
    const int kb1 = (hi - 1) / kBN;

    load_tile(kb0);
    store_tile(0);
    __syncthreads();

    for (int kb = kb0; kb <= kb1; ++kb) {
        const int buf = (kb - kb0) & 1;
        if (kb < kb1) load_tile(kb + 1);

        const int key0 = kb * kBN;
        const bool needed = wave_live && key0 < w_hi && key0 + kBN > w_lo;
        if (needed) {
            // ---- S^T = K Q^T for two 32-key sub-blocks ----
            // The two accumulator chains are interleaved, and the K fragments of step
            // kk+1 are read from LDS while the MFMAs of step kk run.
            f32x16 s[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) s[0][r] = s[1][r] = 0.0f;
            const uint16_t* kr0 = &sm.k[buf][r32][8 * half];
            const uint16_t* kr1 = &sm.k[buf][32 + r32][8 * half];
            uint4 ka0 = *reinterpret_cast<const uint4*>(kr0);
            uint4 ka1 = *reinterpret_cast<const uint4*>(kr1);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                uint4 kn0 = ka0, kn1 = ka1;
                if (kk + 1 < KK) {
                    kn0 = *reinterpret_cast<const uint4*>(kr0 + 16 * (kk + 1));
                    kn1 = *reinterpret_cast<const uint4*>(kr1 + 16 * (kk + 1));
                }
                s[0] = mfma32(__builtin_bit_cast(bf16x8, ka0), qf[kk], s[0]);
                s[1] = mfma32(__builtin_bit_cast(bf16x8, ka1), qf[kk], s[1]);
                ka0 = kn0;
                ka1 = kn1;
            }
            // ---- scale, mask ----
            const bool full = (key0 + kBN - 1 <= prefix + w_first) &&
                              (W == 0 || (prefix + w_last) - key0 < W);
            float mt = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[sb][r] * c2;
                    if (!full) {
                        const int key = key0 + 32 * sb + 8 * (r / 4) + 4 * half + (r % 4);
                        const bool vis = key <= pos_l && (W == 0 || pos_l - key < W);
                        x = vis ? x : -INFINITY;
                    }
                    s[sb][r] = x;
                    mt = fmaxf(mt, x);
                }
            mt = fmaxf(mt, xor_lane<32>(mt));
            const float m_new = fmaxf(m_run, mt);
            if (__any(m_new > m_run)) {
                const float mu = (m_new == -INFINITY) ? 0.0f : m_new;
                const float alpha = fast_exp2(m_run - mu);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
                m_run = m_new;
            }
            const float mu = (m_run == -INFINITY) ? 0.0f : m_run;
            // ---- P = 2^(x - m), packed to bf16 in the B-operand order ----
            uint32_t pk[2][8];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(s[sb][r] - mu);
                    const float p1 = fast_exp2(s[sb][r + 1] - mu);
                    l_run += p0 + p1;
                    pk[sb][r / 2] = pack_bf16_rne(p0, p1);
                }
            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int m = 0; m < kBN / 16; ++m) {
                const int sb = m / 2, r0 = 4 * (m % 2);
                const uint4 pu = make_uint4(pk[sb][r0], pk[sb][r0 + 1], pk[sb][r0 + 2], pk[sb][r0 + 3]);
                const bf16x8 pf = __builtin_bit_cast(bf16x8, pu);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint4 vv = *reinterpret_cast<const uint4*>(&sm.vt[buf][0][0] +
                                                                     vt_off(32 * db + r32, 2 * m + half, 0));
                    acc_o[db] = mfma32(__builtin_bit_cast(bf16x8, vv), pf, acc_o[db]);
                }
            }
        }
        if (kb < kb1) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- finish: combine the two lanes of each row ----
    const float l_tot = l_run + xor_lane<32>(l_run);
    if (!row_ok) return;
    const float mu = (m_run == -INFINITY) ? 0.0f : m_run;
    float inv;
    float* op;
    if constexpr (SPLIT) {
        // softmax-normalised partial and its natural log-sum-exp; no sink here
        const int64_t pr = ((int64_t)(cq0 + tok_l) * Hq + h_l) * a.max_splits + split;
        inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if (half == 0) a.lse_part[pr] = l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
        op = a.o_part + pr * D;
    } else {
        float z = l_tot;
        if (a.sinks) z += fast_exp2(__ldg(a.sinks + h_l) * kLog2e - mu);
        inv = z > 0.0f ? 1.0f / z : 0.0f;
        op = a.out + ((int64_t)(cq0 + tok_l) * Hq + h_l) * D;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 32 * db + 8 * i + 4 * half;
            float4 w = make_float4(acc_o[db][4 * i] * inv, acc_o[db][4 * i + 1] * inv,
                                   acc_o[db][4 * i + 2] * inv, acc_o[db][4 * i + 3] * inv);
            *reinterpret_cast<float4*>(op + d) = w;
        }
}

template <int D, int G>
hipError_t launch_dg(const PrefillArgs& a, hipStream_t s) {
    constexpr int TPB = kRowsPerWave / G * kWaves;
    const int n_tiles = (a.max_q_len + TPB - 1) / TPB;
    const bool split = a.max_splits > 1;
    const int64_t items = (int64_t)a.batch * a.num_kv_heads * n_tiles * (split ? a.max_splits : 1);
    const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
    if (grid == 0) return hipSuccess;
    if (split)
        hipLaunchKernelGGL((prefill_kernel<D, G, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_kernel<D, G, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_dg<D, 1>(a, s);
        case 2: return launch_dg<D, 2>(a, s);
        case 4: return launch_dg<D, 4>(a, s);
        case 8: return launch_dg<D, 8>(a, s);
        case 16: return launch_dg<D, 16>(a, s);
        case 32: return launch_dg<D, 32>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, hipStream_t s) {
    if (a.batch == 0 || a.max_q_len == 0) return hipSuccess;
    return head_dim == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace pfa

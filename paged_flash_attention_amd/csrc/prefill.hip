// Paged flash-attention prefill: causal attention of a chunk of new tokens over
// their sequence's paged K/V.  That K/V is the restored prefix plus the chunk.
//
// Sources: the TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") runs an online softmax over the pages in place, so it never
// writes the q x k score matrix.  The Qml-engine announcement says a session turn
// restores the conversation's KV from a store and prefills only the new turn.
//
// MI355X design (gfx950, v_mfma_f32_32x32x16_bf16):
//  * A workgroup is 8 waves and owns 256 query rows of one (sequence, KV head).
//    A row is one (token, head-of-group) pair, so the G query heads sharing a KV
//    head share every K/V tile (GQA packing).  Each wave owns 32 rows.
//  * K/V go HBM -> LDS with global_load_lds_dwordx4, with no register staging, in
//    a 3-stage ring of 64-key tiles (4 pages).  Two tiles stay in flight while one
//    is consumed, and each wave waits on its own vmcnt, so there is one barrier per
//    tile.  The page ids of the tile after next are read (wave-uniform) while the
//    current tile computes.
//  * LDS rows are the page rows (keys x D), 16-byte chunks XOR-swizzled per row.
//    The swizzle is applied on the global side of the direct loads, and it makes
//    both read patterns below free of bank conflicts.
//  * Scores are computed transposed: S^T = K Q^T, with Q^T in registers.  Then every
//    lane of the MFMA output holds one query row (lane % 32) and 16 of the keys,
//    with the other 16 in lane ^ 32.  The row max and row sum take one cross-lane
//    step, and P^T is already in the B-operand layout of O^T = V^T P^T.  The O^T
//    accumulator of a lane also belongs to its one row, so the online-softmax
//    rescale is a per-lane scalar, skipped when no row's max grew.
//  * The V^T A-operand comes straight from the row-major V tile through
//    ds_read_b64_tr_b16.  In each 16-lane group, lane j points at
//    V[k0 + j/4][d0 + 4(j%4)], and lane i gets V[k0..k0+3][d0 + i].
//  * Softmax arithmetic is trimmed for the VALU:
//      - the row max is taken on raw scores;
//      - p = exp2(s*c - m) is one FMA plus v_exp_f32, with c = sm_scale*log2 e;
//      - P is rounded to bf16 (RNE) for the PV MFMA;
//      - the row sum is a dot2 of those rounded pairs with (1, 1), so l matches the
//        numerator exactly;
//      - the reference max moves only when a row's max grows by more than 2^8.
//  * Causal/window masking costs nothing on tiles that are fully visible.  A wave
//    skips the MFMAs of tiles that lie entirely outside its rows' ranges.  V rows
//    past the sequence end are zeroed in LDS, so poison in unwritten page slots
//    never meets a zero weight.
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

constexpr int kRowsPerWave = 32;
constexpr int kWaves = kPrefillRows / kRowsPerWave;
constexpr int kThreads = kWaves * kWave;
constexpr int kBN = 64;           // keys per tile
constexpr int kXcds = 8;

#define LDS3 __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte-chunk swizzles (chunk c of row r sits at c ^ f(r)).  K: the 16 rows one
// 16-lane MFMA read touches land on 16 distinct bank quads.  V: the 4 rows x 2
// chunks of a 16-lane transposed read, and 4 rows x 4 chunks per 32 lanes, are
// distinct.  (Rows of D = 64 are 128 B, two rows per bank line.)
template <int D> __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The V^T operands of one 16-key slice: for each 32-dim block db, a transposed
// read of keys k..k+3 at addr[db] and of keys k+8..k+11 at addr[db] + HI bytes.
// The reads are issued as one asm block that waits for them itself.  Issued
// through the intrinsic, the compiler treats the read as possibly aliasing any
// in-flight direct load, and would wait for the prefetched tiles too.
template <int DB, int HI>
__device__ __forceinline__ void tr_reads(uint2 (&lo)[DB], uint2 (&hi)[DB], const uint32_t (&addr)[DB]) {
    if constexpr (DB == 4) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
            "ds_read_b64_tr_b16 %2, %9\n\t"
            "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
            "ds_read_b64_tr_b16 %4, %10\n\t"
            "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
            "ds_read_b64_tr_b16 %6, %11\n\t"
            "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]),
              "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]), "=&v"(hi[3])
            : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(HI)
            : "memory");
    } else {
        static_assert(DB == 2, "head dim");
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4\n\t"
            "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
            "ds_read_b64_tr_b16 %2, %5\n\t"
            "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
            : "v"(addr[0]), "v"(addr[1]), "i"(HI)
            : "memory");
    }
}

// 16-byte direct load HBM -> LDS: lane l's bytes land at lds + 16*l.  (A plain,
// non-template function: used straight inside the kernel template, the builtin
// made the host pass drop the launch stubs.)
__device__ __forceinline__ void dma16(const uint16_t* src, uint16_t* lds) {
    __builtin_amdgcn_global_load_lds(src, (LDS3 void*)lds, 16, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(LDS3 const void*)p;
}

template <int D, int G, bool SPLIT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a, const int32_t* __restrict__ block_table) {
    constexpr int TPW = kRowsPerWave / G;               // tokens per wave
    constexpr int TPB = TPW * kWaves;                   // tokens per workgroup
    constexpr int KK = D / 16;                          // MFMA k-steps over D
    constexpr int DB = D / 32;                          // 32-row blocks of O^T
    constexpr int CPR = D / 8;                          // 16-byte chunks per row
    constexpr int ROWS_PER_DMA = kWave / CPR;           // rows one wave-wide direct load fills
    constexpr int DMA_PER_WAVE = kBN / ROWS_PER_DMA / kWaves;   // per tensor per tile
    constexpr int NL = 2 * DMA_PER_WAVE;                // vector-memory ops per tile per wave
    static_assert(DMA_PER_WAVE >= 1, "tile split");

    __shared__ __attribute__((aligned(1024))) uint16_t k_s0[kBN * D], k_s1[kBN * D], k_s2[kBN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s0[kBN * D], v_s1[kBN * D], v_s2[kBN * D];

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

    // ---- direct HBM -> LDS tile loads ----
    // a __restrict__ kernel argument: uniform reads of it become scalar loads, which
    // stay out of the vmcnt queue the direct loads are counted on
    const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
    const int npg = (n + kPage - 1) / kPage;
    const int64_t hblk = (int64_t)kPage * D;            // elements per page-head block
    const int kb0 = lo / kBN;
    const int kb1 = (hi - 1) / kBN;
    auto tile_pages = [&](int kb, int (&pg)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pi = min(kb * 4 + j, npg - 1);
            pg[j] = min(max(__ldg(bt + pi), 0), a.num_pages - 1);
        }
    };
    const int lrow = lane / CPR;                          // row within one direct load
    const int lchunk = lane % CPR;                        // physical chunk this lane fills
    auto issue = [&](const int (&pg)[4], uint16_t* kdst, uint16_t* vdst) {
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i) {
            const int q = wave * DMA_PER_WAVE + i;        // which 1 KB slice of the tile
            const int row0 = q * ROWS_PER_DMA;            // rows row0.. lie in one page
            const int row = row0 + lrow;
            const int64_t pbase = ((int64_t)pg[row0 / kPage] * a.num_kv_heads + kvh) * hblk + (row % kPage) * D;
            dma16(a.k_pool + pbase + (lchunk ^ swz_k<D>(row)) * 8, kdst + row0 * D);
            dma16(a.v_pool + pbase + (lchunk ^ swz_v<D>(row)) * 8, vdst + row0 * D);
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

    // per-lane constants of the transposed V reads
    const int tr_g = lane / 16, tr_j = lane % 16;
    const int tr_row = 4 * (tr_g / 2) + tr_j / 4;                 // + 16m (+ 8 for the upper half)
    const int tr_chunk = 2 * (tr_g % 2) + (tr_j % 4) / 2;         // + 4db
    const int tr_sub = 4 * (tr_j % 2);

    auto compute = [&](int kb, const uint16_t* ks, const uint16_t* vs) {
        const int key0 = kb * kBN;
        // ---- S^T = K Q^T for two 32-key sub-blocks, chains interleaved ----
        f32x16 s[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[0][r] = s[1][r] = 0.0f;
        const int kr0 = r32, kr1 = 32 + r32;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int c = 2 * kk + half;
            const uint4 k0 = *reinterpret_cast<const uint4*>(ks + kr0 * D + ((c ^ swz_k<D>(kr0)) << 3));
            const uint4 k1 = *reinterpret_cast<const uint4*>(ks + kr1 * D + ((c ^ swz_k<D>(kr1)) << 3));
            s[0] = mfma32(__builtin_bit_cast(bf16x8, k0), qf[kk], s[0]);
            s[1] = mfma32(__builtin_bit_cast(bf16x8, k1), qf[kk], s[1]);
        }
        // ---- mask, row max on the raw scores (the scale is positive) ----
        const bool full = (key0 + kBN - 1 <= prefix + w_first) && (W == 0 || (prefix + w_last) - key0 < W);
        if (!full) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + 32 * sb + 8 * (r / 4) + 4 * half + (r % 4);
                    const bool vis = key <= pos_l && (W == 0 || pos_l - key < W);
                    s[sb][r] = vis ? s[sb][r] : -INFINITY;
                }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sb][r]);
        mt = fmaxf(mt, xor_lane<32>(mt)) * c2;               // log2 units
        // Lazy rescale with headroom: the reference max moves only when a row's max
        // exceeds it by more than 8, so p <= 2^8 (exact enough in bf16, no overflow
        // in the fp32 sums).  O and l share the reference, so o/l is unchanged.
        if (__any(mt > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, mt);
            const float mu = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m_run - mu);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
            m_run = m_new;
        }
        const float nmu = (m_run == -INFINITY) ? 0.0f : -m_run;
        // ---- P = 2^(s*c2 - m), packed to bf16 in the B-operand order; l from the
        // rounded P that the PV MFMA uses (a dot2 with (1, 1)) ----
        const bf16x2 ones = as_bf16x2(0x3F803F80u);
        uint32_t pk[2][8];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(s[sb][r], c2, nmu));
                const float p1 = fast_exp2(fmaf(s[sb][r + 1], c2, nmu));
                pk[sb][r / 2] = pack_bf16_rne(p0, p1);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pk[sb][r / 2]), ones, l_run, false);
            }
        // ---- O^T += V^T P^T, V^T fragments by transposed LDS reads ----
#pragma unroll
        for (int m = 0; m < kBN / 16; ++m) {
            const int sb = m / 2, r0 = 4 * (m % 2);
            const uint4 pu = make_uint4(pk[sb][r0], pk[sb][r0 + 1], pk[sb][r0 + 2], pk[sb][r0 + 3]);
            const bf16x8 pf = __builtin_bit_cast(bf16x8, pu);
            const int vr = 16 * m + tr_row;
            uint32_t addr[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db)
                addr[db] = lds_addr(vs + vr * D + (((4 * db + tr_chunk) ^ swz_v<D>(vr)) << 3) + tr_sub);
            uint2 lo[DB], hi[DB];
            tr_reads<DB, 8 * D * 2>(lo, hi, addr);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo[db].x, lo[db].y, hi[db].x, hi[db].y));
                acc_o[db] = mfma32(vf, pf, acc_o[db]);
            }
        }
    };

    // One pipeline step on tile kb, read from stage (kc, vc).  It refills stage
    // (kn, vn) with tile kb + 2.  Steps past kb1 only keep the direct loads
    // balanced: the refill is clamped to kb1, and there is no math.
    int pg_next[4];
    auto step = [&](int kb, uint16_t* kc, uint16_t* vc, uint16_t* kn, uint16_t* vn) {
        wait_vmcnt<NL>();                                  // this wave's share of tile kb landed
        __builtin_amdgcn_s_barrier();                      // ... everyone's; stage kn is free
        if (kb <= kb1 && kb * kBN + kBN > n) {
            // rows past the sequence end hold whatever the page slots hold: zero V
            const int r0 = max(0, n - kb * kBN);
            for (int e = tid; e < (kBN - r0) * CPR; e += kThreads)
                *reinterpret_cast<uint4*>(vc + (r0 + e / CPR) * D + (e % CPR) * 8) = make_uint4(0, 0, 0, 0);
            __syncthreads();
        }
        issue(pg_next, kn, vn);                            // tile min(kb + 2, kb1)
        tile_pages(min(kb + 3, kb1), pg_next);
        const int key0 = kb * kBN;
        if (kb <= kb1 && wave_live && key0 < w_hi && key0 + kBN > w_lo) compute(kb, kc, vc);
    };

    {
        int pg[4];
        tile_pages(kb0, pg);
        issue(pg, k_s0, v_s0);
        tile_pages(min(kb0 + 1, kb1), pg);
        issue(pg, k_s1, v_s1);
        tile_pages(min(kb0 + 2, kb1), pg_next);
    }
    for (int kb = kb0; kb <= kb1; kb += 3) {
        step(kb, k_s0, v_s0, k_s2, v_s2);
        step(kb + 1, k_s1, v_s1, k_s0, v_s0);
        step(kb + 2, k_s2, v_s2, k_s1, v_s1);
    }
    wait_vmcnt<0>();          // drain the trailing refills before the workgroup retires

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
        hipLaunchKernelGGL((prefill_kernel<D, G, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, a.block_table);
    else
        hipLaunchKernelGGL((prefill_kernel<D, G, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, a.block_table);
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

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
//    a 5-stage ring of 64-key tiles (4 pages).  A tile is made visible (each wave
//    waits on its own vmcnt, then the one barrier per tile) two iterations before
//    its PV, so the barrier sits in the middle of an iteration while the matrix
//    core still has queued work.  The page ids of later tiles are read
//    (wave-uniform, scalar loads) a tile before they are needed.
//  * The loop is software-pipelined within each wave, so that the matrix cores
//    and the VALU work at the same time (on gfx950 each MFMA issue also takes
//    VALU issue cycles, so the VALU work is spread evenly): the QK^T MFMAs of
//    tile j+1 are interleaved with the exps of tile j (64-key build; the 32-key
//    build puts three quarters of them there), and the PV MFMAs of tile j with
//    the rest and the row max of tile j+1.
//    Scheduling fences bound how far the compiler hoists LDS reads (registers);
//    K fragments are read two D-slices ahead, and the per-lane LDS offsets are
//    computed once, so a read costs one add of the stage base.
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
//      - Q and K enter the MFMA as they are (bf16), so q.k is exact up to fp32
//        summation; p = exp2(c*s - m) with c = sm_scale*log2 e is one FMA and one
//        v_exp_f32 per score.  (Folding c into Q would save the FMA but round Q*c
//        to bf16, an error that grows with the logits.)
//      - the row max is taken on the raw scores (c > 0);
//      - P is rounded to bf16 (RNE) for the PV MFMA;
//      - the row sum is a dot2 of those rounded pairs with (1, 1), so l matches the
//        numerator exactly;
//      - the reference max moves only when a row's max exceeds it by more than 8
//        (log2 units), so p <= 2^8.
//  * Causal/window masking costs nothing on tiles that are fully visible.  A wave
//    skips the MFMAs of tiles that lie entirely outside its rows' ranges.  V rows
//    past the sequence end are zeroed in LDS, so poison in unwritten page slots
//    never meets a zero weight.
//  * Workgroups map to XCDs so that each XCD's L2 holds the K/V of the heads it
//    serves.  Within an XCD the longest (latest) query tiles go first.
//  * INT8 caches (KV8): the tiles come in through registers (compiler-tracked
//    loads, one tile ahead) and are converted into the same bf16 LDS tiles before
//    the barrier that publishes them.  K is stored exactly, as the codes c (bf16
//    holds every |c| <= 127), so the MFMA yields q.c exactly (up to fp32
//    summation), and each score is then multiplied by its key's scale * sm_scale *
//    log2 e (from LDS) before the mask, max and exp.  V is stored as bf16(c * scale_v): its rounding enters the output
//    linearly, at most 2^-9 relative per element.  The ring has 4 stages (the
//    converted tile reuses the stage freed one barrier earlier).
//  * Split mode covers a short chunk on a long prefix, such as 130 new tokens on
//    8192.  Such a chunk has too few query tiles to fill 256 CUs, so the key
//    range is cut into max_splits ranges of split_keys keys, a multiple of 64.
//    Each workgroup writes a softmax-normalised partial with its natural
//    log-sum-exp, and the combine kernel then merges them with the sink.
#include <type_traits>

#include "pfa_device.h"

// Two builds of this file: the default one (256-row workgroups, 64-key tiles,
// 160 KB of LDS at D = 128, one workgroup per CU) and, from prefill_split.hip, the
// KV-split one (128-row workgroups, 32-key tiles, 80 KB, two workgroups per CU),
// which fills the chip better when a short chunk is spread over key splits.
#ifndef PFA_PREFILL_BN
#define PFA_PREFILL_BN 64
#define PFA_PREFILL_ROWS_WG kPrefillRows
#define PFA_PREFILL_LAUNCH launch_prefill
#endif

// Barrier audit: with PFA_PREFILL_AUDIT=1 every ring step waits for all of the
// wave's loads (vmcnt 0) and then for every wave (s_barrier), before and after it
// refills a stage, and the prologue waits for every tile it issued.  The hand-
// placed waits of the normal build (each wave waits only for the tile it is about
// to make visible) must give the same bits; a GPU test compares the two builds.
#ifndef PFA_PREFILL_AUDIT
#define PFA_PREFILL_AUDIT 0
#endif

namespace pfa {
namespace {

constexpr bool kAudit = PFA_PREFILL_AUDIT != 0;
constexpr int kRowsPerWave = 32;
constexpr int kWaves = PFA_PREFILL_ROWS_WG / kRowsPerWave;
constexpr int kThreads = kWaves * kWave;
constexpr int kBN = PFA_PREFILL_BN;   // keys per tile
constexpr int kStages = 5;        // LDS ring depth: tiles kb-1 .. kb+3 around tile kb
constexpr int kPairs1 = kBN == 64 ? 16 : 6;   // of a tile's 8*kBN/32 score pairs per lane,
                                  // those whose exps run beside the QK^T MFMAs (the rest beside PV)
constexpr int kXcds = 8;

#define LDS3 __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte-chunk swizzles (chunk c of row r sits at c ^ f(r)).  K: the 16 rows one
// 16-lane MFMA read touches land on 16 distinct bank quads.  V: the 4 rows x 2
// chunks of a 16-lane transposed read, and 4 rows x 4 chunks per 32 lanes, are
// distinct.  (Rows of D = 64 are 128 B, two rows per bank line.)
template <int D> __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// A wave-uniform pointer, held in scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Barrier that the compiler may not move memory accesses across, after this
// wave's LDS accesses (and scalar loads) have completed.
__device__ __forceinline__ void lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// x, hidden from the optimiser (so that values derived from it are recomputed
// where they are used rather than hoisted)
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(LDS3 const void*)p;
}

template <int D, int G, bool SPLIT, bool KV8>
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

    // ring of NST stages, each a K tile then a V tile (keys x D, swizzled); INT8
    // adds each stage's per-key score multipliers
    constexpr int NST = KV8 ? 4 : kStages;
    __shared__ __attribute__((aligned(1024))) uint16_t ring_lds[NST * 2 * kBN * D];
    __shared__ __attribute__((aligned(16))) float kmul_lds[KV8 ? NST * kBN : 4];
    // INT8 staging: elements of K (and of V) one thread converts per tile
    constexpr int EPT = kBN * D / kThreads;
    static_assert(!KV8 || (EPT == 8 || EPT == 16), "INT8 staging");

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
    const int n_raw = __ldg(a.seq_lens + b);
    if constexpr (kBoundsCheck) {
        if (tile == 0 && split == 0) {
            report(a.err, n_raw < 0 || n_raw > a.bt_stride * kPage ||
                              (SPLIT && (int64_t)a.max_splits * a.split_keys < n_raw),
                   PFA_BOUNDS_SEQ_LEN);
            report(a.err, q_len < 0 || q_len > a.max_q_len || q_len > n_raw, PFA_BOUNDS_Q_LEN);
        }
    }
    if (tok0 >= q_len) return;
    const int n = min(max(n_raw, 0), a.bt_stride * kPage);
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
    // Scores leave the MFMA as s = q.k; p = 2^(c2 s - mu) with c2 = sm_scale * log2 e
    // and mu the row's reference max (log2 units).
    const float c2 = a.sm_scale * kLog2e;
    // the multiplier of the scores in the exp: c2, or 1 for INT8, whose scores are
    // scaled per key before the mask (by the key's scale times c2)
    const float cexp = KV8 ? 1.0f : c2;
    bf16x8 qf[KK];
    {
        const uint16_t* qp = a.q + ((int64_t)(cq0 + tok_l) * Hq + h_l) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_ok) v = *reinterpret_cast<const uint4*>(qp + 16 * kk);
            if constexpr (KV8) {
                // keys stored smoothed (k / s, s a power of two): q meets q * s, exact
                if (a.k_smooth) {
                    const float* sp = a.k_smooth + 16 * kk + 8 * half;
                    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        w[i] = pack_bf16_rne(bf16_lo(w[i]) * smooth_pow2(__ldg(sp + 2 * i)),
                                             bf16_hi(w[i]) * smooth_pow2(__ldg(sp + 2 * i + 1)));
                    v = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
            qf[kk] = __builtin_bit_cast(bf16x8, v);
        }
        // The direct loads below are invisible to the compiler's vmcnt tracking.
        // Retire the Q loads here, or the compiler would wait for them (vmcnt 0,
        // hence for every tile in flight) at each use of Q inside the tile loop.
        wait_vmcnt<0>();
    }

    // ---- direct HBM -> LDS tile loads ----
    // a __restrict__ kernel argument: uniform reads of it become scalar loads, which
    // stay out of the vmcnt queue the direct loads are counted on
    const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
    const int npg = (n + kPage - 1) / kPage;
    const int64_t hblk = (int64_t)kPage * D;            // elements per page-head block
    const int kb0 = lo / kBN;
    const int kb1 = (hi - 1) / kBN;
    // A wave's direct loads cover 8 consecutive rows of the tile, all in one page.
    static_assert(DMA_PER_WAVE * ROWS_PER_DMA * kWaves == kBN && kPage % (DMA_PER_WAVE * ROWS_PER_DMA) == 0,
                  "a wave's rows lie in one page");
    const int wpage = wave * DMA_PER_WAVE * ROWS_PER_DMA / kPage;    // which page of the tile
    // raw block-table entry of a tile's page for this wave (a scalar load), and
    // its clamp to the pool; the load is issued one tile before its value is used.
    // The entry's index stays inside the sequence's row even when a broken length
    // leaves no visible page (npg <= 0, or a tile range below 0).
    auto raw_page = [&](int kb) __attribute__((always_inline)) {
        return __ldg(bt + min(max(kb * (kBN / kPage) + wpage, 0), max(npg, 1) - 1));
    };
    auto clamp_page = [&](int v) __attribute__((always_inline)) {
        report(a.err, v < 0 || v >= a.num_pages, PFA_BOUNDS_PAGE);
        return min(max(v, 0), a.num_pages - 1);
    };
    const int lrow = lane / CPR;                          // row within one direct load
    const int lchunk = lane % CPR;                        // physical chunk this lane fills
    // per-lane byte offsets within a page-head block (the same for every tile)
    uint32_t koff[DMA_PER_WAVE], voff[DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int row = (wave * DMA_PER_WAVE + i) * ROWS_PER_DMA + lrow;
        koff[i] = 2u * ((row % kPage) * D + (lchunk ^ swz_k<D>(row)) * 8);
        voff[i] = 2u * ((row % kPage) * D + (lchunk ^ swz_v<D>(row)) * 8);
    }
    const uint16_t* kpool_h = uniform_ptr(a.k_pool + (int64_t)kvh * hblk);
    const uint16_t* vpool_h = uniform_ptr(a.v_pool + (int64_t)kvh * hblk);
    const int64_t page_stride = (int64_t)a.num_kv_heads * hblk;
    // LDS byte addresses: the ring's stages, each a K tile then a V tile
    const uint32_t ring0 = lds_addr(ring_lds);
    constexpr uint32_t kTileBytes = kBN * D * 2;
    auto issue = [&](int pg, uint32_t kdst, uint32_t vdst) __attribute__((always_inline)) {
        if constexpr (KV8) return;
        const int64_t pbase = (int64_t)pg * page_stride;
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i) {
            const uint32_t row0 = (wave * DMA_PER_WAVE + i) * ROWS_PER_DMA;
            dma16(kpool_h + pbase, koff[i], kdst + row0 * D * 2);
            dma16(vpool_h + pbase, voff[i], vdst + row0 * D * 2);
        }
    };

    // ---- INT8: tiles through registers ----
    // Thread tid holds EPT codes of key row tid / (D / EPT) of a tile (8 threads
    // per row; a wave's 8 rows lie in one page, the page raw_page reads), for K and
    // for V, plus that row's two scales.
    typedef typename std::conditional<EPT == 16, uint4, uint2>::type CodeT;
    const int st_row = tid / (D / EPT), st_chunk = tid % (D / EPT);
    CodeT st_k{}, st_v{};
    float st_ks = 0.0f, st_vs = 0.0f;
    const int8_t* kcodes_h = reinterpret_cast<const int8_t*>(a.k_pool) + (int64_t)kvh * hblk;
    const int8_t* vcodes_h = reinterpret_cast<const int8_t*>(a.v_pool) + (int64_t)kvh * hblk;
    auto stage_load = [&](int pg) __attribute__((always_inline)) {
        if constexpr (KV8) {
            const int64_t blk = (int64_t)pg * a.num_kv_heads;              // + kvh in the bases
            const int64_t off = blk * hblk + (st_row % kPage) * D + st_chunk * EPT;
            st_k = *reinterpret_cast<const CodeT*>(kcodes_h + off);
            st_v = *reinterpret_cast<const CodeT*>(vcodes_h + off);
            const int64_t si = (blk + kvh) * kPage + st_row % kPage;
            st_ks = __ldg(a.k_scale + si);
            st_vs = __ldg(a.v_scale + si);
        }
    };
    // Convert the staged tile kb (key rows kb*kBN + row) into the bf16 LDS stage
    // kdst/vdst (same layout and swizzles as the direct loads), and its score
    // multipliers into kmul_lds[mi .. mi + kBN).  V:
    // c * scale_v rounded to bf16, 0 past the sequence end (where scales may be
    // poison).  Multiplier: scale_k * sm_scale * log2 e, 0 past the end (the mask
    // then sets those scores to -inf).  K: the codes c themselves, exact in bf16.
    auto stage_convert = [&](int kb, uint32_t kdst, uint32_t vdst, int mi) __attribute__((always_inline)) {
        if constexpr (KV8) {
            const int row = st_row;
            const bool live = kb * kBN + row < n;
            uint32_t cw[EPT / 4];
            uint32_t vw_[EPT / 4];
            __builtin_memcpy(cw, &st_k, sizeof(cw));
            __builtin_memcpy(vw_, &st_v, sizeof(vw_));
            uint32_t ko[EPT / 2], vo[EPT / 2];
            const float vs = live ? st_vs : 0.0f;
#pragma unroll
            for (int i = 0; i < EPT / 4; ++i) {
                float kx[4], vx[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kx[e] = (float)(int8_t)(cw[i] >> (8 * e));
                    vx[e] = (float)(int8_t)(vw_[i] >> (8 * e));
                }
                ko[2 * i] = pack_hi16(kx[0], kx[1]);
                ko[2 * i + 1] = pack_hi16(kx[2], kx[3]);
                // past the end vs is 0 and the codes are finite: the pair is (+-)0
                vo[2 * i] = pack_bf16_rne(vx[0] * vs, vx[1] * vs);
                vo[2 * i + 1] = pack_bf16_rne(vx[2] * vs, vx[3] * vs);
            }
#pragma unroll
            for (int c = 0; c < EPT / 8; ++c) {
                const int lc = st_chunk * (EPT / 8) + c;             // 8-element chunk in the row
                const uint32_t kofs_b = (uint32_t)(row * D * 2 + ((lc ^ swz_k<D>(row)) << 4));
                const uint32_t vofs_b = (uint32_t)(row * D * 2 + ((lc ^ swz_v<D>(row)) << 4));
                *(LDS3 u32x4*)(uintptr_t)(kdst + kofs_b) = u32x4{ko[4 * c], ko[4 * c + 1], ko[4 * c + 2], ko[4 * c + 3]};
                *(LDS3 u32x4*)(uintptr_t)(vdst + vofs_b) = u32x4{vo[4 * c], vo[4 * c + 1], vo[4 * c + 2], vo[4 * c + 3]};
            }
            if (st_chunk == 0) kmul_lds[mi + row] = live ? st_ks * c2 : 0.0f;
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

    // per-lane constants of the transposed V reads
    const int tr_g = lane / 16, tr_j = lane % 16;
    const int tr_row = 4 * (tr_g / 2) + tr_j / 4;                 // + 16m (+ 8 for the upper half)
    const int tr_chunk = 2 * (tr_g % 2) + (tr_j % 4) / 2;         // + 4db
    const int tr_sub = 4 * (tr_j % 2);

    // A tile's scores per lane: NH halves of 32 keys (one f32x16 MFMA output each),
    // NP = 8*NH packed bf16 pairs of P, NS = kBN/16 key slices for the PV MFMAs.
    constexpr int NH = kBN / 32, NP = 8 * NH, NS = kBN / 16;
    typedef f32x16 Scores[NH];
    typedef uint32_t Packed[NH][8];

    // S^T = K Q^T, one MFMA chain per 32-key half.  Per-lane LDS byte offsets of
    // the K reads (one per D-slice kk; the halves add 32 rows) and of the
    // transposed V reads (one per 32-dim block db; slice m and the upper key half
    // add constants), computed once: a read then costs one add of the stage base.
    int kofs[KK], vofs[DB];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kofs[kk] = 2 * r32 * D + (((2 * kk + half) ^ swz_k<D>(r32)) << 4);
    // the swizzle of row 16m + tr_row is that of tr_row
#pragma unroll
    for (int db = 0; db < DB; ++db)
        vofs[db] = 2 * (tr_row * D + (((4 * db + tr_chunk) ^ swz_v<D>(tr_row)) << 3) + tr_sub);
    auto k_frag = [&](uint32_t ks, int kk, bf16x8 (&k)[NH]) __attribute__((always_inline)) {
        const LDS3 char* p = (const LDS3 char*)(uintptr_t)(ks + kofs[kk]);
#pragma unroll
        for (int h = 0; h < NH; ++h) k[h] = *(const LDS3 bf16x8*)(p + 2 * 32 * D * h);
    };
    // mask tile kb's scores in place (only tiles that cross a row's causal or
    // window edge need it)
    auto tile_full = [&](int kb) __attribute__((always_inline)) {
        const int key0 = kb * kBN;
        return (key0 + kBN - 1 <= prefix + w_first) && (W == 0 || (prefix + w_last) - key0 < W);
    };
    // INT8: multiply each score by its key's multiplier (stage of tile kb).  A lane
    // holds keys 32h + 8(r/4) + (r%4) + 4*half: four consecutive ones per read.
    auto scale_scores = [&](int kb, Scores& s) __attribute__((always_inline)) {
        if constexpr (KV8) {
            const int mi = ((kb - kb0) % NST) * kBN + 4 * half;
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 m = *(const LDS3 f32x4*)(uintptr_t)lds_addr(&kmul_lds[mi + 32 * h + 8 * q]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[h][4 * q + i] *= m[i];
                }
        }
    };
    auto mask = [&](int kb, Scores& s) __attribute__((always_inline)) {
        // distance of this lane's first key in the tile from its row position
        const int d0 = opaque(pos_l - kb * kBN - 4 * half);
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dist = d0 - (32 * h + 8 * (r / 4) + (r % 4));      // pos - key
                const bool vis = dist >= 0 && (W == 0 || dist < W);
                s[h][r] = vis ? s[h][r] : -INFINITY;
            }
    };
    // Lazy rescale with headroom: the reference max moves only when a row's max
    // exceeds it by more than 8, so p <= 2^8 (exact enough in bf16, no overflow in
    // the fp32 sums).  O and l share the reference, so o/l is unchanged.  mt is
    // the lane's max of the tile's raw scores.
    auto rescale = [&](float mt) __attribute__((always_inline)) {
        mt = xor32_max(mt) * cexp;
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
    };
    // the row max of the raw scores (the scale is positive), then the rescale
    auto mask_max = [&](int kb, Scores& s) __attribute__((always_inline)) {
        if (!tile_full(kb)) mask(kb, s);
        float mt = -INFINITY;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[h][r]);
        rescale(mt);
    };
    // P = 2^(c2 s - mu), packed to bf16 in the B-operand order; l from the rounded
    // P that the PV MFMA uses (a dot2 with (1, 1))
    auto exp_pair = [&](const Scores& s, Packed& pk, int q, float nmu) __attribute__((always_inline)) {
        const int h = q / 8, r = 2 * (q % 8);
        const float p0 = fast_exp2(fmaf(s[h][r], cexp, nmu));
        const float p1 = fast_exp2(fmaf(s[h][r + 1], cexp, nmu));
        pk[h][r / 2] = pack_bf16_rne(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pk[h][r / 2]), as_bf16x2(0x3F803F80u), l_run, false);
    };
    // exps of pairs [qa, qb) pinned to the current bundle: the empty asm makes their
    // results exist here, so the optimiser cannot sink the exps out of the bundle
    // they are meant to fill (within the bundle the pairs' chains interleave)
    auto exp_pairs_here = [&](const Scores& s, Packed& pk, int qa, int qb, float nmu) __attribute__((always_inline)) {
#pragma unroll
        for (int q = qa; q < qb; ++q) exp_pair(s, pk, q, nmu);
#pragma unroll
        for (int q = qa; q < qb; ++q) asm volatile("" : "+v"(pk[q / 8][q % 8]));
        asm volatile("" : "+v"(l_run));
    };
    auto softmax = [&](const Scores& s, Packed& pk) __attribute__((always_inline)) {
        const float nmu = (m_run == -INFINITY) ? 0.0f : -m_run;
#pragma unroll
        for (int q = 0; q < NP; ++q) exp_pair(s, pk, q, nmu);
    };
    // Block 1: S' = K' Q^T, optionally with pairs [0, P1) of the current tile's
    // exps interleaved (EXP).  Bundles of one D-slice each: the K reads of slice
    // kk+1, the NH MFMAs of slice kk, a share of the exps.  A scheduling fence
    // after each bundle keeps the compiler from hoisting every read of the block
    // (which costs registers the scores need).
    auto qk_block = [&](bool EXP, int P1, uint32_t ks, Scores& sn, const Scores& s, Packed& pk) __attribute__((always_inline)) {
        const float nmu = (m_run == -INFINITY) ? 0.0f : -m_run;
        // K fragments two D-slices ahead of the MFMAs that use them
        bf16x8 kq[KK][NH];
        k_frag(ks, 0, kq[0]);
        if (KK > 1) k_frag(ks, 1, kq[1]);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) k_frag(ks, kk + 2, kq[kk + 2]);
            bf16x8 (&k)[NH] = kq[kk];
            const int pa = kk * P1 / KK, pb = (kk + 1) * P1 / KK;
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                if (kk == 0) {
                    const f32x16 z = {};
                    sn[h] = mfma32(k[h], qf[0], z);
                } else {
                    sn[h] = mfma32(k[h], qf[kk], sn[h]);
                }
                // this MFMA's share of the bundle's exps
                if (EXP) {
                    const int qa = pa + h * (pb - pa) / NH, qb = pa + (h + 1) * (pb - pa) / NH;
                    exp_pairs_here(s, pk, qa, qb, nmu);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Block 2: O^T += V^T P^T over the NS 16-key slices, optionally (FUSED) with
    // the exps of pairs [P1, NP) of the tile (the last slice's P, computed during
    // the slices before it) and the row max of the next tile's scores sn (during
    // the slices after the first, once their MFMAs have long finished), then the
    // rescale.
    auto v_frag = [&](uint32_t vs, int m, int db) __attribute__((always_inline)) {
        const LDS3 char* p = (const LDS3 char*)(uintptr_t)(vs + vofs[db]) + 2 * 16 * m * D;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 s16x4*)p);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 s16x4*)(p + 2 * 8 * D));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // the slice-0 V fragments of a PV block, read ahead of it
    typedef bf16x8 VHead[DB];
    auto pv_head = [&](uint32_t vs, VHead& vh) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) vh[db] = v_frag(vs, 0, db);
    };
    auto pv_block = [&](bool FUSED, int P1, uint32_t vs, VHead& vf, Packed& pk, const Scores& s, Scores& sn) __attribute__((always_inline)) {
        const float nmu = (m_run == -INFINITY) ? 0.0f : -m_run;
        float mt = -INFINITY;
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int h = m / 2, r0 = 4 * (m % 2);
            const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pk[h][r0], pk[h][r0 + 1], pk[h][r0 + 2], pk[h][r0 + 3]));
            // one register set per 32-dim block: slice m+1 is read into it as soon as
            // the MFMA of slice m that reads it has issued
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc_o[db] = mfma32(vf[db], pf, acc_o[db]);
                if (m + 1 < NS) vf[db] = v_frag(vs, m + 1, db);
            }
            if (FUSED) {
                if (m < NS - 1) {
                    const int pa = P1 + m * (NP - P1) / (NS - 1), pb = P1 + (m + 1) * (NP - P1) / (NS - 1);
                    exp_pairs_here(s, pk, pa, pb, nmu);
                }
                if (m > 0) {
#pragma unroll
                    for (int e = 16 * NH * (m - 1) / (NS - 1); e < 16 * NH * m / (NS - 1); ++e)
                        mt = fmaxf(mt, sn[e / 16][e % 16]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FUSED) rescale(mt);
    };
    // rows of a tile past the sequence end hold whatever the page slots hold: zero V
    auto zero_tail = [&](int kb, uint32_t vs) __attribute__((always_inline)) {
        if (kb <= kb1 && kb * kBN + kBN > n) {
            const int r0 = max(0, n - kb * kBN);
            for (int e = tid; e < (kBN - r0) * CPR; e += kThreads)
                *(LDS3 u32x4*)(uintptr_t)(vs + 2 * ((r0 + e / CPR) * D + (e % CPR) * 8)) = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // Software pipeline over a 5-stage ring.  Tile kb sits in stage
    // (kb - kb0) % kStages.  Every wave runs ring(kb) once for each tile kb0..kb1;
    // ring(kb) makes tile kb+2 visible (each wave waits for its own direct loads,
    // then the barrier), refills the stage of tile kb-1 with tile kb+4 (clamped to
    // kb1, so the load count stays balanced) and zeroes tile kb+2's V rows past the
    // sequence end (visible from the next barrier on).  Because tiles are made
    // visible two iterations before their PV, the barrier can sit in the middle of
    // an iteration, where the matrix core still has block 1's MFMAs to run:
    //   block 1: S' = K_{kb+1} Q^T (MFMA) interleaved with most of P = exp2(S - m);
    //   ring(kb), with the first V reads of block 2 issued right after the barrier;
    //   block 2: O += P V_kb (MFMA) interleaved with the rest of the exps and the
    //     row max of S', then the rescale for tile kb+1.
    // A wave computes only on the tiles kw0..kw1 its rows see; the range's first
    // tile gets its S before ring(kw0 - 1), its last one only P and PV.
    auto kst = [&](int kb) { return ring0 + (uint32_t)((kb - kb0) % NST) * (2 * kTileBytes); };
    auto mst = [&](int kb) { return ((kb - kb0) % NST) * kBN; };
    auto vst = [&](int kb) { return kst(kb) + kTileBytes; };
    int pg_raw;                                // raw page entry of tile min(kb + 4, kb1)
    // ring in two parts, so that LDS reads can be issued right after the barrier
    auto ring_pre = [&](int kb) __attribute__((always_inline)) {
        if constexpr (KV8) {
            // tile kb+2 (staged at ring(kb-1)) into the stage of tile kb-2, which the
            // barrier of ring(kb-1) freed
            stage_convert(kb + 2, kst(kb + 2), vst(kb + 2), mst(kb + 2));
        } else {
            // in flight: tiles kb+2 and kb+3 (kb+4 is issued below)
            if constexpr (kAudit) wait_vmcnt<0>();
            else wait_vmcnt<NL>();             // this wave's share of tile kb+2 landed
        }
        lds_sync();                            // everyone's; tile kb-1's stage is free
    };
    auto ring_post = [&](int kb) __attribute__((always_inline)) {
        if constexpr (KV8) {
            stage_load(clamp_page(pg_raw));    // tile min(kb + 3, kb1)
            pg_raw = raw_page(min(kb + 4, kb1));
        } else {
            issue(clamp_page(pg_raw), kst(kb + 4), vst(kb + 4));   // tile min(kb + 4, kb1)
            pg_raw = raw_page(min(kb + 5, kb1));
            zero_tail(kb + 2, vst(kb + 2));
        }
        if constexpr (kAudit) {
            wait_vmcnt<0>();
            lds_sync();
        }
    };
    auto ring = [&](int kb) __attribute__((always_inline)) { ring_pre(kb); ring_post(kb); };
    // this wave's tiles
    int kw0 = kb0, kw1 = kb0 - 1;
    if (wave_live) {
        kw0 = max(kb0, w_lo / kBN);
        kw1 = min(kb1, (w_hi - 1) / kBN);
    }
    const bool any = kw0 <= kw1;

    if constexpr (KV8) {
        // tiles kb0 and kb0+1 converted, kb0+2 staged
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            stage_load(clamp_page(raw_page(min(kb0 + i, kb1))));
            stage_convert(kb0 + i, kst(kb0 + i), vst(kb0 + i), mst(kb0 + i));
        }
        stage_load(clamp_page(raw_page(min(kb0 + 2, kb1))));
        pg_raw = raw_page(min(kb0 + 3, kb1));
        lds_sync();
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) issue(clamp_page(raw_page(min(kb0 + i, kb1))), kst(kb0 + i), vst(kb0 + i));
        pg_raw = raw_page(min(kb0 + 4, kb1));
        if constexpr (kAudit) wait_vmcnt<0>();
        else wait_vmcnt<2 * NL>();             // tiles kb0, kb0+1 landed (kb0+2, kb0+3 in flight)
        lds_sync();
        zero_tail(kb0, vst(kb0));              // visible after the next barrier
        zero_tail(kb0 + 1, vst(kb0 + 1));
    }

    Scores s_a, s_b;                           // scores of the current / next tile
    Packed pk;
    VHead vh;
    int kb = kb0;
    if (any) {
        for (; kb < kw0 - 1; ++kb) ring(kb);
        // tile kw0 became visible at ring(kw0 - 2) or in the prologue
        qk_block(false, 0, kst(kw0), s_a, s_b, pk);
        scale_scores(kw0, s_a);
        mask_max(kw0, s_a);
        if (kw0 > kb0) ring(kb++);             // ring(kw0 - 1)
        // fused iterations kw0 .. kw1-1, two per round (the score buffers swap)
        auto fused = [&](int t, Scores& sc, Scores& sn) __attribute__((always_inline)) {
            qk_block(true, kPairs1, kst(t + 1), sn, sc, pk);
            scale_scores(t + 1, sn);
            if (!tile_full(t + 1)) mask(t + 1, sn);
            ring_pre(t);
            pv_head(vst(t), vh);
            ring_post(t);
            pv_block(true, kPairs1, vst(t), vh, pk, sc, sn);
        };
        for (; kb + 1 < kw1; kb += 2) {
            fused(kb, s_a, s_b);
            fused(kb + 1, s_b, s_a);
        }
        if (kb < kw1) {
            fused(kb, s_a, s_b);
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int r = 0; r < 16; ++r) s_a[h][r] = s_b[h][r];
            ++kb;
        }
        softmax(s_a, pk);                      // tile kw1: P and PV only
        ring_pre(kb);
        pv_head(vst(kw1), vh);
        ring_post(kb++);
        pv_block(false, NP, vst(kw1), vh, pk, s_a, s_a);
    }
    for (; kb <= kb1; ++kb) ring(kb);
    wait_vmcnt<0>();          // drain the trailing refills before the workgroup retires

    // ---- finish: combine the two lanes of each row ----
    const float l_tot = xor32_sum(l_run);
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

template <int D, int G, bool KV8>
hipError_t launch_dg(const PrefillArgs& a, hipStream_t s) {
    constexpr int TPB = kRowsPerWave / G * kWaves;
    const int n_tiles = (a.max_q_len + TPB - 1) / TPB;
    const bool split = a.max_splits > 1;
    const int64_t items = (int64_t)a.batch * a.num_kv_heads * n_tiles * (split ? a.max_splits : 1);
    const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
    if (grid == 0) return hipSuccess;
    if (split)
        hipLaunchKernelGGL((prefill_kernel<D, G, true, KV8>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, a.block_table);
    else
        hipLaunchKernelGGL((prefill_kernel<D, G, false, KV8>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, a.block_table);
    return hipGetLastError();
}

template <int D, bool KV8>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_dg<D, 1, KV8>(a, s);
        case 2: return launch_dg<D, 2, KV8>(a, s);
        case 4: return launch_dg<D, 4, KV8>(a, s);
        case 8: return launch_dg<D, 8, KV8>(a, s);
        case 16: return launch_dg<D, 16, KV8>(a, s);
        case 32: return launch_dg<D, 32, KV8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t PFA_PREFILL_LAUNCH(const PrefillArgs& a, int head_dim, hipStream_t s) {
    if (a.batch == 0 || a.max_q_len == 0) return hipSuccess;
    if (a.k_scale) return head_dim == 128 ? launch_d<128, true>(a, s) : launch_d<64, true>(a, s);
    return head_dim == 128 ? launch_d<128, false>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace pfa

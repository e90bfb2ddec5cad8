// Split-KV paged decode: one query token per sequence, over its cached pages.
//
// The TileInfer.jl performance page ("Fused kernels, FlashAttention and
// PagedAttention") does decode this way.  It runs an online softmax over the pages
// in place, reading each page once through the block table, and splits the keys of
// a sequence so that many workgroups share one sequence.  A separate combine then
// merges the splits.  Its "INT8 KV cache" section keeps one scale per cached
// vector.  It also loads 32-key tiles and each half of the head dimension
// separately, so the INT8 kernel stays spill-free.
//
// MI355X design.  The kernel is HBM-bound (INT8 at G = 8: bound by VALU issue), and
// each K/V element is used by exactly one lane group, so K/V go straight from HBM to
// registers (INT8 at G = 8: straight into a 2-stage LDS ring, below):
//  * One wave per (split, KV head, sequence) streams the split's pages, with the
//    next page always in flight.  The grid is 1-D with the KV head fastest, then
//    the split, then the sequence: workgroup i runs on XCD i % 8, so each XCD
//    gets the same share of every sequence, and the KV-head blocks of a page are
//    read at about the same time.  Measured alternatives, all slower on some
//    workload: the split fastest (XCD imbalance on ragged batches: split i always
//    lands on XCD i % 8), the sequence fastest, several waves per split, several
//    splits per wave, and a balanced persistent schedule over resident waves,
//    static or through an atomic work counter.  The G = Hq/Hkv query heads of the
//    group share every page read (GQA packing).
//  * Page-head block = 16 keys x D.  A lane loads 8 consecutive elements of one key
//    per load (16 B for bf16, 8 B for int8).  LPK = D/8 lanes cover a key, and one
//    load instruction covers a contiguous 512*elem-byte run.  The wave's next page
//    is prefetched while the current one is consumed; two or three pages in
//    flight (a ring of register sets) measured no faster.  For INT8 and for G = 8
//    the page ids are scalar loads issued a page ahead (see kScalarIds), and two
//    register sets take the pages in turn.
//  * q.k: v_dot2_f32_bf16 on (q, k) bf16 pairs.  INT8: v_dot2_f32_f16 on fp16
//    pairs, the codes as 1152 + c (one byte permute per two codes builds the fp16
//    words 0x64uu = 1024 + u, u = c + 128), and 1152*sum(q) is subtracted from
//    the dot.  q is scaled per head by a power of two into fp16's range (exact
//    for every element within 2^28 of the head's largest); at G = 8 the key
//    groups of a wave share that conversion through LDS.  With key smoothing
//    (keys stored as k/s per channel, the "INT8 KV cache" section's smoothing by
//    the key norm's weight, s taken as a power of two), q is first scaled by s,
//    which is exact too.
//    A lane's partial dots for the G heads go through a transposed butterfly over
//    the LPK lanes, on DPP moves only (group_reduce.h).  Slot j of a lane holds
//    head (j ^ myhead), so each stage adds a partner's slots to its own lower half
//    with no selects, and ends with the lane holding its own head's full score.
//    INT8 at G = 8, D = 128 (two lanes per head) runs it over two keys at once,
//    so the two lanes of a head end on different keys and each scores half.
//  * The softmax max is taken per page and the rescale is lazy with headroom: o
//    and l are rescaled only when some head's max exceeds the reference max by
//    more than 8 (log2 units), so weights stay <= 2^8.  At G = 8 a rescale on
//    every growth ran on most of a split's first pages (INT8 at batch 8 x 32768:
//    92 -> 85 us).  (INT8 at G = 8 compares each score with its head's threshold
//    and reduces the page max across lanes only when one passes.)  The weights p
//    are shared within the wave through LDS.
//  * p.v: for G <= 4, fp32 FMAs on the lane's 8 elements for all G heads.  For
//    G = 8, the VALU budget forces dot2 on key pairs from two loads.  The lane
//    that computes a head's weights w for two keys rounds them to a pair once
//    (nearest even) and shares the pair through LDS:
//      - BF16: w = p as a bf16 pair; the (v_a, v_b) pairs are built by v_perm; l
//        sums the same rounded weights (a dot2 with (1, 1)), so numerator and
//        denominator agree;
//      - INT8: by columns.  The page's V codes sit in LDS, and each lane owns
//        the columns d = lane + 64c of all 16 keys (transposed 8-bit reads), so
//        its o is 8 heads x D/64 columns instead of 8 heads x 8 elements of its
//        key group (205 -> 159 registers).  The codes enter as the keys do, fp16
//        1152 + c, against w = p*scale_v*2^-vexp as an fp16 pair: vexp is a
//        wave-uniform exponent that follows the largest value scale, so w < 2^15
//        always fits (see vexp below), and 1152 times the sum of the rounded
//        weights leaves at the end.
//  * At the end of a split each wave reduces its partial o across key groups (INT8
//    at G = 8: nothing to reduce) and writes o/l with lse = ln(sum e^s) (split
//    mode), or the final output with the sink (unsplit mode).
#include "group_reduce.h"
#include "merge_splits.h"

// Audit: with PFA_DECODE_AUDIT=1 every INT8 page at G = 8 waits for all of the
// wave's direct loads (the next page's too) before it reads its ring stage; a GPU
// test checks that the normal build gives the same bits.
#ifndef PFA_DECODE_AUDIT
#define PFA_DECODE_AUDIT 0
#endif

namespace pfa {
namespace {

constexpr bool kDecodeAudit = PFA_DECODE_AUDIT != 0;

template <bool INT8> struct Chunk;
template <> struct Chunk<false> { typedef uint4 T; };   // 8 bf16
template <> struct Chunk<true> { typedef uint2 T; };    // 8 int8

__device__ __forceinline__ uint32_t dw(const uint4& c, int i) {
    return i == 0 ? c.x : i == 1 ? c.y : i == 2 ? c.z : c.w;
}
__device__ __forceinline__ uint32_t dw(const uint2& c, int i) { return i == 0 ? c.x : c.y; }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)as_f16x2(w).x; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)as_f16x2(w).y; }
// Round two floats to fp16 (nearest, ties to even) and pack.
__device__ __forceinline__ uint32_t pack_f16_rne(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// K chunk -> four pairs for the q.k dot2.  BF16: the bf16 pairs as loaded.
// INT8: fp16 pairs 1152 + c, exact.  The byte u = c + 128 (the code with its sign
// bit flipped) becomes the low byte of the fp16 word 0x64uu = 1024 + u, so one
// byte permute against the constant 0x64 bytes builds two elements; the caller
// subtracts 1152*sum(q).
__device__ __forceinline__ void k_pairs(const uint4& c, uint32_t (&k)[4]) {
    k[0] = c.x; k[1] = c.y; k[2] = c.z; k[3] = c.w;
}
constexpr float kK8Offset = 1152.0f;
__device__ __forceinline__ void k_pairs(const uint2& c, uint32_t (&k)[4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t u = dw(c, h) ^ 0x80808080u;
        k[2 * h] = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);        // (u0, u1)
        k[2 * h + 1] = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);    // (u2, u3)
    }
}

// V chunk -> 8 floats (unpaired p.v).  INT8 yields the code c itself.
__device__ __forceinline__ void v_floats(const uint4& c, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(dw(c, i));
        x[2 * i + 1] = bf16_hi(dw(c, i));
    }
}
__device__ __forceinline__ void v_floats(const uint2& c, float (&x)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t u = dw(c, h) ^ 0x80808080u;
        x[4 * h + 0] = (float)(u & 0xffu) - 128.0f;
        x[4 * h + 1] = (float)((u >> 8) & 0xffu) - 128.0f;
        x[4 * h + 2] = (float)((u >> 16) & 0xffu) - 128.0f;
        x[4 * h + 3] = (float)(u >> 24) - 128.0f;
    }
}

// Element pairs (a[d], b[d]) of two keys' chunks as bf16, d = 0..7 (paired p.v).
// BF16: by byte permute.  INT8: u = c + 128 of each code, exact in bf16 (the
// caller removes the offset).
__device__ __forceinline__ void v_pairs(const uint4& a, const uint4& b, uint32_t (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __builtin_amdgcn_perm(dw(b, i), dw(a, i), 0x05040100u);
        v[2 * i + 1] = __builtin_amdgcn_perm(dw(b, i), dw(a, i), 0x07060302u);
    }
}
__device__ __forceinline__ void v_pairs(const uint2& a, const uint2& b, uint32_t (&v)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t ua = dw(a, h) ^ 0x80808080u, ub = dw(b, h) ^ 0x80808080u;
        v[4 * h + 0] = pack_hi16((float)(ua & 0xffu), (float)(ub & 0xffu));
        v[4 * h + 1] = pack_hi16((float)((ua >> 8) & 0xffu), (float)((ub >> 8) & 0xffu));
        v[4 * h + 2] = pack_hi16((float)((ua >> 16) & 0xffu), (float)((ub >> 16) & 0xffu));
        v[4 * h + 3] = pack_hi16((float)(ua >> 24), (float)(ub >> 24));
    }
}

// Column p.v (INT8 at G = 8).  A page's V tile is staged in LDS with its rows in
// key-pair order, and each lane reads the columns it owns (d = lane + 64c) for
// 8 rows at a time with ds_read_b64_tr_b8: in each 16-lane group, lane j points
// at row j/2, bytes 8(j%2)..+7 of an 8 x 16-byte block, and lane i receives
// column i of the block, rows in order (checked on gfx950).  The codes enter the
// dot2 as the keys' do, fp16 pairs 1152 + c (k_pairs), against fp16 weights; the
// offset leaves at the end as 1152 times the sum of the rounded weights.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS3 __attribute__((address_space(3)))

// An empty asm that makes x depend on every element of o: loads addressed by x
// cannot then be hoisted above the code that produced o.
template <int G, int N>
__device__ __forceinline__ void order_after(uint32_t& x, float (&o)[G][N]) {
    static_assert(G * N <= 16, "asm operands");
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if constexpr (N == 1) asm volatile("" : "+v"(x) : "v"(o[g][0]));
        else asm volatile("" : "+v"(x) : "v"(o[g][0]), "v"(o[g][1]));
    }
}

// Splits whose merge weights sit in LDS at a time, in the fused merge.
constexpr int kFusedMergeChunk = 256;

// Page ids.  The block table also comes in as a __restrict__ argument of its own:
// reads of it with a wave-uniform index then become scalar loads, counted apart
// from the K/V loads, and each is issued a page ahead of its use.  As a vector
// load issued just before the page's K/V loads, a page id waits for every load in
// flight.  Measured on one MI355X (us per launch, vector -> scalar ids): INT8 at
// G = 8 (batch 8 x 32768) 102 -> 93, BF16 at G = 8 (gpt-oss full layer) 201 ->
// 192, but BF16 at G = 4 on the ragged batch 131 -> 136; so BF16 at G <= 4 keeps
// the vector form.
template <int G, bool INT8>
constexpr bool kScalarIds = INT8 || G >= 8;

template <int D, int G, bool INT8, bool FINAL>
__global__ __launch_bounds__(kWave)
void decode_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
    constexpr int EB = INT8 ? 1 : 2;           // bytes per element
    constexpr int LPK = D / 8;                 // lanes per key
    constexpr int KPL = kWave / LPK;           // keys per load instruction
    constexpr int NLOAD = kPage / KPL;         // loads per page per tensor
    constexpr int HG = LPK / G;                // lanes holding each head after the reduce
    constexpr bool PAIRED = G >= 8;            // p.v by dot2 on key pairs
    constexpr bool VCOL = INT8 && PAIRED;      // column p.v through an LDS V tile
    constexpr int NC = D / kWave;              // VCOL: columns per lane
    constexpr int OJ = VCOL ? NC : 8;          // o elements per lane and head
    static_assert(G <= LPK, "group size");
    static_assert(!PAIRED || NLOAD % 2 == 0, "key pairs");
    static_assert(!VCOL || (2 * kPage * D + 512) * 2 >= kFusedMergeChunk * 4, "merge weights in the ring");
    // VCOL with two lanes per head (D = 128): the two lanes of a head end the
    // butterfly on different keys, so each lane scores and weighs half the keys
    constexpr bool JOINT = VCOL && HG == 2;
    constexpr int NS = JOINT ? NLOAD / 2 : NLOAD;   // scores per lane and page
    typedef typename Chunk<INT8>::T CT;

    // weights of a page, double-buffered: [key][head] floats (G <= 4), or for
    // G = 8 [key pair][key group][head] bf16 pairs (VCOL: one buffer, since a
    // wave's LDS accesses run in order)
    __shared__ __attribute__((aligned(16))) float p_buf[VCOL ? 1 : 2][kPage][G];
    // VCOL: a 2-stage ring of pages loaded straight from HBM (global_load_lds):
    // per stage the K tile, the V tile (16 rows of D codes each), then the K and
    // the V scales (256 bytes each, four copies of the page's 16).  After the page
    // loop the fused merge takes the ring for its weights.
    constexpr int kTile = kPage * D;
    constexpr int kStage = 2 * kTile + 512;
    constexpr int NDMA = 2 * (kTile / 1024) + 2;   // direct loads per page
    __shared__ __attribute__((aligned(16))) int8_t ring[VCOL ? 2 * kStage : 16];
    __shared__ float w_own[(FINAL || VCOL) ? 1 : kFusedMergeChunk];
    float* const w_lds = VCOL ? reinterpret_cast<float*>(ring) : w_own;

    const int lane = threadIdx.x;
    const int sub = lane % LPK;
    const int kg = lane / LPK;
    const int myhead = sub / HG;
    const int Hq = a.num_q_heads;
    const int Hkv = a.num_kv_heads;
    // 1-D grid, KV head fastest, then split, then sequence.  Workgroup i runs on
    // XCD i % 8, so every XCD gets the same share of every sequence whatever the
    // lengths; the KV heads of one page are read at about the same time, and a
    // sequence's splits are dispatched together.
    const int kvh = blockIdx.x % Hkv;
    const int sp = FINAL ? 0 : (blockIdx.x / Hkv) % a.max_splits;
    const int b = FINAL ? blockIdx.x / Hkv : blockIdx.x / (Hkv * a.max_splits);
    const int head0 = kvh * G;
    const int64_t row0 = (int64_t)b * Hq + head0;                // (b, head0)

    int len = __ldg(a.seq_lens + b);
    report(a.err, len < 0 || len > a.bt_stride * kPage ||
                      (!FINAL && sp == 0 && (int64_t)a.max_splits * a.split_keys < len),
           PFA_BOUNDS_SEQ_LEN);
    len = min(max(len, 0), a.bt_stride * kPage);
    int lo = a.window > 0 ? max(0, len - a.window) : 0;         // first visible key
    int hi = len;

    // Fused merge (counters given).  The partials go out as agent-scope atomic
    // stores, which write through to the point where all XCDs see them.  After
    // they complete (vmcnt 0), the split adds one to its (sequence, KV head)
    // counter; the split that brings it to the split count reads the row's
    // partials back with agent-scope atomic loads, merges them for its G heads,
    // writes out, and resets the counter.  No L2 write-back or invalidate is
    // needed (agent-scope fences would write back or invalidate a whole XCD's L2
    // for every workgroup), and no wave waits on another.
    const bool fused = !FINAL && a.counters != nullptr;
    auto put = [&](float* p, float v) __attribute__((always_inline)) {
        if (fused) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *p = v;
    };
    auto arrive = [&]() __attribute__((always_inline)) {
        if constexpr (!FINAL) {
            if (!fused) return;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            int32_t* ctr = a.counters + (int64_t)b * Hkv + kvh;
            int old = 0;
            if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __builtin_amdgcn_readfirstlane(old);
            const int nsp = min((len + a.split_keys - 1) / a.split_keys, a.max_splits);
            if (old != nsp - 1) return;
            asm volatile("" ::: "memory");
            for (int g = 0; g < G; ++g) {
                const int64_t r = row0 + g;
                merge_splits<D, kFusedMergeChunk, true>(a.lse_part + r * a.max_splits,
                                                        a.o_part + r * a.max_splits * D, nsp,
                                                        a.sinks ? a.sinks + head0 + g : nullptr, w_lds,
                                                        a.out + r * D);
            }
            if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    if constexpr (FINAL) {
        if (lo >= hi) {   // no keys: output 0
            for (int e = lane; e < G * D; e += kWave) a.out[row0 * D + e] = 0.0f;
            return;
        }
    } else {
        const int s0 = sp * a.split_keys;
        if (s0 >= len) return;
        if (s0 + a.split_keys <= lo) {   // the window hides the whole split
            if (lane < G) put(a.lse_part + (row0 + lane) * a.max_splits + sp, -INFINITY);
            arrive();
            return;
        }
        lo = max(lo, s0);
        hi = min(hi, s0 + a.split_keys);
    }

    const int p0 = lo / kPage, p1 = (hi - 1) / kPage;
    const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
    const int64_t head_stride = (int64_t)kPage * D;              // elements per page-head block
    const char* kbase = static_cast<const char*>(a.k_pool);
    const char* vbase = static_cast<const char*>(a.v_pool);
    const int lane_off = lane * 8 * EB;

    // a page's K/V (and INT8 scales) as this lane loads them
    // (VCOL: the page's ring stage instead)
    struct PageRegs {
        CT k[VCOL ? 1 : NLOAD], v[VCOL ? 1 : NLOAD];
        float ks[VCOL ? 1 : NLOAD], vs[VCOL ? 1 : NLOAD];
        const LDS3 int8_t* st;   // VCOL: the page's stage
    };
    // (stage addresses as LDS pointers, so that constant offsets fold into the reads)
    const LDS3 int8_t* const ring3 = (const LDS3 int8_t*)ring;
    auto lds_u32 = [](const LDS3 int8_t* x) __attribute__((always_inline)) { return (uint32_t)(uintptr_t)x; };
    // a page's block-table entry (a scalar load; the index is clamped to the
    // split's last page so that the read stays inside the row), read one page
    // ahead of the loads that use it
    auto page_id = [&](int p) __attribute__((always_inline)) { return __ldg(bt + min(p, p1)); };
    auto load_page = [&](int raw_id, PageRegs& r) __attribute__((always_inline)) {
        report(a.err, raw_id < 0 || raw_id >= a.num_pages, PFA_BOUNDS_PAGE);
        const int id = min(max(raw_id, 0), a.num_pages - 1);
        const int64_t blk = (int64_t)id * Hkv + kvh;
        if constexpr (VCOL) {
            // straight into the stage: the tiles as they lie in the pool, then the
            // scales (lane l loads the page's scale l % 16)
            const char* kt = kbase + blk * head_stride;
            const char* vt = vbase + blk * head_stride;
#pragma unroll
            for (int c = 0; c < kTile / 1024; ++c) {
                dma16(kt + 1024 * c, 16u * (uint32_t)lane, lds_u32(r.st + 1024 * c));
                dma16(vt + 1024 * c, 16u * (uint32_t)lane, lds_u32(r.st + kTile + 1024 * c));
            }
            dma4(a.k_scale + blk * kPage, 4u * (uint32_t)(lane % kPage), lds_u32(r.st + 2 * kTile));
            dma4(a.v_scale + blk * kPage, 4u * (uint32_t)(lane % kPage), lds_u32(r.st + 2 * kTile + 256));
        } else {
            const char* kp = kbase + blk * head_stride * EB + lane_off;
            const char* vp = vbase + blk * head_stride * EB + lane_off;
#pragma unroll
            for (int i = 0; i < NLOAD; ++i) {
                r.k[i] = *reinterpret_cast<const CT*>(kp + i * 512 * EB);
                r.v[i] = *reinterpret_cast<const CT*>(vp + i * 512 * EB);
            }
            if constexpr (INT8) {
#pragma unroll
                for (int i = 0; i < NLOAD; ++i) {
                    r.ks[i] = __ldg(a.k_scale + blk * kPage + i * KPL + kg);
                    r.vs[i] = __ldg(a.v_scale + blk * kPage + i * KPL + kg);
                }
            }
        }
    };

    // kScalarIds: two register sets (VCOL: two ring stages) take the pages in turn.
    // The first page's loads go out right after q's own loads, so the INT8 query
    // setup below runs while both are in flight.
    PageRegs ra, rb;
    ra.st = ring3;
    rb.st = ring3 + kStage;
    auto issue_first = [&]() __attribute__((always_inline)) {
        if constexpr (kScalarIds<G, INT8>) load_page(page_id(p0), ra);
    };

    // q: slot j holds head (j ^ myhead), dims sub*8 .. sub*8+7, as bf16 pairs.
    // INT8: q meets the fp16 key pairs in fp16.  Each head is first scaled by the
    // power of two 2^sh that brings its largest |q| into [2^14, 2^15); a bf16
    // element then converts exactly unless it is more than 2^28 below that
    // largest one (a subnormal in fp16), where the rounding is below the fp32
    // summation error of the dot.  The score is scaled back by 2^-sh.
    uint32_t q[G][4];
    float c2 = a.sm_scale * kLog2e;      // scores kept in log2 units
    float qbias = 0.0f;   // INT8: 1152 * sum_d q'[myhead][d]
    if constexpr (VCOL) {
        // The KPL key groups hold the same q elements.  Each converts G/KPL of
        // the heads, and the wave shares them through the ring's second
        // stage, which no page load writes before the page loop: per head and
        // lane its 4 fp16 pairs and its part of the head's element sum.
        constexpr int HPK = G / KPL;
        static_assert(HPK >= 1 && HPK * KPL == G, "heads per key group");
        static_assert(G * LPK * 16 + LPK * G * 4 <= kStage, "q staging in one stage");
        __shared__ uint32_t qmax[G];
        if (lane < G) qmax[lane] = 0u;
        uint32_t qc[HPK][4];
#pragma unroll
        for (int e = 0; e < HPK; ++e) {
            const uint4 v = *reinterpret_cast<const uint4*>(a.q + (row0 + kg * HPK + e) * D + sub * 8);
            qc[e][0] = v.x; qc[e][1] = v.y; qc[e][2] = v.z; qc[e][3] = v.w;
        }
        issue_first();   // (stage 0; the staging below uses stage 1)
        if (a.k_smooth) {   // keys stored smoothed (k / s): the query meets q * s (s a power of two: exact)
            const float4* sp = reinterpret_cast<const float4*>(a.k_smooth + sub * 8);
            const float4 s0 = __ldg(sp), s1 = __ldg(sp + 1);
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int e = 0; e < HPK; ++e)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    qc[e][w] = pack_bf16_rne(bf16_lo(qc[e][w]) * smooth_pow2(sv[2 * w]),
                                             bf16_hi(qc[e][w]) * smooth_pow2(sv[2 * w + 1]));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int e = 0; e < HPK; ++e) {
            uint32_t mx = 0u;   // bit patterns of |bf16| order as the values do
#pragma unroll
            for (int w = 0; w < 4; ++w) mx = max(mx, max(qc[e][w] & 0x7fffu, (qc[e][w] >> 16) & 0x7fffu));
            atomicMax(&qmax[kg * HPK + e], mx);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        LDS3 int8_t* const stage1 = (LDS3 int8_t*)ring + kStage;
        LDS3 u32x4* const qs = (LDS3 u32x4*)stage1;                       // [G][LPK]
        LDS3 float* const ts = (LDS3 float*)(stage1 + G * LPK * 16);       // [LPK][G]
#pragma unroll
        for (int e = 0; e < HPK; ++e) {
            const int h = kg * HPK + e;
            const int sh = min(141 - (int)(qmax[h] >> 7), 127);   // 14 - exponent of the max
            float t = 0.0f;
            u32x4 w4;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t x = pack_f16_rne(ldexpf(bf16_lo(qc[e][w]), sh), ldexpf(bf16_hi(qc[e][w]), sh));
                t += f16_lo(x) + f16_hi(x);
                w4[w] = x;
            }
            qs[h * LPK + sub] = w4;
            ts[sub * G + h] = t;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float part[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const u32x4 w4 = qs[(j ^ myhead) * LPK + sub];
            q[j][0] = w4.x; q[j][1] = w4.y; q[j][2] = w4.z; q[j][3] = w4.w;
            part[j] = ts[sub * G + (j ^ myhead)];
        }
        c2 = ldexpf(c2, -min(141 - (int)(qmax[myhead] >> 7), 127));
        qbias = kK8Offset * transpose_reduce<LPK, G>(part);
        // the staging reads are complete before the page loads write the stage
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint16_t* qp = a.q + (row0 + (j ^ myhead)) * D + sub * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(qp);
            q[j][0] = v.x; q[j][1] = v.y; q[j][2] = v.z; q[j][3] = v.w;
        }
        issue_first();
        if constexpr (INT8) {
            if (a.k_smooth) {   // keys stored smoothed (k / s): the query meets q * s (s a power of two: exact)
                const float4* sp = reinterpret_cast<const float4*>(a.k_smooth + sub * 8);
                const float4 s0 = __ldg(sp), s1 = __ldg(sp + 1);
                const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        q[j][w] = pack_bf16_rne(bf16_lo(q[j][w]) * smooth_pow2(sv[2 * w]),
                                                bf16_hi(q[j][w]) * smooth_pow2(sv[2 * w + 1]));
            }
        }
        if constexpr (INT8) {
            __shared__ uint32_t qmax[G];
            if (lane < G) qmax[lane] = 0u;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int j = 0; j < G; ++j) {
                uint32_t mx = 0u;   // bit patterns of |bf16| order as the values do
#pragma unroll
                for (int w = 0; w < 4; ++w) mx = max(mx, max(q[j][w] & 0x7fffu, (q[j][w] >> 16) & 0x7fffu));
                atomicMax(&qmax[j ^ myhead], mx);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float part[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int sh = min(141 - (int)(qmax[j ^ myhead] >> 7), 127);   // 14 - exponent of the max
                float t = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    q[j][w] = pack_f16_rne(ldexpf(bf16_lo(q[j][w]), sh), ldexpf(bf16_hi(q[j][w]), sh));
                    t += f16_lo(q[j][w]) + f16_hi(q[j][w]);
                }
                part[j] = t;
                if (j == 0) c2 = ldexpf(c2, -sh);   // slot 0 is this lane's own head
            }
            qbias = kK8Offset * transpose_reduce<LPK, G>(part);
        }
    }

    float o[G][OJ];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < OJ; ++j) o[g][j] = 0.0f;
    // VCOL: this lane's byte offset into a stage's V tile for the transposed reads.
    // Lane j of a 16-lane group points at row j/2 of an 8-row block in key-pair
    // order: pair m = j/4 (+4 per block), member (j/2) % 2, which is pool row
    // m % KPL + KPL * (2 * (m / KPL) + member); the next block is kTrStep on.
    const int tr_j = lane % 16, tr_m = tr_j / 4, tr_t = (tr_j / 2) % 2;
    const int tr_off = (tr_m % KPL + KPL * (2 * (tr_m / KPL) + tr_t)) * D + 16 * (lane / 16) + 8 * (tr_j % 2);
    constexpr int kTrStep = (KPL == 4 ? 8 : 4) * D;
    float m_run = -INFINITY;   // running max (log2 units) of this lane's head
    float l_run = 0.0f;        // this lane's share of sum 2^(s - m_run) (its keys, its head)
    // VCOL: a weight enters the p.v dot2 as fp16 w = p * vs * 2^-vexp (vs the key's
    // value scale).  vexp is wave-uniform and only rises: whenever a value scale
    // exceeds vlim = 2^(vexp + 7), vexp moves to 4 above the exponent of the page's
    // largest scale and o and wsum are rescaled by the power of two, so w <= 2^8 *
    // 2^7 always fits fp16.  Scales far below the largest lose fp16 precision:
    // a weight below 2^-14 keeps an absolute error of at most 2^-25, which bounds
    // the output's error by about 2^-16 times the split's largest value scale.
    int vexp = -1000;
    float vlim = 0.0f;
    float wsum = 0.0f;   // VCOL: sum of this lane's head's rounded weights (its key groups)

    int pb = 0;
    // one page: scores, lazy rescale, weights, p.v
    auto page = [&](int p, PageRegs& r) __attribute__((always_inline)) {
        const int kpos0 = p * kPage;
        if constexpr (VCOL) {
            // this page's stage has landed once at most the next page's direct loads
            // (issued before this page whenever p < p1) are in flight; the memory
            // clobber keeps the stage's LDS reads below the wait
            if (!kDecodeAudit && p < p1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }

        // ---- scores ----
        float s[NS];
        bool valid[NLOAD];   // BF16
        float vsl[NS];       // INT8: the value scales (VCOL: from the stage)
        // the load group of score i (JOINT: lane t = sub % 2 of a head pair holds
        // load groups 2i + t)
        auto group_of = [&](int i) __attribute__((always_inline)) { return JOINT ? 2 * i + (sub & 1) : i; };
        auto outside = [&](int i) __attribute__((always_inline)) {
            const int key = kpos0 + group_of(i) * KPL + kg;
            return key < lo || key >= hi;
        };
        if constexpr (JOINT) {
            // load groups (2i, 2i+1) in one butterfly over 2G sums: slot 2a + b holds
            // head (a ^ myhead) on group 2i + (b ^ t), so the lanes end on
            // (head sub / 2, group 2i + sub % 2)
            const int own = (sub & 1) * KPL * D, oth = KPL * D - own;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const LDS3 int8_t* kr = r.st + (2 * i * KPL + kg) * D + sub * 8;
                const u32x2 wa = *(const LDS3 u32x2*)(kr + own);
                const u32x2 wb = *(const LDS3 u32x2*)(kr + oth);
                uint32_t ka[4], kb[4];
                k_pairs(make_uint2(wa.x, wa.y), ka);
                k_pairs(make_uint2(wb.x, wb.y), kb);
                float acc[2 * G];
#pragma unroll
                for (int a2 = 0; a2 < G; ++a2) {
                    float ta, tb;
                    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(ta) : "v"(q[a2][0]), "v"(ka[0]));
                    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(tb) : "v"(q[a2][0]), "v"(kb[0]));
#pragma unroll
                    for (int w = 1; w < 4; ++w) {
                        ta = __builtin_amdgcn_fdot2(as_f16x2(q[a2][w]), as_f16x2(ka[w]), ta, false);
                        tb = __builtin_amdgcn_fdot2(as_f16x2(q[a2][w]), as_f16x2(kb[w]), tb, false);
                    }
                    acc[2 * a2] = ta;
                    acc[2 * a2 + 1] = tb;
                }
                const float dot = transpose_reduce<LPK, 2 * G>(acc) - qbias;
                const int key = group_of(i) * KPL + kg;
                const float ksv = *(const LDS3 float*)(r.st + 2 * kTile + 4 * key);
                vsl[i] = *(const LDS3 float*)(r.st + 2 * kTile + 256 + 4 * key);
                s[i] = dot * (c2 * ksv);
            }
        }
#pragma unroll
        for (int i = 0; i < (JOINT ? 0 : NLOAD); ++i) {
            uint32_t kp[4];
            if constexpr (VCOL) {
                const u32x2 w = *(const LDS3 u32x2*)(r.st + (i * KPL + kg) * D + sub * 8);
                k_pairs(make_uint2(w.x, w.y), kp);
            } else {
                k_pairs(r.k[i], kp);
            }
            float acc[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float t = 0.0f;
                if constexpr (INT8) {
                    // the chain's first product in the three-operand form with a zero
                    // addend (the compiler otherwise zeroes a register and accumulates
                    // in place: one more VALU op per head and key)
                    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(t) : "v"(q[j][0]), "v"(kp[0]));
#pragma unroll
                    for (int w = 1; w < 4; ++w)
                        t = __builtin_amdgcn_fdot2(as_f16x2(q[j][w]), as_f16x2(kp[w]), t, false);
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[j][w]), as_bf16x2(kp[w]), t, false);
                }
                acc[j] = t;
            }
            float dot = transpose_reduce<LPK, G>(acc);
            if constexpr (INT8) dot -= qbias;
            float ksv = 0.0f;
            if constexpr (VCOL) {
                ksv = *(const LDS3 float*)(r.st + 2 * kTile + 4 * (i * KPL + kg));
                vsl[i] = *(const LDS3 float*)(r.st + 2 * kTile + 256 + 4 * (i * KPL + kg));
            } else if constexpr (INT8) {
                ksv = r.ks[i];
                vsl[i] = r.vs[i];
            }
            const float sc = INT8 ? c2 * ksv : c2;
            if constexpr (INT8) {
                s[i] = dot * sc;
            } else {
                const int key = kpos0 + i * KPL + kg;
                valid[i] = key >= lo && key < hi;
                s[i] = valid[i] ? dot * sc : -INFINITY;
            }
        }
        // INT8 (VALU-bound) masks only the pages that cross [lo, hi), a split's first
        // and last at most: the scores of keys outside become -inf by a select, never
        // by arithmetic, since their scales may be poison, and their value scales
        // become 0 (the weight is then 0, not 0 * NaN).
        if constexpr (INT8) {
            if (!(kpos0 >= lo && kpos0 + kPage <= hi)) {
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const bool out = outside(i);
                    s[i] = out ? -INFINITY : s[i];
                    vsl[i] = out ? 0.0f : vsl[i];
                }
            }
        }
        if constexpr (VCOL) {
            bool big = false;
#pragma unroll
            for (int i = 0; i < NS; ++i) big |= vsl[i] > vlim;
            if (__any(big)) {   // the first page with a non-zero scale, then rarely
                float vm = vsl[0];
#pragma unroll
                for (int i = 1; i < NS; ++i) vm = fmaxf(vm, vsl[i]);
                vm = stride_max<1>(vm);                                       // > 0 here
                const int en = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(vm)) - 3;
                const float f = ldexpf(1.0f, vexp - en);                       // 0 the first time
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int j = 0; j < OJ; ++j) o[g][j] *= f;
                wsum *= f;
                vexp = en;
                vlim = ldexpf(1.0f, en + 7);
            }
        }
        // ---- running max, lazy rescale with headroom: the reference max moves only
        // when a head's max exceeds it by more than 8, so every weight is <= 2^8
        // (no overflow in fp32 or bf16) and the rescale, G*8 multiplies, runs on
        // few pages.  o and l share the reference, so o/l and m + log2(l) hold. ----
        auto rescale = [&](float m_new) __attribute__((always_inline)) {
            const float alpha = fast_exp2(m_run - m_new);   // 0 on the first page
            l_run *= alpha;
            if constexpr (VCOL) wsum *= alpha;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float ag = lane_read(alpha, g * HG);
#pragma unroll
                for (int j = 0; j < OJ; ++j) o[g][j] *= ag;
            }
            m_run = m_new;
        };
        if constexpr (JOINT && NS == 2) {
            // VALU-bound: a page whose scores all stay within the headroom needs no
            // max at all, so each lane only compares its own scores with its head's
            // threshold m_run + 8; the maxima (without fmaxf's input quieting
            // moves, the head pair's lanes first) are taken when one is above it
            if (__any(s[0] > m_run + 8.0f || s[1] > m_run + 8.0f)) {
                float pm = vmax(s[0], s[1]);
                pm = xor32_vmax(xor16_vmax(vmax(pm, dpp_xor<1>(pm))));
                rescale(vmax(m_run, pm));
            }
        } else {
            float pm = s[0];
#pragma unroll
            for (int i = 1; i < NLOAD; ++i) pm = fmaxf(pm, s[i]);
            pm = stride_max<LPK>(pm);
            const float m_new = fmaxf(m_run, pm);
            if (__any(m_new > m_run + 8.0f)) rescale(m_new);
        }
        // ---- weights, shared within the wave (masked keys weigh 0) ----
        if constexpr (!PAIRED) {
#pragma unroll
            for (int i = 0; i < NLOAD; ++i) {
                const float pw = fast_exp2(s[i] - m_run);      // 0 for masked keys
                l_run += pw;
                float pv = pw;
                if constexpr (INT8) pv = pw * vsl[i];
                if (sub % HG == 0) p_buf[pb][i * KPL + kg][myhead] = pv;
            }
        } else {
            // the weights of keys (i, i+1) as one pair (BF16: bf16; INT8: fp16 scaled by
            // 2^-vexp), at [i/2][kg][head]
            uint32_t* pp_buf = reinterpret_cast<uint32_t*>(&p_buf[pb][0][0]);
            if constexpr (JOINT) {
                // lane t weighs group 2i + t; lane 0 of the pair packs both
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const float pw = fast_exp2(s[i] - m_run);
                    l_run += pw;
                    const float pv = pw * ldexpf(vsl[i], -vexp);
                    const uint32_t pr = pack_f16_rne(pv, dpp_xor<1>(pv));
                    wsum = __builtin_amdgcn_fdot2(as_f16x2(pr), as_f16x2(0x3C003C00u), wsum, false);
                    if (sub % HG == 0) pp_buf[(i * KPL + kg) * G + myhead] = pr;
                }
            }
#pragma unroll
            for (int i = 0; i < (JOINT ? 0 : NLOAD); i += 2) {
                const float p0 = fast_exp2(s[i] - m_run), p1 = fast_exp2(s[i + 1] - m_run);
                uint32_t pr;
                if constexpr (VCOL) {   // (every paired INT8 build)
                    l_run += p0 + p1;
                    pr = pack_f16_rne(p0 * ldexpf(vsl[i], -vexp), p1 * ldexpf(vsl[i + 1], -vexp));
                    wsum = __builtin_amdgcn_fdot2(as_f16x2(pr), as_f16x2(0x3C003C00u), wsum, false);
                } else {
                    pr = pack_bf16_rne(p0, p1);
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pr), as_bf16x2(0x3F803F80u), l_run, false);
                }
                if (sub % HG == 0) pp_buf[((i / 2) * KPL + kg) * G + myhead] = pr;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- p.v ----
        if constexpr (VCOL) {
            // pair m's G weight pairs from LDS (the same words for every lane), read
            // one pair ahead; the lane's columns from the V tile, 8 rows (4 pairs)
            // per transposed read.  Each read's address passes through an empty asm
            // that also takes the last result of the pair before, so the compiler
            // cannot hoist every pair's reads (64 registers) to the top.
            const uint32_t pp_base = (uint32_t)(uintptr_t)(const LDS3 void*)&p_buf[pb][0][0];
            const LDS3 int8_t* vt = r.st + kTile + tr_off;
            auto read_pp = [&](uint32_t addr, uint32_t (&pp)[G]) __attribute__((always_inline)) {
#pragma unroll
                for (int q4 = 0; q4 < G / 4; ++q4) {
                    const u32x4 w = *(const LDS3 u32x4*)(uintptr_t)(addr + 16 * q4);
                    pp[4 * q4] = w.x; pp[4 * q4 + 1] = w.y; pp[4 * q4 + 2] = w.z; pp[4 * q4 + 3] = w.w;
                }
            };
            i32x2 raw[2][NC];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    raw[h][c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS3 i32x2*)(vt + h * kTrStep + 64 * c));
            uint32_t ppc[G], ppn[G], pp_b = pp_base;
            read_pp(pp_b, ppc);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t vv[NC][4];
#pragma unroll
                for (int c = 0; c < NC; ++c) k_pairs(make_uint2((uint32_t)raw[h][c].x, (uint32_t)raw[h][c].y), vv[c]);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int m = 4 * h + u;
                    if (m + 1 < 8) {
                        order_after(pp_b, o);
                        read_pp(pp_b + (m + 1) * G * 4, ppn);
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int c = 0; c < NC; ++c)
                            o[g][c] = __builtin_amdgcn_fdot2(as_f16x2(ppc[g]), as_f16x2(vv[c][u]), o[g][c], false);
#pragma unroll
                    for (int g = 0; g < G; ++g) ppc[g] = ppn[g];
                }
            }
        } else {
            CT vcur[NLOAD];
#pragma unroll
            for (int i = 0; i < NLOAD; ++i) vcur[i] = r.v[i];
            if constexpr (!INT8) {
                // BF16 values past the sequence end may be poison: zero them (weight 0 *
                // NaN), on the pages that cross [lo, hi) only
                if (!(kpos0 >= lo && kpos0 + kPage <= hi)) {
#pragma unroll
                    for (int i = 0; i < NLOAD; ++i)
                        if (!valid[i]) vcur[i] = CT{};
                }
            }
            if constexpr (!PAIRED) {
#pragma unroll
                for (int i = 0; i < NLOAD; ++i) {
                    float pw[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) pw[g] = p_buf[pb][i * KPL + kg][g];
                    float x[8];
                    v_floats(vcur[i], x);
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pw[g], x[j], o[g][j]);
                }
            } else {
                const uint4* pp4 = reinterpret_cast<const uint4*>(&p_buf[pb][0][0]);
#pragma unroll
                for (int i = 0; i < NLOAD; i += 2) {
                    uint32_t vv[8];
                    v_pairs(vcur[i], vcur[i + 1], vv);
                    // the G weight pairs of keys (i, i+1) of this key group
                    uint32_t pp[G];
#pragma unroll
                    for (int q4 = 0; q4 < G / 4; ++q4) {
                        const uint4 w = pp4[((i / 2) * KPL + kg) * (G / 4) + q4];
                        pp[4 * q4] = w.x; pp[4 * q4 + 1] = w.y; pp[4 * q4 + 2] = w.z; pp[4 * q4 + 3] = w.w;
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            o[g][j] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp[g]), as_bf16x2(vv[j]), o[g][j], false);
                }
            }
        }
        if constexpr (!VCOL) pb ^= 1;
    };
    // page p is consumed from one register set while page p+1 loads into the other
    if constexpr (kScalarIds<G, INT8>) {
        // two sets used in turn (a copy from one to the other would cost a move per
        // register and page)
        int nid = page_id(p0 + 1);
        int p = p0;
        for (; p < p1; p += 2) {
            load_page(nid, rb);
            nid = page_id(p + 2);
            page(p, ra);
            if (p + 1 < p1) {
                load_page(nid, ra);
                nid = page_id(p + 3);
            }
            page(p + 1, rb);
        }
        if (p == p1) page(p, ra);
    } else {
        PageRegs rn;
        const int32_t* vbt = a.block_table + (int64_t)b * a.bt_stride;
        load_page(__ldg(vbt + p0), rn);
        for (int p = p0; p <= p1; ++p) {
            PageRegs rc = rn;
            if (p < p1) load_page(__ldg(vbt + p + 1), rn);
            page(p, rc);
        }
    }

    // ---- reduce across key groups (VCOL: each lane's columns are complete); head
    // g's row is written by the lanes of key group g % KPL, or VCOL by all lanes ----
    if constexpr (!VCOL) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < 8; ++j) o[g][j] = stride_sum<LPK>(o[g][j]);
    }
    // (JOINT: the two lanes of a head summed different keys)
    const float l_tot = stride_sum<LPK>(JOINT ? l_run + dpp_xor<1>(l_run) : l_run);
    const float w_tot = VCOL ? stride_sum<LPK>(wsum) : 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mg = lane_read(m_run, g * HG);
        const float lg = lane_read(l_tot, g * HG);
        float den = lg;
        if constexpr (FINAL) {
            if (a.sinks) den += fast_exp2(__ldg(a.sinks + head0 + g) * kLog2e - mg);
        }
        const float f = (FINAL && !(den > 0.0f)) ? 0.0f : 1.0f / den;
        float* row = FINAL ? a.out + (row0 + g) * D : a.o_part + ((row0 + g) * a.max_splits + sp) * D;
        if constexpr (VCOL) {
            // the offset out (1152 per unit of weight), then the scale 2^vexp back
            const float wg = lane_read(w_tot, g * HG);
#pragma unroll
            for (int c = 0; c < NC; ++c) put(row + 64 * c + lane, ldexpf(fmaf(-kK8Offset, wg, o[g][c]) * f, vexp));
        } else if (g % KPL == kg) {
            float* dst = row + sub * 8;
            if (fused) {
#pragma unroll
                for (int j = 0; j < 8; ++j) put(dst + j, o[g][j] * f);
            } else {
                float4* d4 = reinterpret_cast<float4*>(dst);
                d4[0] = make_float4(o[g][0] * f, o[g][1] * f, o[g][2] * f, o[g][3] * f);
                d4[1] = make_float4(o[g][4] * f, o[g][5] * f, o[g][6] * f, o[g][7] * f);
            }
        }
        if constexpr (!FINAL) {
            if (lane == 0) put(a.lse_part + (row0 + g) * a.max_splits + sp, (mg + fast_log2(lg)) * kLn2);
        }
    }
    arrive();
}

template <int D, int G, bool INT8>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t s) {
    const int rows = a.num_kv_heads * a.batch;
    if (a.max_splits == 1)
        hipLaunchKernelGGL((decode_kernel<D, G, INT8, true>), dim3(rows), dim3(kWave), 0, s, a, a.block_table);
    else
        hipLaunchKernelGGL((decode_kernel<D, G, INT8, false>), dim3(a.max_splits * rows), dim3(kWave), 0, s, a,
                           a.block_table);
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

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
// MI355X design.  The kernel is HBM-bound, and each K/V element is used by exactly
// one lane group, so K/V go straight from HBM to registers.  (INT8 at G = 8 runs
// its two products on the matrix cores instead: decode_mfma.hip.)
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
//    for every element within 2^28 of the head's largest).  With key smoothing
//    (keys stored as k/s per channel, the "INT8 KV cache" section's smoothing by
//    the key norm's weight, s taken as a power of two), q is first scaled by s,
//    which is exact too.
//    A lane's partial dots for the G heads go through a transposed butterfly over
//    the LPK lanes, on DPP moves only (group_reduce.h).  Slot j of a lane holds
//    head (j ^ myhead), so each stage adds a partner's slots to its own lower half
//    with no selects, and ends with the lane holding its own head's full score.
//  * The softmax max is taken per page and the rescale is lazy with headroom: o
//    and l are rescaled only when some head's max exceeds the reference max by
//    more than 8 (log2 units), so weights stay <= 2^8.  At G = 8 a rescale on
//    every growth ran on most of a split's first pages (INT8 at batch 8 x 32768:
//    92 -> 85 us).  The weights p are shared within the wave through LDS.
//  * p.v: for G <= 4, fp32 FMAs on the lane's 8 elements for all G heads.  For
//    BF16 at G = 8, the VALU budget forces dot2 on key pairs from two loads: the
//    lane that computes a head's weights for two keys rounds them to a bf16 pair
//    once (nearest even) and shares the pair through LDS; the (v_a, v_b) pairs
//    are built by v_perm, and l sums the same rounded weights (a dot2 with
//    (1, 1)), so numerator and denominator agree.
//  * At the end of a split each wave reduces its partial o across key groups and
//    writes o/l with lse = ln(sum e^s) (split mode), or the final output with the
//    sink (unsplit mode).
#include "group_reduce.h"
#include "merge_splits.h"

namespace pfa {
namespace {

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

// Element pairs (a[d], b[d]) of two keys' bf16 chunks, d = 0..7 (paired p.v), by
// byte permute.
__device__ __forceinline__ void v_pairs(const uint4& a, const uint4& b, uint32_t (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __builtin_amdgcn_perm(dw(b, i), dw(a, i), 0x05040100u);
        v[2 * i + 1] = __builtin_amdgcn_perm(dw(b, i), dw(a, i), 0x07060302u);
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
    constexpr bool PAIRED = G >= 8;            // p.v by dot2 on key pairs (BF16)
    static_assert(G <= LPK, "group size");
    static_assert(!(INT8 && PAIRED), "INT8 at G = 8 runs on the matrix cores");
    static_assert(!PAIRED || NLOAD % 2 == 0, "key pairs");
    typedef typename Chunk<INT8>::T CT;

    // weights of a page, double-buffered: [key][head] floats (G <= 4), or for
    // G = 8 [key pair][key group][head] bf16 pairs
    __shared__ __attribute__((aligned(16))) float p_buf[2][kPage][G];
    __shared__ float w_lds[FINAL ? 1 : kFusedMergeChunk];

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
    struct PageRegs {
        CT k[NLOAD], v[NLOAD];
        float ks[NLOAD], vs[NLOAD];
    };
    // a page's block-table entry (a scalar load; the index is clamped to the
    // split's last page so that the read stays inside the row), read one page
    // ahead of the loads that use it
    auto page_id = [&](int p) __attribute__((always_inline)) { return __ldg(bt + min(p, p1)); };
    auto load_page = [&](int raw_id, PageRegs& r) __attribute__((always_inline)) {
        report(a.err, raw_id < 0 || raw_id >= a.num_pages, PFA_BOUNDS_PAGE);
        const int id = min(max(raw_id, 0), a.num_pages - 1);
        const int64_t blk = (int64_t)id * Hkv + kvh;
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
    };

    // kScalarIds: two register sets take the pages in turn.  The first page's loads
    // go out right after q's own loads, so the INT8 query setup below runs while
    // both are in flight.
    PageRegs ra, rb;
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
    {
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

    float o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = 0.0f;
    float m_run = -INFINITY;   // running max (log2 units) of this lane's head
    float l_run = 0.0f;        // this lane's share of sum 2^(s - m_run) (its keys, its head)
    int pb = 0;
    // one page: scores, lazy rescale, weights, p.v
    auto page = [&](int p, PageRegs& r) __attribute__((always_inline)) {
        const int kpos0 = p * kPage;
        // ---- scores ----
        float s[NLOAD];
        bool valid[NLOAD];   // BF16
        float vsl[NLOAD];    // INT8: the value scales
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            uint32_t kp[4];
            k_pairs(r.k[i], kp);
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
            if constexpr (INT8) {
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
                for (int i = 0; i < NLOAD; ++i) {
                    const int key = kpos0 + i * KPL + kg;
                    const bool out = key < lo || key >= hi;
                    s[i] = out ? -INFINITY : s[i];
                    vsl[i] = out ? 0.0f : vsl[i];
                }
            }
        }
        // ---- running max, lazy rescale with headroom: the reference max moves only
        // when a head's max exceeds it by more than 8, so every weight is <= 2^8
        // (no overflow in fp32 or bf16) and the rescale, G*8 multiplies, runs on
        // few pages.  o and l share the reference, so o/l and m + log2(l) hold. ----
        auto rescale = [&](float m_new) __attribute__((always_inline)) {
            const float alpha = fast_exp2(m_run - m_new);   // 0 on the first page
            l_run *= alpha;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float ag = lane_read(alpha, g * HG);
#pragma unroll
                for (int j = 0; j < 8; ++j) o[g][j] *= ag;
            }
            m_run = m_new;
        };
        {
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
            // the weights of keys (i, i+1) as one bf16 pair, at [i/2][kg][head]
            uint32_t* pp_buf = reinterpret_cast<uint32_t*>(&p_buf[pb][0][0]);
#pragma unroll
            for (int i = 0; i < NLOAD; i += 2) {
                const float p0 = fast_exp2(s[i] - m_run), p1 = fast_exp2(s[i + 1] - m_run);
                const uint32_t pr = pack_bf16_rne(p0, p1);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pr), as_bf16x2(0x3F803F80u), l_run, false);
                if (sub % HG == 0) pp_buf[((i / 2) * KPL + kg) * G + myhead] = pr;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- p.v ----
        {
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
        pb ^= 1;
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

    // ---- reduce across key groups; head g's row is written by the lanes of key
    // group g % KPL ----
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = stride_sum<LPK>(o[g][j]);
    const float l_tot = stride_sum<LPK>(l_run);
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
        if (g % KPL == kg) {
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
        case 8:   // INT8 at G = 8: on the matrix cores
            if constexpr (INT8) return launch_decode_int8_mfma(a, D, s);
            else return launch_dg<D, 8, false>(a, s);
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

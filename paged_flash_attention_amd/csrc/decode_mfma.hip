// INT8 split-KV decode at G = 8 query heads per KV head, on the matrix cores.
//
// What is computed is the decode of the TileInfer.jl performance page ("Fused
// kernels, FlashAttention and PagedAttention": online softmax over the pages in
// place, keys split across waves, a separate combine) over its INT8 cache ("INT8
// KV cache": one fp32 scale per cached vector).  The per-page work of a KV head is
// a dense product: the G = 8 queries of the group against the page's 16 keys
// (8 x D by D x 16), then the 16 weights of each query against the page's values
// (8 x 16 by 16 x D).  On the vector ALU that is 2*G*D/2 dot2 lane-ops per key,
// which bounds the VALU version by issue rate, not by HBM.  Here both products
// run as fp16 MFMAs with fp32 accumulation; the G = 8 heads fill half of the 16
// columns and the other half carries zeros.
//
//  * One wave per (split, KV head, sequence), the same 1-D grid as the other decode
//    kernels (KV head fastest, then split, then sequence).  The pages of a split go
//    straight from HBM into a 2-stage LDS ring (global_load_lds): per stage the K
//    tile and the V tile (16 rows of D codes), then the page's 16 K and 16 V scales
//    (four copies each).  Rows are stored with their 16-byte slots swizzled (slot
//    s of key k at s ^ (k % (D/16))), so that the 16 keys' reads of one slot, and
//    the transposed reads of 8 keys' column blocks, spread over the banks.
//  * Codes enter the products as fp16 1152 + c: the byte u = c + 128 is the low
//    byte of the fp16 word 0x64uu = 1024 + u, one byte permute per two codes.
//    q is scaled per head by the power of two that brings its largest element into
//    [2^14, 2^15) and converted to fp16 (exact unless an element is more than 2^28
//    below the largest), and 1152 times the head's element sum enters the q.k
//    accumulator as its initial value, negated.  With key smoothing (keys stored
//    as k / s, s a power of two per channel) q is first scaled by s, exactly.
//  * q.k: S^T = K q^T with v_mfma_f32_16x16x32_f16, D/32 per page.  Lane l holds
//    key l % 16 of the K operand (8 codes of one 16-byte slot) and head l % 16 of
//    q; the result leaves lane l with head l % 16's scores of keys 4(l/16)..+3.
//  * softmax: running max per head in log2 units, with the lazy rescale of the
//    other decode kernels (o and l move only when a score exceeds the reference
//    max by more than 8, so weights stay <= 2^8); lanes compare their own scores
//    with the threshold and the max is reduced over the head's four lanes only
//    when one passes.
//  * p.v: O^T += V^T W with v_mfma_f32_16x16x16f16, one per 16 columns.  The
//    scores' layout is already the weight operand's: lane l's four keys, head
//    l % 16.  The weight is w = p * scale_v * 2^-vexp in fp16 (nearest even):
//    vexp is wave-uniform and only rises, so that w stays below 2^15 (below).
//    The V operand is 4 codes of one column for 4 keys, read with ds_read_b64_tr_b8,
//    which hands each lane one column of an 8-row block: rows 0..3 are the lane
//    group's keys at one 16-column block, rows 4..7 the same keys at the next, so
//    one read feeds two MFMAs.  1152 times the sum of the rounded weights is
//    subtracted at the end, and the scale 2^vexp restored.
//  * The output O^T leaves lane l with head l % 16's columns 16m + 4(l/16)..+3:
//    each wave writes its G rows (o/l and the lse per split, or the final row
//    with the sink when unsplit), and in the fused mode merges like the other
//    decode kernels.
#include "merge_splits.h"

#ifndef PFA_DECODE_AUDIT
#define PFA_DECODE_AUDIT 0
#endif

namespace pfa {
namespace {

constexpr bool kAudit = PFA_DECODE_AUDIT != 0;
constexpr int kG = 8;                  // query heads per KV head
constexpr int kMergeChunk = 256;       // fused merge: split weights in LDS at a time
constexpr float kCodeOffset = 1152.0f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS3 __attribute__((address_space(3)))

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).x; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).y; }
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
// Four INT8 codes (one dword) -> two fp16 pairs 1152 + c, in order.
__device__ __forceinline__ u32x2 codes_f16(uint32_t w) {
    const uint32_t u = w ^ 0x80808080u;
    u32x2 r;
    r[0] = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    return r;
}
// Unsigned max over lanes i, i ^ 16 and i ^ 32, i ^ 48.
__device__ __forceinline__ uint32_t head_umax(uint32_t x) {
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max(r[0], r[1]);
}

template <int D, bool FINAL>
__global__ __launch_bounds__(kWave, 4)
void decode_int8_mfma_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
    constexpr int SL = D / 16;               // 16-byte slots per row
    constexpr int NQK = D / 32;              // q.k MFMAs per page
    constexpr int NMB = D / 16;              // p.v MFMAs per page (16 columns each)
    constexpr int kTile = kPage * D;         // bytes of a K or V page-head block
    constexpr int kStage = 2 * kTile + 512;
    constexpr int NDMA = 2 * (kTile / 1024) + 2;   // direct loads per page
    static_assert(kTile % 1024 == 0 && (1024 / D) % SL == 0, "swizzle repeats every 1024 bytes");
    static_assert(2 * kStage >= kMergeChunk * 4, "merge weights in the ring");
    __shared__ __attribute__((aligned(16))) int8_t ring[2 * kStage];

    const int lane = threadIdx.x;
    const int hl = lane % 16;     // head column; key row of the K operand; column of the V operand
    const int grp = lane / 16;    // this lane's keys: 4 grp .. 4 grp + 3
    const int Hq = a.num_q_heads;
    const int Hkv = a.num_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int sp = FINAL ? 0 : (blockIdx.x / Hkv) % a.max_splits;
    const int b = FINAL ? blockIdx.x / Hkv : blockIdx.x / (Hkv * a.max_splits);
    const int head0 = kvh * kG;
    const int64_t row0 = (int64_t)b * Hq + head0;
    const bool hv = hl < kG;      // a real head (columns 8..15 carry zeros)

    int len = __ldg(a.seq_lens + b);
    report(a.err, len < 0 || len > a.bt_stride * kPage ||
                      (!FINAL && sp == 0 && (int64_t)a.max_splits * a.split_keys < len),
           PFA_BOUNDS_SEQ_LEN);
    len = min(max(len, 0), a.bt_stride * kPage);
    int lo = a.window > 0 ? max(0, len - a.window) : 0;
    int hi = len;

    // Fused merge, as in the other decode kernels: partials out as agent-scope
    // atomic stores, then (vmcnt 0) one arrival on the (sequence, KV head) counter;
    // the last split merges the row's partials and resets the counter.
    const bool fused = !FINAL && a.counters != nullptr;
    float* const w_lds = reinterpret_cast<float*>(ring);
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
            for (int g = 0; g < kG; ++g) {
                const int64_t r = row0 + g;
                merge_splits<D, kMergeChunk, true>(a.lse_part + r * a.max_splits, a.o_part + r * a.max_splits * D,
                                                   nsp, a.sinks ? a.sinks + head0 + g : nullptr, w_lds,
                                                   a.out + r * D);
            }
            if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    if constexpr (FINAL) {
        if (lo >= hi) {
            for (int e = lane; e < kG * D; e += kWave) a.out[row0 * D + e] = 0.0f;
            return;
        }
    } else {
        const int s0 = sp * a.split_keys;
        if (s0 >= len) return;
        if (s0 + a.split_keys <= lo) {   // the window hides the whole split
            if (lane < kG) put(a.lse_part + (row0 + lane) * a.max_splits + sp, -INFINITY);
            arrive();
            return;
        }
        lo = max(lo, s0);
        hi = min(hi, s0 + a.split_keys);
    }

    const int p0 = lo / kPage, p1 = (hi - 1) / kPage;
    const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
    const char* kbase = static_cast<const char*>(a.k_pool);
    const char* vbase = static_cast<const char*>(a.v_pool);
    const LDS3 int8_t* const ring3 = (const LDS3 int8_t*)ring;
    auto lds_u32 = [](const LDS3 int8_t* x) __attribute__((always_inline)) { return (uint32_t)(uintptr_t)x; };

    // Direct loads: lane l's 16 bytes land at 1024c + 16l of the tile, which is
    // key k = (1024c + 16l) / D, stored slot t = l % SL; they come from the key's
    // slot t ^ (k % SL).  (1024 bytes hold a whole number of SL-row periods, so
    // the offset is the same for every c.)
    const int dkey = (16 * lane) / D;
    const uint32_t dsrc = (uint32_t)(dkey * D + 16 * ((lane % SL) ^ (dkey % SL)));
    auto page_id = [&](int p) __attribute__((always_inline)) { return __ldg(bt + min(p, p1)); };
    auto load_page = [&](int raw_id, const LDS3 int8_t* st) __attribute__((always_inline)) {
        report(a.err, raw_id < 0 || raw_id >= a.num_pages, PFA_BOUNDS_PAGE);
        const int id = min(max(raw_id, 0), a.num_pages - 1);
        const int64_t blk = (int64_t)id * Hkv + kvh;
        const char* kt = kbase + blk * kTile;
        const char* vt = vbase + blk * kTile;
        // the stage's previous reads have completed before the loads can write it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < kTile / 1024; ++c) {
            dma16(kt + 1024 * c, dsrc, lds_u32(st + 1024 * c));
            dma16(vt + 1024 * c, dsrc, lds_u32(st + kTile + 1024 * c));
        }
        dma4(a.k_scale + blk * kPage, 4u * (uint32_t)(lane % kPage), lds_u32(st + 2 * kTile));
        dma4(a.v_scale + blk * kPage, 4u * (uint32_t)(lane % kPage), lds_u32(st + 2 * kTile + 256));
    };
    const LDS3 int8_t* const st0 = ring3;
    const LDS3 int8_t* const st1 = ring3 + kStage;

    // ---- q: the B operand of q.k, head hl, dims 32c + 8 grp .. +7 (fp16) ----
    uint32_t qw[NQK][4];
    if (hv) {
#pragma unroll
        for (int c = 0; c < NQK; ++c) {
            const uint4 v = *reinterpret_cast<const uint4*>(a.q + (row0 + hl) * D + 32 * c + 8 * grp);
            qw[c][0] = v.x; qw[c][1] = v.y; qw[c][2] = v.z; qw[c][3] = v.w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < NQK; ++c) qw[c][0] = qw[c][1] = qw[c][2] = qw[c][3] = 0u;
    }
    load_page(page_id(p0), st0);   // the first page loads while q is prepared
    if (a.k_smooth) {   // keys stored smoothed (k / s): the query meets q * s (s a power of two: exact)
#pragma unroll
        for (int c = 0; c < NQK; ++c) {
            const float4* sp4 = reinterpret_cast<const float4*>(a.k_smooth + 32 * c + 8 * grp);
            const float4 s0 = __ldg(sp4), s1 = __ldg(sp4 + 1);
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int w = 0; w < 4; ++w)
                qw[c][w] = pack_bf16_rne(bf16_lo(qw[c][w]) * smooth_pow2(sv[2 * w]),
                                         bf16_hi(qw[c][w]) * smooth_pow2(sv[2 * w + 1]));
        }
    }
    uint32_t mx = 0u;   // bit patterns of |bf16| order as the values do
#pragma unroll
    for (int c = 0; c < NQK; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) mx = max(mx, max(qw[c][w] & 0x7fffu, (qw[c][w] >> 16) & 0x7fffu));
    mx = head_umax(mx);
    const int sh = min(141 - (int)(mx >> 7), 127);   // 14 - exponent of the head's largest |q|
    f16x8 qb[NQK];
    float qsum = 0.0f;
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
        u32x4 w4;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t x = pack_f16(ldexpf(bf16_lo(qw[c][w]), sh), ldexpf(bf16_hi(qw[c][w]), sh));
            qsum += f16_lo(x) + f16_hi(x);
            w4[w] = x;
        }
        qb[c] = __builtin_bit_cast(f16x8, w4);
    }
    const float qbias = -kCodeOffset * stride_sum<16>(qsum);
    const f32x4 acc0 = {qbias, qbias, qbias, qbias};
    const float c2 = ldexpf(a.sm_scale * kLog2e, -sh);   // scores in log2 units

    // LDS read offsets (from a stage's start).  K operand of q.k c: key hl, bytes
    // 32c + 8 grp .. +7, which is slot 2c + grp/2, half grp % 2.  V operand of
    // p.v pair m (column blocks 2m, 2m+1): lane j of a 16-lane group points at
    // row j/2 of the 8-row block, half j % 2: rows 0..3 are keys 4 grp + r of
    // block 2m, rows 4..7 the same keys of block 2m + 1.
    uint32_t koff[NQK], voff[NMB / 2];
#pragma unroll
    for (int c = 0; c < NQK; ++c)
        koff[c] = (uint32_t)(hl * D + 16 * ((2 * c + grp / 2) ^ (hl % SL)) + 8 * (grp % 2));
    {
        const int r = hl / 2, key = 4 * grp + r % 4;
#pragma unroll
        for (int m = 0; m < NMB / 2; ++m)
            voff[m] = (uint32_t)(kTile + key * D + 16 * ((2 * m + r / 4) ^ (key % SL)) + 8 * (hl % 2));
    }

    f32x4 o[NMB];
#pragma unroll
    for (int m = 0; m < NMB; ++m) o[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY;   // running max (log2 units) of head hl
    float l_run = 0.0f;        // sum of 2^(s - m_run) over this lane's keys
    // The weights enter p.v as fp16 w = p * scale_v * 2^-vexp.  vexp is wave-uniform
    // and only rises: when a value scale exceeds vlim = 2^(vexp + 7), vexp moves to
    // 3 below the exponent of the page's largest scale (frexp's), and o and wsum
    // are rescaled by the power of two, so w <= 2^8 * 2^7 always fits fp16.
    int vexp = -1000;
    float vlim = 0.0f;
    float wsum = 0.0f;         // sum of this lane's rounded weights

    auto page = [&](int p, const LDS3 int8_t* st) __attribute__((always_inline)) {
        // this page's stage has landed once at most the next page's direct loads
        // (issued before this page whenever p < p1) are in flight
        if (!kAudit && p < p1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int kpos0 = p * kPage;

        // ---- q.k ----
        f32x4 acc = acc0;
#pragma unroll
        for (int c = 0; c < NQK; ++c) {
            const u32x2 w = *(const LDS3 u32x2*)(st + koff[c]);
            const u32x2 ka = codes_f16(w.x), kb = codes_f16(w.y);
            const u32x4 k4 = {ka[0], ka[1], kb[0], kb[1]};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k4), qb[c], acc, 0, 0, 0);
        }
        i32x2 raw[NMB / 2];
#pragma unroll
        for (int m = 0; m < NMB / 2; ++m) raw[m] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS3 i32x2*)(st + voff[m]));
        const f32x4 ks4 = *(const LDS3 f32x4*)(st + 2 * kTile + 16 * grp);
        const f32x4 vs4 = *(const LDS3 f32x4*)(st + 2 * kTile + 256 + 16 * grp);
        float s[4], vsl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j] = acc[j] * (c2 * ks4[j]);
            vsl[j] = vs4[j];
        }
        // keys outside [lo, hi) (on a split's first and last pages only): score
        // -inf and value scale 0 by a select, never by arithmetic, since their
        // scales may be poison
        if (!(kpos0 >= lo && kpos0 + kPage <= hi)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = kpos0 + 4 * grp + j;
                const bool out = key < lo || key >= hi;
                s[j] = out ? -INFINITY : s[j];
                vsl[j] = out ? 0.0f : vsl[j];
            }
        }
        // ---- value-scale exponent (the first page with a non-zero scale, then rarely) ----
        if (__any(vsl[0] > vlim || vsl[1] > vlim || vsl[2] > vlim || vsl[3] > vlim)) {
            float vm = vmax(vmax(vsl[0], vsl[1]), vmax(vsl[2], vsl[3]));
            vm = xor32_vmax(xor16_vmax(vm));   // > 0 here
            const int en = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(vm)) - 3;
            const float f = ldexpf(1.0f, vexp - en);   // 0 the first time
#pragma unroll
            for (int m = 0; m < NMB; ++m) o[m] *= f;
            wsum *= f;
            vexp = en;
            vlim = ldexpf(1.0f, en + 7);
        }
        // ---- running max with headroom 8 ----
        if (__any(s[0] > m_run + 8.0f || s[1] > m_run + 8.0f || s[2] > m_run + 8.0f || s[3] > m_run + 8.0f)) {
            float pm = vmax(vmax(s[0], s[1]), vmax(s[2], s[3]));
            pm = xor32_vmax(xor16_vmax(pm));
            const float m_new = vmax(m_run, pm);
            const float alpha = fast_exp2(m_run - m_new);   // 0 on the first page
            l_run *= alpha;
            wsum *= alpha;
#pragma unroll
            for (int m = 0; m < NMB; ++m) o[m] *= alpha;
            m_run = m_new;
        }
        // ---- weights (masked keys weigh 0) ----
        float w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float pw = fast_exp2(s[j] - m_run);
            l_run += pw;
            w[j] = pw * ldexpf(vsl[j], -vexp);
        }
        const uint32_t w01 = pack_f16(w[0], w[1]), w23 = pack_f16(w[2], w[3]);
        const f16x2 one2 = __builtin_bit_cast(f16x2, 0x3C003C00u);
        wsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w01), one2, wsum, false);
        wsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w23), one2, wsum, false);
        const u32x2 wp = {w01, w23};
        const f16x4 wb = __builtin_bit_cast(f16x4, wp);
        // ---- p.v ----
#pragma unroll
        for (int m = 0; m < NMB / 2; ++m) {
            const u32x2 va = codes_f16((uint32_t)raw[m].x), vb = codes_f16((uint32_t)raw[m].y);
            o[2 * m] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, va), wb, o[2 * m], 0, 0, 0);
            o[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vb), wb, o[2 * m + 1], 0, 0, 0);
        }
    };

    // page p is consumed from one stage while page p + 1 loads into the other
    {
        int nid = page_id(p0 + 1);
        int p = p0;
        for (; p < p1; p += 2) {
            load_page(nid, st1);
            nid = page_id(p + 2);
            page(p, st0);
            if (p + 1 < p1) {
                load_page(nid, st0);
                nid = page_id(p + 3);
            }
            page(p + 1, st1);
        }
        if (p == p1) page(p, st0);
    }

    // ---- out: head hl's row, columns 16m + 4 grp .. +3 ----
    const float l_tot = stride_sum<16>(l_run);
    const float w_tot = stride_sum<16>(wsum);
    if (hv) {
        float den = l_tot;
        if constexpr (FINAL) {
            if (a.sinks) den += fast_exp2(__ldg(a.sinks + head0 + hl) * kLog2e - m_run);
        }
        const float f = (FINAL && !(den > 0.0f)) ? 0.0f : 1.0f / den;
        float* row = FINAL ? a.out + (row0 + hl) * D : a.o_part + ((row0 + hl) * a.max_splits + sp) * D;
#pragma unroll
        for (int m = 0; m < NMB; ++m) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = ldexpf(fmaf(-kCodeOffset, w_tot, o[m][j]) * f, vexp);
            float* dst = row + 16 * m + 4 * grp;
            if (fused) {
#pragma unroll
                for (int j = 0; j < 4; ++j) put(dst + j, v[j]);
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
        if constexpr (!FINAL) {
            if (grp == 0) put(a.lse_part + (row0 + hl) * a.max_splits + sp, (m_run + fast_log2(l_tot)) * kLn2);
        }
    }
    arrive();
}

template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t s) {
    const int rows = a.num_kv_heads * a.batch;
    if (a.max_splits == 1)
        hipLaunchKernelGGL((decode_int8_mfma_kernel<D, true>), dim3(rows), dim3(kWave), 0, s, a, a.block_table);
    else
        hipLaunchKernelGGL((decode_int8_mfma_kernel<D, false>), dim3(a.max_splits * rows), dim3(kWave), 0, s, a,
                           a.block_table);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_int8_mfma(const DecodeArgs& a, int head_dim, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    return head_dim == 128 ? launch<128>(a, s) : launch<64>(a, s);
}

}  // namespace pfa

// Device-side helpers shared by the gfx950 kernels: bf16 unpacking, cross-lane
// moves within a 64-wide wavefront, and the launch-side declarations each kernel
// file exports to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pfa.h"

namespace pfa {

constexpr int kWave = 64;
constexpr int kPage = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPrefillRows = 256;       // query rows (token x head-of-group) per prefill workgroup
constexpr int kPrefillRowsSplit = 128;  // the same, for the KV-split kernel (short chunks on long prefixes)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 pair packed in a dword -> the two floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// Two floats that are exact in bf16 (small integers) -> packed pair, by truncation.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Round two floats to bf16 (nearest, ties to even) and pack.
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ---- cross-lane moves -------------------------------------------------------
// x from lane (lane ^ M).  Chooses a DPP or swizzle form where one exists.
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
    int v = __float_as_int(x);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);        // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);        // quad_perm [2,3,0,1]
    } else if constexpr (M == 8) {
        r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);       // row_ror:8
    } else if constexpr (M == 4 || M == 16) {
        r = __builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1F);         // bitmask mode, xor M
    } else {
        static_assert(M == 32, "xor mask");
        r = __builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32) << 2), v);
    }
    return __int_as_float(r);
}

// max / sum of x over lanes i and i ^ 32, on the VALU.  v_permlane32_swap with x
// in both operands leaves (x_i, x_{i^32}) in the two results, in either order.
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x from lane ((lane & ~(W-1)) | src) for groups of W lanes, W in {4, 8, 16, 32}.
template <int W>
__device__ __forceinline__ float group_bcast(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(
        (int)(((__lane_id() & ~(W - 1)) | src) << 2), __float_as_int(x)));
}

// max / sum of x over lanes i and i ^ 16, on the VALU: v_permlane16_swap with x in
// both operands leaves (x of row 2r, x of row 2r+1) in the two results.
__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v_max_f32 / v_max3_f32 as they stand.  fmaxf makes the compiler quiet
// signalling NaNs in inputs it cannot prove canonical (a move per operand); these
// are for scores, which are never NaN where they are compared.
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// vmax over lanes i and i ^ 16, i ^ 32 (the permlane swaps)
__device__ __forceinline__ float xor16_vmax(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_vmax(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x + / max with x of lane (lane ^ M).  M = 16 and 32 use the permlane swaps (VALU);
// the others a DPP or swizzle move.
template <int M>
__device__ __forceinline__ float xor_sum(float x) {
    if constexpr (M == 16) return xor16_sum(x);
    else if constexpr (M == 32) return xor32_sum(x);
    else return x + xor_lane<M>(x);
}
template <int M>
__device__ __forceinline__ float xor_max(float x) {
    if constexpr (M == 16) return xor16_max(x);
    else if constexpr (M == 32) return xor32_max(x);
    else return fmaxf(x, xor_lane<M>(x));
}

// Sum / max over all lanes whose ids differ only in bits [LO, 64): lane groups
// of stride LO.  LO is a power of two < 64.
template <int LO>
__device__ __forceinline__ float stride_sum(float x) {
    if constexpr (LO <= 1) x = xor_sum<1>(x);
    if constexpr (LO <= 2) x = xor_sum<2>(x);
    if constexpr (LO <= 4) x = xor_sum<4>(x);
    if constexpr (LO <= 8) x = xor_sum<8>(x);
    if constexpr (LO <= 16) x = xor_sum<16>(x);
    x = xor_sum<32>(x);
    return x;
}
template <int LO>
__device__ __forceinline__ float stride_max(float x) {
    if constexpr (LO <= 1) x = xor_max<1>(x);
    if constexpr (LO <= 2) x = xor_max<2>(x);
    if constexpr (LO <= 4) x = xor_max<4>(x);
    if constexpr (LO <= 8) x = xor_max<8>(x);
    if constexpr (LO <= 16) x = xor_max<16>(x);
    x = xor_max<32>(x);
    return x;
}

// INT8 key smoothing uses, per channel, the largest power of two not above the
// given weight s (the weight with its mantissa bits cleared), so that k / s and
// q * s are exact.
__device__ __forceinline__ float smooth_pow2(float s) { return __uint_as_float(__float_as_uint(s) & 0xff800000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace pfa

// ---- launchers exported by each kernel file to the C-ABI layer ---------------
namespace pfa {

// The 3-bit rotated cache's codebook as the kernels use it (fp32): magnitudes
// M[0..3] (ascending) and the magnitude thresholds T[0..2].
struct Tq3Book {
    float m[4];
    float t[3];
};

// Bounds-check build (PFA_BOUNDS_CHECK=1): the kernels also report violations of
// the device-side contract (page ids, lengths) by OR-ing PFA_BOUNDS_* bits into
// an error word (Args::err).  The clamps that keep every access in bounds are the
// same in both builds.
#ifndef PFA_BOUNDS_CHECK
#define PFA_BOUNDS_CHECK 0
#endif
constexpr bool kBoundsCheck = PFA_BOUNDS_CHECK != 0;

// One lane of the active ones ORs `bit` into *err when any of them is `bad`.
__device__ __forceinline__ void report(uint32_t* err, bool bad, uint32_t bit) {
    if constexpr (kBoundsCheck) {
        const uint64_t m = __ballot(bad);
        if (m != 0 && __lane_id() == (unsigned)(__ffsll((unsigned long long)m) - 1)) atomicOr(err, bit);
    }
}

struct KvWriteArgs {
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int32_t* cu_new;
    const int32_t* seq_lens;
    const int32_t* block_table;
    void* k_pool;
    void* v_pool;
    float* k_scale;
    float* v_scale;
    const float* k_smooth;      // INT8: [D] per-channel key smoothing, or NULL
    int32_t bt_stride, batch, num_tokens, num_pages, num_kv_heads, head_dim;
    Tq3Book book;               // 3-bit pools only

    uint32_t* err;             // bounds-check build: the error word; else NULL
};

struct DecodeArgs {
    const uint16_t* q;
    const void* k_pool;
    const void* v_pool;
    const float* k_scale;
    const float* v_scale;
    const float* k_smooth;      // INT8: [D] per-channel key smoothing (q is scaled by it), or NULL
    const int32_t* block_table;
    const int32_t* seq_lens;
    const float* sinks;
    float* o_part;
    float* lse_part;
    float* out;
    int32_t* counters;         // split mode, fused merge: [batch * num_kv_heads], zero on entry; else NULL
    int32_t bt_stride, batch, num_pages, num_q_heads, num_kv_heads;
    int32_t split_keys, max_splits, window;
    float sm_scale;
    uint32_t* err;             // bounds-check build: the error word; else NULL
};

struct AttnInputArgs {
    const uint16_t* qkv;        // [T][(Hq + 2 Hkv) * D] bf16
    const uint16_t* q_norm_w;   // [D] bf16
    const uint16_t* k_norm_w;   // [D] bf16
    const float* rope;          // [rope_max_pos][D/2][2] fp32 (cos, sin)
    const int32_t* cu_new;
    const int32_t* seq_lens;
    const int32_t* block_table;
    uint16_t* q_out;            // [T][Hq][D] bf16
    void* k_pool;
    void* v_pool;
    float* k_scale;
    float* v_scale;
    const float* k_smooth;      // INT8: [D] per-channel key smoothing, or NULL
    float eps;
    int32_t bt_stride, batch, num_tokens, num_pages, num_q_heads, num_kv_heads, rope_max_pos;

    uint32_t* err;             // bounds-check build: the error word; else NULL
};

struct CombineArgs {
    const float* o_part;
    const float* lse_part;
    const int32_t* seq_lens;   // decode: splits per row = ceil(len/S); NULL: all max_splits
    const int32_t* cu_rows;    // prefill: rows of sequence s are cu_rows[s]..cu_rows[s+1]-1
    const float* sinks;
    float* out;
    int32_t batch, num_q_heads, split_keys, max_splits;
    int32_t rows_per_seq;      // with cu_rows: host bound on rows per sequence
};

struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k_pool;     // bf16, or INT8 codes (then k_scale != NULL)
    const uint16_t* v_pool;
    const float* k_scale;       // INT8: [num_pages][Hkv][P]; NULL for BF16
    const float* v_scale;
    const float* k_smooth;      // INT8: [D] per-channel key smoothing (q is scaled by it), or NULL
    const int32_t* cu_q;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const float* sinks;
    float* out;
    float* o_part;             // split mode: [Tq][Hq][max_splits][D]
    float* lse_part;           // split mode: [Tq][Hq][max_splits]
    int32_t bt_stride, batch, num_pages, num_q_heads, num_kv_heads, max_q_len, window;
    int32_t split_keys, max_splits;   // max_splits == 1: no split
    float sm_scale;

    uint32_t* err;             // bounds-check build: the error word; else NULL
};

// kv_dtype: 0 bf16, 1 int8, 2 3-bit rotated
hipError_t launch_kv_write(const KvWriteArgs& a, int kv_dtype, hipStream_t s);
hipError_t launch_attn_input(const AttnInputArgs& a, int head_dim, bool int8, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool int8, hipStream_t s);
// INT8 at 8 query heads per KV head, on the matrix cores (launch_decode calls it)
hipError_t launch_decode_int8_mfma(const DecodeArgs& a, int head_dim, hipStream_t s);
hipError_t launch_decode_tq3(const DecodeArgs& a, int head_dim, const Tq3Book& bk, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, hipStream_t s);
hipError_t launch_prefill_split(const PrefillArgs& a, int head_dim, hipStream_t s);

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte direct load HBM -> LDS: lane l's 16 bytes come from base + voff (bytes)
// and land at LDS byte address lds + 16*l.  base and lds are wave-uniform.  Issued
// as asm, so the compiler keeps no LDS-DMA bookkeeping of its own: it would
// otherwise make every transposed LDS read wait for all direct loads in flight.
// The caller orders LDS accesses against these loads (vmcnt waits and barriers).
// (M0 is the LDS base; a write of M0 needs one wait state before the load.)
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    // (readfirstlane returns int: both halves go through uint32_t, so that the
    // low word is zero-extended)
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint64_t sb = ((uint64_t)hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// 4-byte direct load HBM -> LDS: lane l's 4 bytes come from base + voff and land
// at LDS byte address lds + 4*l; otherwise as dma16.
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint64_t sb = ((uint64_t)hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

}  // namespace pfa

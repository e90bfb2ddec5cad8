/*
 * pfa.h - paged flash attention for AMD MI355X (gfx950): the C ABI.
 *
 * What it computes
 * ----------------
 * Attention for LLM inference over a KV cache kept in a pool of fixed-size pages.
 * Each sequence reaches its pages through its own row of a block table.  The
 * TileInfer.jl performance page ("Fused kernels, FlashAttention and
 * PagedAttention") describes the operation.  The result is the one reference ops
 * produce when they gather the pages into dense K and V and materialise the
 * softmax.  The kernels instead read each page once, in place, with an online
 * softmax: split-KV for decode, then a separate combine kernel.  Prefill appends
 * a new turn to a restored prefix.  The Qml-engine announcement explains that a
 * session turn restores the conversation's KV from the store, so only the new turn
 * is prefilled.  Its model table also covers gpt-oss-20b, with attention sinks and
 * a sliding window.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers to memory the caller owns.  The
 *    library never allocates, frees or keeps a pointer past the call.
 *  - Every call only enqueues work on `stream`, a hipStream_t passed as void*.
 *    NULL means the null stream.  The caller synchronises.
 *  - Arrays are dense, row-major, in the layouts stated below.  bf16 means IEEE
 *    bfloat16.  Integers are int32.
 *  - Pool layout: k_pool/v_pool [num_pages][Hkv][P][D].  Position j of sequence s
 *    lives in page block_table[s*bt_stride + j/P], slot j%P.  INT8 pools add
 *    k_scale/v_scale [num_pages][Hkv][P] fp32, one scale per cached vector.
 *  - Positions: a sequence holds seq_lens[s] tokens.  That count includes the new
 *    ones.  Its q_len new tokens sit at positions seq_lens[s]-q_len ... seq_lens[s]-1.
 *    The query at position `pos` sees key j when j <= pos and, if window W > 0,
 *    when pos - j < W.  GQA uses contiguous groups: query head h reads KV head
 *    h / (Hq/Hkv).
 *  - Sinks: when desc->sinks != NULL, query head h has one extra logit sinks[h].
 *    It is not multiplied by sm_scale.  It enters the softmax max and denominator
 *    only, with no value vector.
 *  - Errors: host-checkable problems return a status and launch nothing.  That
 *    covers NULL pointers, inconsistent sizes and unsupported shapes.  A failed
 *    launch returns PFA_ERR_HIP, and pfa_last_hip_error() then gives the hipError_t
 *    code (thread-local).  Device-resident contents are the caller's contract:
 *    block-table entries in [0, num_pages), 0 <= seq_lens[s] <= bt_stride*P, each
 *    sequence's new-token count (from cu_q / cu_new) between 0 and seq_lens[s]
 *    (and at most max_q_len), and cu arrays that stay inside the q/out tensors.
 *    The kernels clamp page ids and lengths so that a broken page id or length
 *    gives wrong numbers, never an access outside the pool or the block table.  A
 *    debug build of the library (PFA_BOUNDS_CHECK=1, libpfa_debug.so) also reports
 *    such violations: see pfa_bounds_errors.
 *
 * Supported shapes: head_dim 64 or 128; page_size 16; Hq % Hkv == 0.
 *  - Decode: group size G = Hq/Hkv in {1,2,4,8}; BF16, INT8 or TQ3 K/V.
 *  - Prefill and verify: G in {1,2,4,8,16,32}; BF16 or INT8 K/V.
 */
#ifndef PFA_H
#define PFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PFA_OK = 0,
    PFA_ERR_NULL = 1,          /* a required pointer is NULL                          */
    PFA_ERR_SHAPE = 2,         /* sizes inconsistent or out of range                  */
    PFA_ERR_UNSUPPORTED = 3,   /* head_dim / page_size / dtype / group size not built */
    PFA_ERR_WORKSPACE = 4,     /* split buffers too small for max_seq_len/split_keys  */
    PFA_ERR_HIP = 5            /* a HIP call failed; see pfa_last_hip_error()         */
} pfa_status;

/*
 * KV cache element formats.
 *   PFA_KV_TQ3: the 3-bit rotated cache of the qengine README's feature list (a
 *   Walsh-Hadamard rotation followed by an 8-level Lloyd-Max scalar quantiser).
 *   Each cached K or V vector x of D elements is stored as:
 *     y = H_D x          (Walsh-Hadamard, Sylvester order, unnormalised)
 *     s = sqrt(sum(y^2) / D)                        (fp32 scale, one per vector)
 *     t = y / s  (t = 0 when s = 0), coded by the symmetric 8-level Lloyd-Max
 *     quantiser of N(0, 1) (pfa_tq3_codebook): bits 0-1 of a code are the
 *     magnitude index m = #{k : |t| >= T[k]}, bit 2 is 1 when t >= 0;
 *     packed as D/8 little-endian 24-bit fields of 3 bytes: field j holds the
 *     codes of elements 8j .. 8j+7, element 8j+i in bits 3i .. 3i+2.
 *   The cache stands for x^ = H_D (s * c) / D with c = +-M[m].  kv_write and
 *   decode (split or not; not the fused merge) take it; prefill, verify and
 *   attn_input return PFA_ERR_UNSUPPORTED.  The encoder's decisions are made in
 *   fp32 in a fixed order: butterflies of stride 1, 2, ..., D/2, each (a+b, a-b);
 *   the squares summed over consecutive groups of 8 in order, then the groups in
 *   a pairwise tree (group g with g^1, then g^2, ...); a correctly rounded sqrt
 *   and division.
 */
typedef enum { PFA_KV_BF16 = 0, PFA_KV_INT8 = 1, PFA_KV_TQ3 = 2 } pfa_kv_dtype;

/* Attention shape and options. */
typedef struct {
    int32_t num_q_heads;       /* Hq                                                  */
    int32_t num_kv_heads;      /* Hkv, divides Hq                                     */
    int32_t head_dim;          /* D: 64 or 128                                        */
    int32_t page_size;         /* P: 16                                               */
    int32_t kv_dtype;          /* pfa_kv_dtype                                        */
    int32_t window;            /* 0 = full attention; W > 0: keys pos-W < j <= pos    */
    float sm_scale;            /* multiplies q.k (e.g. 1/sqrt(D)); decode, prefill and */
                               /* verify need it positive and finite (PFA_ERR_SHAPE)  */
    const float* sinks;        /* device [Hq] fp32 sink logits, or NULL               */
} pfa_attn_desc;

/* The page pool.
 *   k_smooth (INT8 only, optional): the key smoothing of the TileInfer.jl
 *   performance page ("INT8 KV cache": keys smoothed by the key norm's weight).
 *   A device [D] fp32 vector w, every w_d a positive normal float (e.g. |k_norm
 *   weight|).  The cache smooths channel d by s_d, the largest power of two not
 *   above w_d (w_d with its mantissa bits cleared).  The KV writes quantise k/s
 *   per vector and decode meets q*s; both are exact, so q.k is unchanged.  The
 *   cache dequantises to code * scale * s.  NULL: no smoothing.  A BF16 pool with
 *   k_smooth set is PFA_ERR_UNSUPPORTED. */
typedef struct {
    void* k_pool;              /* device [num_pages][Hkv][P][D], bf16 or int8;        */
                               /* TQ3: [num_pages][Hkv][P][3D/8] bytes (packed codes) */
    void* v_pool;              /* same                                                */
    float* k_scale;            /* device [num_pages][Hkv][P] fp32; INT8/TQ3, else NULL */
    float* v_scale;            /* same                                                */
    int32_t num_pages;
    const float* k_smooth;     /* device [D] fp32 key smoothing (INT8 only), or NULL  */
} pfa_kv_pool;

/*
 * pfa_tq3_codebook: the codebook of PFA_KV_TQ3 as the kernels use it.
 *   magnitudes  host float[4]: M[0..3], ascending, the positive levels;
 *   thresholds  host float[3]: T[0..2], the magnitude thresholds.
 *   It is the 8-level Lloyd-Max (minimum mean-square error) quantiser of the unit
 *   normal: Lloyd's iteration in double precision (thresholds at the midpoints of
 *   adjacent levels, levels at the centroids of their cells) until no level moves
 *   by more than 1e-13, then each value rounded to float.  Host-only; no GPU call.
 *   Returns PFA_ERR_NULL for a NULL pointer.
 */
pfa_status pfa_tq3_codebook(float* magnitudes, float* thresholds);

/*
 * pfa_kv_write: append new tokens' K and V to their sequences' pages.
 *   The TileInfer.jl performance page names this step the KV cache write.  Its
 *   "INT8 KV cache" section adds one scale per cached vector.
 *
 *   k_new, v_new   device [num_tokens][Hkv][D] bf16.  The tokens of sequence s are
 *                  rows cu_new[s] .. cu_new[s+1]-1.
 *   cu_new         device [batch+1] int32, nondecreasing, with cu_new[0] = 0 and
 *                  cu_new[batch] = num_tokens.
 *   seq_lens       device [batch] int32: sequence lengths after the append.
 *                  Token i of s goes to position seq_lens[s] - n_s + i.
 *   block_table    device [batch][bt_stride] int32 page ids.
 *
 *   BF16 pools receive the bits unchanged.  INT8 pools receive codes and scales.
 *   For each (token, KV head) vector x, computed separately for K and V:
 *     scale = absmax(x) / 127                         (IEEE fp32 division)
 *     code  = clamp(rint(x / scale), -127, 127)       (ties to even)
 *   An all-zero vector gets scale 0 and codes 0.  TQ3 pools receive packed codes and
 *   scales as described at pfa_kv_dtype.  Tokens whose slot falls outside the block
 *   table or the pool are skipped.  PFA_ERR_SHAPE if num_tokens * Hkv * D/8 exceeds
 *   (2^31 - 1) * 256 (one thread per 8 elements).
 */
pfa_status pfa_kv_write(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                        const void* k_new, const void* v_new, const int32_t* cu_new,
                        const int32_t* seq_lens, const int32_t* block_table,
                        int32_t bt_stride, int32_t batch, int32_t num_tokens,
                        void* stream);

/*
 * pfa_attn_input: the attention inputs of new tokens, straight from the fused
 *   q/k/v projection: q/k RMSNorm, RoPE, and the KV-cache write, in one kernel.
 *   The TileInfer.jl performance page ("Fused kernels, FlashAttention and
 *   PagedAttention") fuses these, bit-identical to the chain of per-op kernels.
 *   The chain: each op reads and writes bf16 (round to nearest even); inside an
 *   op, IEEE fp32 with every product and sum rounded on its own:
 *     RMSNorm (per head vector x, weight w):
 *       ss = sum of x_d^2: left to right within each group of 8 consecutive
 *            elements, then the D/8 group sums pairwise (group j adds group
 *            j xor m, for m = D/16, ..., 1)
 *       y  = bf16((x * r) * w),  r = 1 / sqrt(ss / D + eps)
 *     RoPE (rotate-half), (c, s) = rope_cos_sin[pos][i], i < D/2:
 *       out_i = bf16(y_i c - y_(i+D/2) s),  out_(i+D/2) = bf16(y_(i+D/2) c + y_i s)
 *   q heads: RMSNorm(q_norm_weight), RoPE -> q_out.  k heads: RMSNorm(k_norm_weight),
 *   RoPE -> the pool.  v heads -> the pool unchanged.  INT8 pools receive codes and
 *   scales of the final k and v as pfa_kv_write computes them.
 *
 *   qkv          device [num_tokens][(Hq + 2 Hkv) * D] bf16: per token the Hq q heads,
 *                then the Hkv k heads, then the Hkv v heads.
 *   cu_new, seq_lens, block_table, bt_stride, batch: as pfa_kv_write; token i of
 *                sequence s sits at position seq_lens[s] - n_s + i.
 *   q_out        device [num_tokens][Hq][D] bf16.
 *   The positions must be < prm->rope_max_pos (the kernel clamps the table row).
 *   Tokens whose slot falls outside the block table or the pool write no K/V.
 */
typedef struct {
    const void* q_norm_weight;   /* device [D] bf16 */
    const void* k_norm_weight;   /* device [D] bf16 */
    const float* rope_cos_sin;   /* device [rope_max_pos][D/2][2] fp32: (cos, sin) */
    int32_t rope_max_pos;
    float eps;                   /* RMSNorm epsilon, 0 <= eps <= 1 */
} pfa_attn_input_params;

pfa_status pfa_attn_input(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                          const pfa_attn_input_params* prm, const void* qkv, const int32_t* cu_new,
                          const int32_t* seq_lens, const int32_t* block_table, int32_t bt_stride,
                          int32_t batch, int32_t num_tokens, void* q_out, void* stream);

/*
 * pfa_paged_attn_decode: one query per sequence, at position seq_lens[s]-1.  That
 *   token's K/V must already be written.  Split-KV: the TileInfer.jl performance
 *   page ("Fused kernels, ...") keeps the combine as a separate kernel.
 *
 *   q              device [batch][Hq][D] bf16.
 *   max_seq_len    host upper bound on seq_lens[].
 *   split_keys     S, a multiple of P.  Split i of a sequence covers keys
 *                  [i*S, min((i+1)*S, len)).
 *   max_splits     >= ceil(max_seq_len / S).
 *
 *   If max_splits == 1 (unsplit), the kernel writes the final result, sink
 *   included, to out [batch][Hq][D] fp32.  o_part and lse_part may be NULL.
 *   Otherwise, for every split i < ceil(seq_lens[s]/S), it writes:
 *     o_part   [batch][Hq][max_splits][D] fp32, the softmax-normalised partial output;
 *     lse_part [batch][Hq][max_splits] fp32, the natural log-sum-exp of the split's
 *              visible scores, or -inf when the window hides the whole split;
 *              the o_part rows of such a split are left unwritten.
 *   Partials never include the sink, and out is left untouched.  Then call
 *   pfa_paged_attn_combine.
 *
 *   The grid has one 64-lane workgroup per (split, KV head, sequence) for
 *   max_splits splits.  With a short sliding window, most splits of a long
 *   sequence are hidden and only write lse = -inf, so unsplit is the faster
 *   launch there: each wave then reads at most the window's pages.
 *
 *   A TQ3 pool is attended as the cache it stands for (pfa_kv_dtype).  The kernel
 *   works in the rotated domain: q . x^ = s * ((H_D q / D) . c), and the split's
 *   sum of p * s * c is rotated back by H_D / D at its end.
 *
 *   Arithmetic: scores and sums in fp32.  An INT8 pool meets q in fp16 after a
 *   per-head power-of-two scale (exact for every element within 2^28 of its head's
 *   largest).  At G = 8 the weights are rounded once before the p.v products: to
 *   bf16 pairs for BF16 pools (dot2 on key pairs); for INT8 pools, whose q.k and p.v
 *   run as fp16 matrix products with fp32 accumulation, to fp16 p * scale_v * 2^-e,
 *   with e a power of two that follows the split's largest value scale, so no
 *   weight overflows; a
 *   weight's rounding error is at most 2^-11 of it, or 2^-25 * 2^e in absolute terms
 *   where p * scale_v is more than about 2^17 below that largest scale (an fp16
 *   subnormal).
 */
pfa_status pfa_paged_attn_decode(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                                 const void* q, const int32_t* block_table, int32_t bt_stride,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                 int32_t split_keys, int32_t max_splits,
                                 float* o_part, float* lse_part, float* out, void* stream);

/*
 * pfa_paged_attn_decode_fused: decode with the combine fused into the split
 *   kernel, through an arrival counter per (sequence, KV head): the variant the
 *   TileInfer.jl performance page ("Fused kernels, FlashAttention and
 *   PagedAttention") measured, with an acquire-release counter, and did not keep.
 *   Arguments as pfa_paged_attn_decode, plus:
 *
 *   counters       device [batch][Hkv] int32, all zero on entry.  The call leaves
 *                  them zero when it completes, so one zeroed array serves every
 *                  later call on the same stream.  Calls that may run at the same
 *                  time (other streams) need arrays of their own.
 *   out            device [batch][Hq][D] fp32, always written.
 *
 *   Each split writes its partial to o_part / lse_part as in pfa_paged_attn_decode,
 *   with agent-scope atomic stores (written through to the device-coherent level),
 *   waits until those stores have completed, then adds one to its counter with an
 *   agent-scope atomic.  The split that brings the counter to ceil(seq_lens[s]/S)
 *   reads the row's partials back with agent-scope atomic loads, merges them with
 *   the combine formula, writes out, and resets the counter.  The ordering rests on
 *   the completed stores and the coherent loads rather than on release/acquire
 *   fences (which would write back or invalidate a whole L2 per workgroup).  No
 *   workgroup waits on another.  out equals, bit for bit, that of
 *   pfa_paged_attn_decode followed by pfa_paged_attn_combine.  seq_lens[s] >= 1.
 *   With max_splits == 1 this is pfa_paged_attn_decode (counters unused).
 */
pfa_status pfa_paged_attn_decode_fused(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                                       const void* q, const int32_t* block_table, int32_t bt_stride,
                                       const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                       int32_t split_keys, int32_t max_splits, float* o_part,
                                       float* lse_part, int32_t* counters, float* out, void* stream);

/*
 * pfa_paged_attn_decode_static: pfa_paged_attn_decode followed by
 *   pfa_paged_attn_combine, allocating nothing: the split partials live in a
 *   device array the library holds.  For callers that cannot allocate device
 *   memory: code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc.
 *
 *   Arguments as pfa_paged_attn_decode.  split_keys == 0 runs unsplit (out written
 *   directly, the array unused); otherwise max_splits = ceil(max_seq_len /
 *   split_keys), and o_part/lse_part take batch*Hq*max_splits*(D+1)*4 bytes (plus
 *   alignment) of the array.  PFA_ERR_WORKSPACE, with nothing launched, when that
 *   exceeds PFA_STATIC_SCRATCH_BYTES.  out [batch][Hq][D] fp32 is always written.
 *
 *   The array is per device (the current device, which must own `stream`), is
 *   looked up on the first call on that device and lasts until the process ends.
 *   It keeps the last call's partials; nothing in it needs to start at zero.
 *   Calls that can overlap on one device (other streams, other threads) race on
 *   it and must be serialised by the caller.
 */
#define PFA_STATIC_SCRATCH_BYTES (32u << 20)
pfa_status pfa_paged_attn_decode_static(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                                        const void* q, const int32_t* block_table, int32_t bt_stride,
                                        const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                        int32_t split_keys, float* out, void* stream);

/*
 * pfa_paged_attn_combine: merge the split partials (same page and section as
 *   decode).  For each (b, h), over the ceil(seq_lens[b]/S) splits of b:
 *     M   = max(max_i lse_i, sink_h)
 *     out = sum_i e^(lse_i - M) o_i / (sum_i e^(lse_i - M) + e^(sink_h - M))
 *   The sink terms appear only when desc->sinks != NULL.  out is [batch][Hq][D] fp32.
 *   The o_part rows of the leading splits with lse -inf are not read.
 */
pfa_status pfa_paged_attn_combine(const pfa_attn_desc* desc, const float* o_part,
                                  const float* lse_part, const int32_t* seq_lens, int32_t batch,
                                  int32_t split_keys, int32_t max_splits, float* out,
                                  void* stream);

/*
 * pfa_paged_attn_prefill: causal attention of every new token over its sequence.
 *   The keys are the restored prefix plus the new tokens, and the new tokens'
 *   K/V must already be written.  This covers a fresh prompt (prefix 0) and a
 *   chunked turn appended to a restored paged prefix.
 *
 *   q              device [num_q_tokens][Hq][D] bf16.  The new tokens of sequence s
 *                  are rows cu_q[s] .. cu_q[s+1]-1.
 *   cu_q           device [batch+1] int32, as cu_new above.
 *   seq_lens       device [batch] int32, prefix + new tokens.
 *   max_q_len      host upper bound on cu_q[s+1]-cu_q[s].
 *   max_seq_len    host upper bound on seq_lens[].
 *   out            device [num_q_tokens][Hq][D] fp32.
 *
 *   Split mode, when max_splits > 1: the key range is cut into ranges of
 *   split_keys keys, a multiple of 64, with max_splits >= ceil(max_seq_len /
 *   split_keys).  Use it when a chunk has too few query tiles to fill the GPU,
 *   e.g. a short turn on a long prefix.  Each range writes a softmax-normalised
 *   partial to o_part and its natural log-sum-exp to lse_part:
 *     o_part   [num_q_tokens][Hq][max_splits][D] fp32
 *     lse_part [num_q_tokens][Hq][max_splits] fp32
 *   A range with no visible key writes lse -inf.  A second kernel on the same
 *   stream then merges the partials into out, as pfa_paged_attn_combine does.
 *   When max_splits == 1, split_keys, o_part and lse_part are ignored.
 *
 *   With a sliding window of at most 512 keys, the work runs on the KV-split
 *   kernel build (128-row workgroups, 32-key tiles) whether or not the key range
 *   is split: each workgroup then sees only a few tiles, and the smaller
 *   workgroups keep more of them resident per CU.  So does an unsplit chunk whose
 *   256-row query tiles would number fewer than 256 (fewer workgroups than the
 *   MI355X has CUs): the 128-row tiles double them.
 *
 *   INT8 pools (the TileInfer.jl performance page prefills over its INT8 cache
 *   too) are attended as the cache they stand for, code * scale (* the smoothing
 *   factor).  Scores use the exact codes and each key's scale in fp32; values
 *   enter the matrix cores as bf16(code * scale_v), an error of at most 2^-9
 *   relative per value element.  TQ3 pools return PFA_ERR_UNSUPPORTED.
 */
pfa_status pfa_paged_attn_prefill(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                                  const void* q, const int32_t* cu_q,
                                  const int32_t* block_table, int32_t bt_stride,
                                  const int32_t* seq_lens, int32_t batch, int32_t max_q_len,
                                  int32_t max_seq_len, int32_t split_keys, int32_t max_splits,
                                  float* o_part, float* lse_part, float* out, void* stream);

/*
 * A prefill split choice for `num_cus` compute units (0 means 256).  It returns
 * max_splits, 1 when the query tiles alone give at least two workgroups per CU
 * or when the keys beyond the chunk (max_seq_len - max_q_len) are fewer than
 * half the chunk (a fresh prompt's causal triangle runs faster unsplit than
 * split and merged), and writes the matching split_keys to *split_keys (0 when
 * unsplit).  This is host-side arithmetic only.
 */
int32_t pfa_prefill_num_splits(const pfa_attn_desc* desc, int32_t batch, int32_t max_q_len,
                               int32_t max_seq_len, int32_t num_cus, int32_t* split_keys);

/*
 * pfa_paged_attn_verify: attention of a speculative-decoding verify step, the
 *   2-16 tokens per sequence (the last accepted token plus the drafted ones) that
 *   one forward pass checks.  TileInfer.jl performance page, section "Speculative
 *   decoding", paragraph on attention for verify steps: such steps run the
 *   split-KV kernels rather than the prefill kernel.
 *
 *   The result is the one pfa_paged_attn_prefill defines for a chunk of q_len new
 *   tokens: causal among the new tokens and over the whole cached prefix, with the
 *   same window and sinks.  Arguments, layouts and the split contract are those of
 *   pfa_paged_attn_prefill, with max_q_len <= 16 (PFA_ERR_SHAPE otherwise).  The
 *   work runs on the KV-split kernel build (128-row workgroups, 32-key tiles); use
 *   pfa_verify_num_splits for split_keys / max_splits.  max_splits == 1 is allowed
 *   and writes out directly.
 */
pfa_status pfa_paged_attn_verify(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                                 const void* q, const int32_t* cu_q,
                                 const int32_t* block_table, int32_t bt_stride,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_q_len,
                                 int32_t max_seq_len, int32_t split_keys, int32_t max_splits,
                                 float* o_part, float* lse_part, float* out, void* stream);

/*
 * A verify split choice for `num_cus` compute units (0 means 256): split_keys a
 * multiple of 64, enough ranges for about two workgroups per CU.  Returns
 * max_splits (1 and *split_keys = 0 when unsplit).  Host-side arithmetic only.
 */
int32_t pfa_verify_num_splits(const pfa_attn_desc* desc, int32_t batch, int32_t max_q_len,
                              int32_t max_seq_len, int32_t num_cus, int32_t* split_keys);

/* ceil(max_seq_len / split_keys), at least 1 (0 when split_keys <= 0). */
int32_t pfa_decode_num_splits(int32_t max_seq_len, int32_t split_keys);

/*
 * Bytes of the split buffers pfa_paged_attn_decode needs for `batch` sequences
 * and `max_splits` splits: o_part [batch][Hq][max_splits][D] fp32 plus lse_part
 * [batch][Hq][max_splits] fp32, i.e. batch*Hq*max_splits*(D+1)*4.  0 when
 * max_splits <= 1 (unsplit decode writes out directly), batch <= 0, or desc is
 * NULL or invalid.  The caller allocates them as two arrays.  Host-side
 * arithmetic only.
 */
size_t pfa_decode_workspace_bytes(const pfa_attn_desc* desc, int32_t batch, int32_t max_splits);

/*
 * pfa_bounds_errors: the device-side contract violations the kernels met on the
 * current device since the last call, as PFA_BOUNDS_* bits in *flags; the word is
 * then cleared.  Only a library built with PFA_BOUNDS_CHECK=1 (libpfa_debug.so)
 * checks: its kernels test each block-table entry they read against
 * [0, num_pages) and each length against its limits, and OR a bit into a device
 * error word.  Both builds clamp the same way, so a violation still yields wrong
 * numbers and no access outside the pool; the debug build also says so.  This
 * call synchronises the device (it is a debugging aid, not a hot-path call).  The
 * normal build returns PFA_ERR_UNSUPPORTED and sets *flags to 0.  PFA_ERR_NULL if
 * flags is NULL.
 */
#define PFA_BOUNDS_PAGE 1u     /* a block-table entry outside [0, num_pages)                   */
#define PFA_BOUNDS_SEQ_LEN 2u  /* seq_lens[s] < 0 or > bt_stride*P, or beyond the keys the      */
                               /* call covers (max_splits * split_keys)                        */
#define PFA_BOUNDS_Q_LEN 4u    /* a new-token count < 0, > seq_lens[s], or > max_q_len          */
pfa_status pfa_bounds_errors(uint32_t* flags);

/* Static description of a status code; never NULL. */
const char* pfa_status_string(pfa_status status);

/* hipError_t of the last PFA_ERR_HIP on this thread (0 if none). */
int32_t pfa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PFA_H */

// The C ABI of include/pfa.h: host-side argument checks, then one launch on the
// caller's stream.  Nothing here allocates.  State: the thread-local last HIP
// error, and for pfa_paged_attn_decode_static a file-scope device array whose
// per-device address is looked up once.
#include "pfa.h"

#include <algorithm>
#include <cmath>
#include <mutex>

#include "pfa_device.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

pfa_status hip_status(hipError_t e) {
    if (e == hipSuccess) return PFA_OK;
    g_last_hip_error = (int32_t)e;
    return PFA_ERR_HIP;
}

pfa_status check_desc(const pfa_attn_desc* d) {
    if (!d) return PFA_ERR_NULL;
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
        return PFA_ERR_SHAPE;
    if (d->window < 0) return PFA_ERR_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128) return PFA_ERR_UNSUPPORTED;
    if (d->page_size != 16) return PFA_ERR_UNSUPPORTED;
    if (d->kv_dtype != PFA_KV_BF16 && d->kv_dtype != PFA_KV_INT8 && d->kv_dtype != PFA_KV_TQ3)
        return PFA_ERR_UNSUPPORTED;
    return PFA_OK;
}

// The attention kernels take the softmax maximum over scores before the scale
// (prefill) or fold the scale into per-key factors, which holds for a positive
// scale only.
pfa_status check_scale(const pfa_attn_desc* d) {
    return (d->sm_scale > 0.0f && d->sm_scale <= 3.4e38f) ? PFA_OK : PFA_ERR_SHAPE;   // (false for NaN)
}

pfa_status check_pool(const pfa_attn_desc* d, const pfa_kv_pool* p) {
    if (!p || !p->k_pool || !p->v_pool) return PFA_ERR_NULL;
    if (d->kv_dtype != PFA_KV_BF16 && (!p->k_scale || !p->v_scale)) return PFA_ERR_NULL;
    if (d->kv_dtype != PFA_KV_INT8 && p->k_smooth) return PFA_ERR_UNSUPPORTED;
    if (p->num_pages <= 0) return PFA_ERR_SHAPE;
    return PFA_OK;
}

bool decode_group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

bool prefill_group_ok(int g) {
    return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32;
}

// The 3-bit rotated cache's codebook: the symmetric 8-level Lloyd-Max quantiser
// of N(0, 1) (the qengine README's feature list names a Lloyd-Max quantiser).  Lloyd's
// iteration on the positive half in double precision: thresholds at midpoints of
// adjacent levels (the first at 0), levels at the centroids of their cells,
// E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)), from 0.25, 0.75, 1.25,
// 2.0 until no level moves by more than 1e-13.  Then rounded to float.
const pfa::Tq3Book& tq3_book() {
    static const pfa::Tq3Book book = [] {
        auto phi = [](double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); };
        auto cdf = [](double x) { return std::isinf(x) ? 1.0 : 0.5 * (1.0 + std::erf(x / std::sqrt(2.0))); };
        double m[4] = {0.25, 0.75, 1.25, 2.0};
        for (int it = 0; it < 100000; ++it) {
            const double e[5] = {0.0, 0.5 * (m[0] + m[1]), 0.5 * (m[1] + m[2]), 0.5 * (m[2] + m[3]), INFINITY};
            double moved = 0.0;
            double n[4];
            for (int k = 0; k < 4; ++k) {
                n[k] = (phi(e[k]) - phi(e[k + 1])) / (cdf(e[k + 1]) - cdf(e[k]));
                moved = std::max(moved, std::fabs(n[k] - m[k]));
            }
            for (int k = 0; k < 4; ++k) m[k] = n[k];
            if (moved <= 1e-13) break;
        }
        pfa::Tq3Book b;
        for (int k = 0; k < 4; ++k) b.m[k] = (float)m[k];
        for (int k = 0; k < 3; ++k) b.t[k] = (float)(0.5 * (m[k] + m[k + 1]));
        return b;
    }();
    return book;
}

#define PFA_TRY(expr)                    \
    do {                                 \
        pfa_status st_ = (expr);         \
        if (st_ != PFA_OK) return st_;   \
    } while (0)

// The split partials of pfa_paged_attn_decode_static.  Every GPU the library
// runs on holds its own copy of this array from the code object's load until the
// process ends.  In host code `scratch` names a host-side stand-in, never a device
// address: the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = (size_t)PFA_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

pfa_status static_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return PFA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return PFA_ERR_HIP;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return PFA_OK;
}

// The device error word of the bounds-check build (PFA_BOUNDS_CHECK=1), one per
// GPU; its address comes from hipGetSymbolAddress once per device, like the
// scratch array's.  The normal build passes no error word to its kernels.
static __device__ uint32_t bounds_word;

pfa_status bounds_word_ptr(uint32_t** ptr) {
    *ptr = nullptr;
    if constexpr (!pfa::kBoundsCheck) return PFA_OK;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return PFA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(bounds_word));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return PFA_ERR_HIP;
        addr[dev] = p;
    }
    *ptr = static_cast<uint32_t*>(addr[dev]);
    return PFA_OK;
}

}  // namespace

extern "C" {

pfa_status pfa_bounds_errors(uint32_t* flags) {
    if (!flags) return PFA_ERR_NULL;
    *flags = 0u;
    if constexpr (!pfa::kBoundsCheck) return PFA_ERR_UNSUPPORTED;
    uint32_t* w = nullptr;
    PFA_TRY(bounds_word_ptr(&w));
    PFA_TRY(hip_status(hipDeviceSynchronize()));
    PFA_TRY(hip_status(hipMemcpy(flags, w, sizeof(uint32_t), hipMemcpyDeviceToHost)));
    const uint32_t zero = 0u;
    PFA_TRY(hip_status(hipMemcpy(w, &zero, sizeof(uint32_t), hipMemcpyHostToDevice)));
    return PFA_OK;
}

pfa_status pfa_kv_write(const pfa_attn_desc* desc, const pfa_kv_pool* pool, const void* k_new,
                        const void* v_new, const int32_t* cu_new, const int32_t* seq_lens,
                        const int32_t* block_table, int32_t bt_stride, int32_t batch,
                        int32_t num_tokens, void* stream) {
    PFA_TRY(check_desc(desc));
    PFA_TRY(check_pool(desc, pool));
    if (batch < 0 || num_tokens < 0 || bt_stride <= 0) return PFA_ERR_SHAPE;
    if (num_tokens > 0 && batch == 0) return PFA_ERR_SHAPE;
    // one thread per 8 elements of a (token, KV head) vector, 256 per workgroup
    if ((int64_t)num_tokens * desc->num_kv_heads * (desc->head_dim / 8) > (int64_t)0x7fffffff * 256)
        return PFA_ERR_SHAPE;
    if (num_tokens == 0) return PFA_OK;
    if (!k_new || !v_new || !cu_new || !seq_lens || !block_table) return PFA_ERR_NULL;
    pfa::KvWriteArgs a;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.cu_new = cu_new;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.k_pool = pool->k_pool;
    a.v_pool = pool->v_pool;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.k_smooth = pool->k_smooth;
    a.bt_stride = bt_stride;
    a.batch = batch;
    a.num_tokens = num_tokens;
    a.num_pages = pool->num_pages;
    a.num_kv_heads = desc->num_kv_heads;
    a.head_dim = desc->head_dim;
    a.book = tq3_book();
    PFA_TRY(bounds_word_ptr(&a.err));
    return hip_status(pfa::launch_kv_write(a, desc->kv_dtype, (hipStream_t)stream));
}

pfa_status pfa_attn_input(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                          const pfa_attn_input_params* prm, const void* qkv, const int32_t* cu_new,
                          const int32_t* seq_lens, const int32_t* block_table, int32_t bt_stride,
                          int32_t batch, int32_t num_tokens, void* q_out, void* stream) {
    PFA_TRY(check_desc(desc));
    PFA_TRY(check_pool(desc, pool));
    if (desc->kv_dtype == PFA_KV_TQ3) return PFA_ERR_UNSUPPORTED;
    if (!prm) return PFA_ERR_NULL;
    if (batch < 0 || num_tokens < 0 || bt_stride <= 0 || prm->rope_max_pos <= 0) return PFA_ERR_SHAPE;
    if (!(prm->eps >= 0.0f) || prm->eps > 1.0f) return PFA_ERR_SHAPE;
    if (num_tokens > 0 && batch == 0) return PFA_ERR_SHAPE;
    if ((int64_t)num_tokens * pfa::kWave > 0xffffffffLL - 256) return PFA_ERR_SHAPE;   // one wave per token
    if ((int64_t)desc->num_q_heads + 2 * desc->num_kv_heads > 65536) return PFA_ERR_SHAPE;
    if (num_tokens == 0) return PFA_OK;
    if (!qkv || !cu_new || !seq_lens || !block_table || !q_out || !prm->q_norm_weight ||
        !prm->k_norm_weight || !prm->rope_cos_sin)
        return PFA_ERR_NULL;
    pfa::AttnInputArgs a;
    a.qkv = static_cast<const uint16_t*>(qkv);
    a.q_norm_w = static_cast<const uint16_t*>(prm->q_norm_weight);
    a.k_norm_w = static_cast<const uint16_t*>(prm->k_norm_weight);
    a.rope = prm->rope_cos_sin;
    a.cu_new = cu_new;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.q_out = static_cast<uint16_t*>(q_out);
    a.k_pool = pool->k_pool;
    a.v_pool = pool->v_pool;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.k_smooth = pool->k_smooth;
    a.eps = prm->eps;
    a.bt_stride = bt_stride;
    a.batch = batch;
    a.num_tokens = num_tokens;
    a.num_pages = pool->num_pages;
    a.num_q_heads = desc->num_q_heads;
    a.num_kv_heads = desc->num_kv_heads;
    a.rope_max_pos = prm->rope_max_pos;
    PFA_TRY(bounds_word_ptr(&a.err));
    return hip_status(pfa::launch_attn_input(a, desc->head_dim, desc->kv_dtype == PFA_KV_INT8,
                                             (hipStream_t)stream));
}

pfa_status pfa_tq3_codebook(float* magnitudes, float* thresholds) {
    if (!magnitudes || !thresholds) return PFA_ERR_NULL;
    const pfa::Tq3Book& b = tq3_book();
    for (int k = 0; k < 4; ++k) magnitudes[k] = b.m[k];
    for (int k = 0; k < 3; ++k) thresholds[k] = b.t[k];
    return PFA_OK;
}

int32_t pfa_decode_num_splits(int32_t max_seq_len, int32_t split_keys) {
    if (split_keys <= 0) return 0;
    if (max_seq_len <= 0) return 1;
    return (int32_t)(((int64_t)max_seq_len + split_keys - 1) / split_keys);
}

size_t pfa_decode_workspace_bytes(const pfa_attn_desc* desc, int32_t batch, int32_t max_splits) {
    if (check_desc(desc) != PFA_OK || batch <= 0 || max_splits <= 1) return 0;
    return (size_t)batch * (size_t)desc->num_q_heads * (size_t)max_splits * ((size_t)desc->head_dim + 1) *
           sizeof(float);
}

namespace {

// pfa_paged_attn_decode and pfa_paged_attn_decode_fused: shared checks and launch.
// counters == nullptr is the plain decode.
pfa_status decode_like(const pfa_attn_desc* desc, const pfa_kv_pool* pool, const void* q,
                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                       int32_t batch, int32_t max_seq_len, int32_t split_keys, int32_t max_splits,
                       float* o_part, float* lse_part, int32_t* counters, float* out, void* stream,
                       bool fused) {
    PFA_TRY(check_desc(desc));
    PFA_TRY(check_scale(desc));
    PFA_TRY(check_pool(desc, pool));
    const int g = desc->num_q_heads / desc->num_kv_heads;
    if (!decode_group_ok(g)) return PFA_ERR_UNSUPPORTED;
    if (fused && desc->kv_dtype == PFA_KV_TQ3) return PFA_ERR_UNSUPPORTED;
    if (batch < 0 || batch > 65535 || bt_stride <= 0 || max_seq_len < 0 || max_splits < 1 ||
        desc->num_kv_heads > 65535)
        return PFA_ERR_SHAPE;
    if (max_seq_len > (int64_t)bt_stride * desc->page_size) return PFA_ERR_SHAPE;
    // one 64-lane workgroup per (split, KV head, sequence) in a 1-D grid
    if ((int64_t)max_splits * desc->num_kv_heads * batch > (int64_t)1 << 26) return PFA_ERR_SHAPE;
    if (batch == 0) return PFA_OK;
    if (!q || !block_table || !seq_lens) return PFA_ERR_NULL;
    if (max_splits == 1) {
        if (!out) return PFA_ERR_NULL;
    } else {
        if (split_keys <= 0 || split_keys % desc->page_size != 0) return PFA_ERR_SHAPE;
        if (max_splits < pfa_decode_num_splits(max_seq_len, split_keys)) return PFA_ERR_WORKSPACE;
        if (!o_part || !lse_part) return PFA_ERR_NULL;
        if (fused && (!counters || !out)) return PFA_ERR_NULL;
    }
    pfa::DecodeArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_pool = pool->k_pool;
    a.v_pool = pool->v_pool;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.k_smooth = pool->k_smooth;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.sinks = desc->sinks;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.out = out;
    a.counters = (fused && max_splits > 1) ? counters : nullptr;
    a.bt_stride = bt_stride;
    a.batch = batch;
    a.num_pages = pool->num_pages;
    a.num_q_heads = desc->num_q_heads;
    a.num_kv_heads = desc->num_kv_heads;
    a.split_keys = max_splits == 1 ? 0 : split_keys;
    a.max_splits = max_splits;
    a.window = desc->window;
    a.sm_scale = desc->sm_scale;
    PFA_TRY(bounds_word_ptr(&a.err));
    if (desc->kv_dtype == PFA_KV_TQ3)
        return hip_status(pfa::launch_decode_tq3(a, desc->head_dim, tq3_book(), (hipStream_t)stream));
    return hip_status(pfa::launch_decode(a, desc->head_dim, desc->kv_dtype == PFA_KV_INT8,
                                         (hipStream_t)stream));
}

}  // namespace

pfa_status pfa_paged_attn_decode(const pfa_attn_desc* desc, const pfa_kv_pool* pool, const void* q,
                                 const int32_t* block_table, int32_t bt_stride,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                 int32_t split_keys, int32_t max_splits, float* o_part,
                                 float* lse_part, float* out, void* stream) {
    return decode_like(desc, pool, q, block_table, bt_stride, seq_lens, batch, max_seq_len, split_keys,
                       max_splits, o_part, lse_part, nullptr, out, stream, false);
}

pfa_status pfa_paged_attn_decode_fused(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                                       const void* q, const int32_t* block_table, int32_t bt_stride,
                                       const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                       int32_t split_keys, int32_t max_splits, float* o_part,
                                       float* lse_part, int32_t* counters, float* out, void* stream) {
    return decode_like(desc, pool, q, block_table, bt_stride, seq_lens, batch, max_seq_len, split_keys,
                       max_splits, o_part, lse_part, counters, out, stream, true);
}

pfa_status pfa_paged_attn_decode_static(const pfa_attn_desc* desc, const pfa_kv_pool* pool,
                                        const void* q, const int32_t* block_table, int32_t bt_stride,
                                        const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                        int32_t split_keys, float* out, void* stream) {
    PFA_TRY(check_desc(desc));
    PFA_TRY(check_scale(desc));
    if (split_keys < 0 || batch < 0 || max_seq_len < 0) return PFA_ERR_SHAPE;
    const int32_t ms = split_keys == 0 ? 1 : pfa_decode_num_splits(max_seq_len, split_keys);
    const size_t o_bytes = (size_t)batch * desc->num_q_heads * ms * desc->head_dim * sizeof(float);
    const size_t lse_off = (o_bytes + 255) / 256 * 256;
    const size_t need = lse_off + (size_t)batch * desc->num_q_heads * ms * sizeof(float);
    if (ms > 1 && need > kStaticScratchBytes) return PFA_ERR_WORKSPACE;
    if (ms == 1 || batch == 0)   // unsplit: the kernel writes out directly, no partials
        return decode_like(desc, pool, q, block_table, bt_stride, seq_lens, batch, max_seq_len, 0, 1,
                           nullptr, nullptr, nullptr, out, stream, false);
    if (!out) return PFA_ERR_NULL;
    void* base = nullptr;
    PFA_TRY(static_scratch(&base));
    float* o_part = static_cast<float*>(base);
    float* lse_part = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + lse_off);
    PFA_TRY(decode_like(desc, pool, q, block_table, bt_stride, seq_lens, batch, max_seq_len, split_keys, ms,
                        o_part, lse_part, nullptr, out, stream, false));
    return pfa_paged_attn_combine(desc, o_part, lse_part, seq_lens, batch, split_keys, ms, out, stream);
}

pfa_status pfa_paged_attn_combine(const pfa_attn_desc* desc, const float* o_part,
                                  const float* lse_part, const int32_t* seq_lens, int32_t batch,
                                  int32_t split_keys, int32_t max_splits, float* out,
                                  void* stream) {
    PFA_TRY(check_desc(desc));
    if (batch < 0 || max_splits < 1 || split_keys <= 0 || split_keys % desc->page_size != 0)
        return PFA_ERR_SHAPE;
    if ((int64_t)batch * desc->num_q_heads > 0x7fffffff) return PFA_ERR_SHAPE;
    if (batch == 0) return PFA_OK;
    if (!o_part || !lse_part || !seq_lens || !out) return PFA_ERR_NULL;
    pfa::CombineArgs a;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.seq_lens = seq_lens;
    a.cu_rows = nullptr;
    a.sinks = desc->sinks;
    a.out = out;
    a.batch = batch;
    a.num_q_heads = desc->num_q_heads;
    a.split_keys = split_keys;
    a.max_splits = max_splits;
    a.rows_per_seq = 0;
    return hip_status(pfa::launch_combine(a, desc->head_dim, (hipStream_t)stream));
}

namespace {

// The prefill and verify entry points share their checks and launch; `split_build`
// selects the 128-row / 32-key kernel build (always for verify, and for prefill in
// split mode).
pfa_status prefill_like(const pfa_attn_desc* desc, const pfa_kv_pool* pool, const void* q,
                        const int32_t* cu_q, const int32_t* block_table, int32_t bt_stride,
                        const int32_t* seq_lens, int32_t batch, int32_t max_q_len,
                        int32_t max_seq_len, int32_t split_keys, int32_t max_splits, float* o_part,
                        float* lse_part, float* out, void* stream, bool split_build) {
    PFA_TRY(check_desc(desc));
    PFA_TRY(check_scale(desc));
    PFA_TRY(check_pool(desc, pool));
    if (desc->kv_dtype == PFA_KV_TQ3) return PFA_ERR_UNSUPPORTED;
    const int g = desc->num_q_heads / desc->num_kv_heads;
    if (!prefill_group_ok(g)) return PFA_ERR_UNSUPPORTED;
    if (batch < 0 || max_q_len < 0 || bt_stride <= 0 || max_seq_len < max_q_len || max_splits < 1)
        return PFA_ERR_SHAPE;
    if (max_seq_len > (int64_t)bt_stride * desc->page_size) return PFA_ERR_SHAPE;
    const int tpb = (split_build ? pfa::kPrefillRowsSplit : pfa::kPrefillRows) / g;
    const int64_t items =
        (int64_t)batch * desc->num_kv_heads * ((max_q_len + tpb - 1) / tpb) * max_splits;
    if (items > 0x7fffffff - 8) return PFA_ERR_SHAPE;
    if ((int64_t)batch * max_q_len * desc->num_q_heads > 0x7fffffff) return PFA_ERR_SHAPE;
    if (max_splits > 1) {
        if (split_keys <= 0 || split_keys % 64 != 0) return PFA_ERR_SHAPE;
        if (max_splits < pfa_decode_num_splits(max_seq_len, split_keys)) return PFA_ERR_WORKSPACE;
    }
    if (batch == 0 || max_q_len == 0) return PFA_OK;
    if (!q || !cu_q || !block_table || !seq_lens || !out) return PFA_ERR_NULL;
    if (max_splits > 1 && (!o_part || !lse_part)) return PFA_ERR_NULL;
    pfa::PrefillArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_pool = static_cast<const uint16_t*>(pool->k_pool);
    a.v_pool = static_cast<const uint16_t*>(pool->v_pool);
    const bool int8 = desc->kv_dtype == PFA_KV_INT8;
    a.k_scale = int8 ? pool->k_scale : nullptr;
    a.v_scale = int8 ? pool->v_scale : nullptr;
    a.k_smooth = int8 ? pool->k_smooth : nullptr;
    a.cu_q = cu_q;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.sinks = desc->sinks;
    a.out = out;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.bt_stride = bt_stride;
    a.batch = batch;
    a.num_pages = pool->num_pages;
    a.num_q_heads = desc->num_q_heads;
    a.num_kv_heads = desc->num_kv_heads;
    a.max_q_len = max_q_len;
    a.window = desc->window;
    a.split_keys = max_splits > 1 ? split_keys : 0;
    a.max_splits = max_splits;
    a.sm_scale = desc->sm_scale;
    PFA_TRY(bounds_word_ptr(&a.err));
    if (!split_build) return hip_status(pfa::launch_prefill(a, desc->head_dim, (hipStream_t)stream));
    PFA_TRY(hip_status(pfa::launch_prefill_split(a, desc->head_dim, (hipStream_t)stream)));
    if (max_splits == 1) return PFA_OK;
    pfa::CombineArgs c;
    c.o_part = o_part;
    c.lse_part = lse_part;
    c.seq_lens = nullptr;
    c.cu_rows = cu_q;
    c.sinks = desc->sinks;
    c.out = out;
    c.batch = batch;
    c.num_q_heads = desc->num_q_heads;
    c.split_keys = split_keys;
    c.max_splits = max_splits;
    c.rows_per_seq = max_q_len;
    return hip_status(pfa::launch_combine(c, desc->head_dim, (hipStream_t)stream));
}

}  // namespace

pfa_status pfa_paged_attn_prefill(const pfa_attn_desc* desc, const pfa_kv_pool* pool, const void* q,
                                  const int32_t* cu_q, const int32_t* block_table,
                                  int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                                  int32_t max_q_len, int32_t max_seq_len, int32_t split_keys,
                                  int32_t max_splits, float* o_part, float* lse_part, float* out,
                                  void* stream) {
    // A short sliding window gives each workgroup a few key tiles at most, so the
    // kernel is its prologue and epilogue: the 128-row build, with more workgroups
    // resident per CU, hides more of that latency.  A chunk whose 256-row tiles
    // would leave CUs idle also takes the 128-row build, with twice the
    // workgroups (fresh prompts of 512 and 1024 tokens: 22.3 -> 19.3 us and
    // 35.9 -> 32.4 us; 2048 tokens, 256 workgroups either way, unchanged).
    const bool short_window = desc && desc->window > 0 && desc->window <= 512;
    bool few_tiles = false;
    if (desc && desc->num_kv_heads > 0 && desc->num_q_heads % desc->num_kv_heads == 0) {
        const int g = desc->num_q_heads / desc->num_kv_heads;
        if (prefill_group_ok(g)) {
            const int tpb = pfa::kPrefillRows / g;
            few_tiles = (int64_t)batch * desc->num_kv_heads * ((max_q_len + tpb - 1) / tpb) < 256;
        }
    }
    return prefill_like(desc, pool, q, cu_q, block_table, bt_stride, seq_lens, batch, max_q_len,
                        max_seq_len, split_keys, max_splits, o_part, lse_part, out, stream,
                        max_splits > 1 || short_window || few_tiles);
}

pfa_status pfa_paged_attn_verify(const pfa_attn_desc* desc, const pfa_kv_pool* pool, const void* q,
                                 const int32_t* cu_q, const int32_t* block_table,
                                 int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                                 int32_t max_q_len, int32_t max_seq_len, int32_t split_keys,
                                 int32_t max_splits, float* o_part, float* lse_part, float* out,
                                 void* stream) {
    if (max_q_len > 16) return PFA_ERR_SHAPE;
    return prefill_like(desc, pool, q, cu_q, block_table, bt_stride, seq_lens, batch, max_q_len,
                        max_seq_len, split_keys, max_splits, o_part, lse_part, out, stream, true);
}

int32_t pfa_verify_num_splits(const pfa_attn_desc* desc, int32_t batch, int32_t max_q_len,
                              int32_t max_seq_len, int32_t num_cus, int32_t* split_keys) {
    if (split_keys) *split_keys = 0;
    if (!desc || desc->num_kv_heads <= 0 || desc->num_q_heads % desc->num_kv_heads != 0) return 1;
    const int g = desc->num_q_heads / desc->num_kv_heads;
    if (!prefill_group_ok(g) || batch <= 0 || max_q_len <= 0 || max_seq_len <= 0) return 1;
    if (num_cus <= 0) num_cus = 256;
    const int tps = pfa::kPrefillRowsSplit / g;
    const int64_t items = (int64_t)batch * desc->num_kv_heads * ((max_q_len + tps - 1) / tps);
    const int64_t target = 2 * (int64_t)num_cus;
    if (items >= target || max_seq_len <= 64) return 1;
    const int64_t want = (target + items - 1) / items;
    int64_t sk = (max_seq_len + want - 1) / want;
    sk = std::max<int64_t>(64, (sk + 63) / 64 * 64);
    const int64_t ns = (max_seq_len + sk - 1) / sk;
    if (ns <= 1) return 1;
    if (split_keys) *split_keys = (int32_t)sk;
    return (int32_t)ns;
}

int32_t pfa_prefill_num_splits(const pfa_attn_desc* desc, int32_t batch, int32_t max_q_len,
                               int32_t max_seq_len, int32_t num_cus, int32_t* split_keys) {
    if (split_keys) *split_keys = 0;
    if (!desc || desc->num_kv_heads <= 0 || desc->num_q_heads % desc->num_kv_heads != 0) return 1;
    const int g = desc->num_q_heads / desc->num_kv_heads;
    if (!prefill_group_ok(g) || batch <= 0 || max_q_len <= 0 || max_seq_len <= 0) return 1;
    if (num_cus <= 0) num_cus = 256;
    const int tpb = pfa::kPrefillRows / g;
    const int64_t items = (int64_t)batch * desc->num_kv_heads * ((max_q_len + tpb - 1) / tpb);
    const int64_t target = 2 * (int64_t)num_cus;
    // keys a row of the chunk sees at most: the window, else the whole sequence
    const int64_t span = desc->window > 0 ? std::min<int64_t>(max_seq_len, desc->window + max_q_len)
                                          : max_seq_len;
    // A chunk on little or no cached prefix is a causal triangle: unsplit, its
    // tiles' work ranges from one tile to the whole chunk, and splitting it (more
    // workgroups plus the partials' write, read and merge) measured slower at
    // every prompt length tried (fresh prompts of 512 and 1024 tokens: 22.6 vs
    // 24.8 us and 37.6 vs 43.9 us).  A chunk on a long prefix is where it pays.
    if (items >= target || span <= 256 || (int64_t)max_seq_len - max_q_len < max_q_len / 2) return 1;
    // the split kernel's workgroups hold kPrefillRowsSplit rows, two per CU
    const int tps = pfa::kPrefillRowsSplit / g;
    const int64_t items_s = (int64_t)batch * desc->num_kv_heads * ((max_q_len + tps - 1) / tps);
    const int64_t target_s = target;
    int64_t want = (target_s + items_s - 1) / items_s;
    int64_t sk = (max_seq_len + want - 1) / want;
    sk = std::max<int64_t>(256, (sk + 63) / 64 * 64);
    const int64_t ns = (max_seq_len + sk - 1) / sk;
    if (ns <= 1) return 1;
    if (split_keys) *split_keys = (int32_t)sk;
    return (int32_t)ns;
}

const char* pfa_status_string(pfa_status s) {
    switch (s) {
        case PFA_OK: return "ok";
        case PFA_ERR_NULL: return "a required pointer is NULL";
        case PFA_ERR_SHAPE: return "sizes inconsistent or out of range";
        case PFA_ERR_UNSUPPORTED: return "shape or dtype not supported by the library";
        case PFA_ERR_WORKSPACE: return "split buffers too small (max_splits < ceil(max_seq_len/split_keys))";
        case PFA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

int32_t pfa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

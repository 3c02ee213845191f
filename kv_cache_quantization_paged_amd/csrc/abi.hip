// abi.hip - the extern "C" boundary: argument checks, then one launch
// sequence on the caller's stream. Every check runs before anything is
// queued, so a rejected call has no effect. Tensor values are not read on the
// host (that would need a synchronization); see include/kvfp4.h.
#include <math.h>
#include <string.h>

#include "kvfp4_internal.h"

using namespace kvfp4;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned16(int64_t v) { return (v & 15) == 0; }

// host-side E4M3 decode, used only to check that a recipe clamp is an E4M3 value
float e4m3_value_host(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 0)
        return (float)m * 0x1p-9f;
    return ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
}

bool is_finite_e4m3_value(float v)
{
    for (uint32_t b = 0; b < 0x7F; ++b)
        if (e4m3_value_host(b) == v)
            return true;
    return false;
}

kvfp4_status_t check_cache(const kvfp4_paged_cache_t *c)
{
    if (!c || !c->k_data || !c->v_data || !c->k_sf || !c->v_sf)
        return KVFP4_EINVAL;
    if (c->num_pages <= 0 || c->page_size <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
        return KVFP4_EINVAL;
    if (c->head_dim % 16 != 0)
        return KVFP4_EINVAL;
    if (c->layout != KVFP4_NHD && c->layout != KVFP4_HND)
        return KVFP4_EINVAL;
    const int64_t elems = (int64_t)c->page_size * c->num_kv_heads * c->head_dim;
    if (elems > (int64_t)1 << 30)
        return KVFP4_EINVAL;
    if (c->k_page_stride < elems / 2 || c->v_page_stride < elems / 2)
        return KVFP4_EINVAL;
    if (c->k_sf_page_stride < elems / 16 || c->v_sf_page_stride < elems / 16)
        return KVFP4_EINVAL;
    if (!aligned16(c->k_data) || !aligned16(c->v_data) || !aligned16(c->k_page_stride) ||
        !aligned16(c->v_page_stride))
        return KVFP4_EALIGN;
    return KVFP4_OK;
}

kvfp4_status_t from_hip(hipError_t e) { return e == hipSuccess ? KVFP4_OK : KVFP4_ELAUNCH; }

kvfp4_status_t check_recipe(const kvfp4_recipe_t *recipe)
{
    if (!recipe)
        return KVFP4_OK;
    if (!(recipe->e4m3_max > 0.0f && recipe->e4m3_max <= 448.0f) || !is_finite_e4m3_value(recipe->e4m3_max))
        return KVFP4_EINVAL;
    if (recipe->err_mode != KVFP4_ERR_MSE && recipe->err_mode != KVFP4_ERR_MAE)
        return KVFP4_EINVAL;
    return KVFP4_OK;
}

constexpr int64_t kMaxBlocks = ((int64_t)1 << 31) - 1;   // blocks of 16 per quantize call and tensor

}  // namespace

extern "C" {

}  // extern "C"

// ---------------------------------------------------------------------------
// prepared calls: a *_prepare function runs every check of its entry point and
// stores the checked arguments in the caller's kvfp4_call_t; kvfp4_launch then
// only launches. The seal (a hash over the stored record) lets kvfp4_launch
// refuse a record that no prepare call wrote or that was changed since.
// ---------------------------------------------------------------------------
namespace {

enum : uint32_t { kOpAppend = 1, kOpDequant = 2, kOpMaterialize = 3, kOpAppendDequant = 4 };

struct AppendRec {
    kvfp4_paged_cache_t cache;
    const void *key, *value;
    int64_t nnz;
    const int32_t *batch_indices, *positions, *kv_indices, *kv_indptr;
    float k_scale, v_scale;
    int32_t bf16, has_recipe;
    kvfp4_recipe_t recipe;
};

struct DequantRec {
    kvfp4_paged_cache_t cache;
    const void *block_tables;
    int64_t bt_row_stride;
    const int32_t *seq_lens;
    const float *k_scale, *v_scale;
    void *out_k, *out_v;
    int32_t bt64, batch, out_bf16, max_seq_len;
};

struct MaterializeRec {
    kvfp4_paged_cache_t cache;
    const int32_t *block_tables;
    int64_t bt_row_stride, bt_kv_stride;
    const int32_t *seq_lens, *kv_page_indptr;
    void *out;
    int64_t num_out_pages;
    int32_t *fp8_block_tables;
    int32_t interleaved, shared, batch, max_pages_per_seq;
};

// the append and the dequantize of one decode step over one cache
struct AppendDequantRec {
    kvfp4_paged_cache_t cache;
    const void *key, *value;
    int64_t nnz;
    const int32_t *batch_indices, *positions, *kv_indices, *kv_indptr;
    float k_scale, v_scale;
    int32_t in_bf16, has_recipe;
    kvfp4_recipe_t recipe;
    const void *block_tables;
    int64_t bt_row_stride;
    const int32_t *seq_lens;
    const float *dq_k_scale, *dq_v_scale;
    void *out_k, *out_v;
    int32_t bt64, batch, out_bf16, max_seq_len;
};

struct CallRec {
    uint64_t seal;
    uint32_t op;
    uint32_t nothing_to_do;      // checks passed, but the call queues no work
    union {
        AppendRec append;
        DequantRec dequant;
        MaterializeRec materialize;
        AppendDequantRec append_dequant;
    } u;
};
static_assert(sizeof(CallRec) <= sizeof(kvfp4_call_t), "kvfp4_call_t is too small for the call records");
static_assert(alignof(kvfp4_call_t) >= alignof(CallRec), "kvfp4_call_t alignment");

// FNV-1a over the whole kvfp4_call_t after the seal (unused tail bytes
// included, so that no byte can change unnoticed), mixed with a library constant
uint64_t seal_of(const CallRec *r)
{
    const unsigned char *p = (const unsigned char *)r + sizeof(uint64_t);
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < sizeof(kvfp4_call_t) - sizeof(uint64_t); ++i) {
        h ^= p[i];
        h *= 0x100000001b3ull;
    }
    return h ^ 0x6b76667034ull;
}

CallRec *begin(kvfp4_call_t *call, uint32_t op)
{
    memset(call, 0, sizeof(*call));        // padding bytes too: the seal covers them
    CallRec *r = (CallRec *)call;
    r->op = op;
    return r;
}

kvfp4_status_t finish(CallRec *r, kvfp4_status_t s)
{
    if (s == KVFP4_OK)
        r->seal = seal_of(r);
    else
        memset(r, 0, sizeof(kvfp4_call_t));  // a failed prepare leaves a record no launch accepts
    return s;
}

kvfp4_status_t prepare_append(CallRec *r, const kvfp4_paged_cache_t *cache, const void *append_key,
                              const void *append_value, int32_t in_dtype, int64_t nnz, const int32_t *batch_indices,
                              const int32_t *positions, const int32_t *kv_indices, const int32_t *kv_indptr,
                              const int32_t *kv_last_page_len, int32_t batch_size, float k_scale, float v_scale,
                              const kvfp4_recipe_t *recipe)
{
    kvfp4_status_t s = check_cache(cache);
    if (s != KVFP4_OK)
        return s;
    if (in_dtype != KVFP4_F16 && in_dtype != KVFP4_BF16)
        return KVFP4_EINVAL;
    if (nnz < 0 || batch_size < 0)
        return KVFP4_EINVAL;
    if (!(k_scale > 0.0f) || !isfinite(k_scale) || !(v_scale > 0.0f) || !isfinite(v_scale))
        return KVFP4_EINVAL;
    s = check_recipe(recipe);
    if (s != KVFP4_OK)
        return s;
    if (nnz == 0) {
        r->nothing_to_do = 1;
        return KVFP4_OK;
    }
    if (batch_size == 0 || !append_key || !append_value || !batch_indices || !positions || !kv_indices ||
        !kv_indptr || !kv_last_page_len)
        return KVFP4_EINVAL;
    if (!aligned16(append_key) || !aligned16(append_value))
        return KVFP4_EALIGN;
    AppendRec &a = r->u.append;
    a.cache = *cache;
    a.key = append_key;
    a.value = append_value;
    a.nnz = nnz;
    a.batch_indices = batch_indices;
    a.positions = positions;
    a.kv_indices = kv_indices;
    a.kv_indptr = kv_indptr;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.bf16 = in_dtype == KVFP4_BF16;
    a.has_recipe = recipe != nullptr;
    if (recipe)
        a.recipe = *recipe;
    return KVFP4_OK;
}

kvfp4_status_t prepare_dequant(CallRec *r, const kvfp4_paged_cache_t *cache, const void *block_tables,
                               int32_t bt_dtype, int64_t bt_row_stride, int32_t bt_cols, const int32_t *seq_lens,
                               int32_t batch_size, const float *k_scale, const float *v_scale, void *output_k,
                               void *output_v, int32_t out_dtype, int32_t max_seq_len)
{
    kvfp4_status_t s = check_cache(cache);
    if (s != KVFP4_OK)
        return s;
    if (bt_dtype != KVFP4_I32 && bt_dtype != KVFP4_I64)
        return KVFP4_EINVAL;
    if (out_dtype != KVFP4_F16 && out_dtype != KVFP4_BF16)
        return KVFP4_EINVAL;
    if (batch_size < 0 || max_seq_len < 0 || bt_cols < 0 || bt_row_stride < bt_cols)
        return KVFP4_EINVAL;
    if (batch_size == 0 || max_seq_len == 0) {
        r->nothing_to_do = 1;
        return KVFP4_OK;
    }
    // each row needs ceil(min(seq_len, max_seq_len) / page_size) columns: a value, not checked
    if (bt_cols < 1 || !block_tables || !seq_lens || !k_scale || !v_scale || !output_k || !output_v)
        return KVFP4_EINVAL;
    if (!aligned16(output_k) || !aligned16(output_v))
        return KVFP4_EALIGN;
    DequantRec &d = r->u.dequant;
    d.cache = *cache;
    d.block_tables = block_tables;
    d.bt_row_stride = bt_row_stride;
    d.seq_lens = seq_lens;
    d.k_scale = k_scale;
    d.v_scale = v_scale;
    d.out_k = output_k;
    d.out_v = output_v;
    d.bt64 = bt_dtype == KVFP4_I64;
    d.batch = batch_size;
    d.out_bf16 = out_dtype == KVFP4_BF16;
    d.max_seq_len = max_seq_len;
    return KVFP4_OK;
}

kvfp4_status_t prepare_materialize(CallRec *r, const kvfp4_paged_cache_t *cache, int32_t v_sf_interleaved,
                                   const int32_t *block_tables, int32_t uses_shared_paged_kv_idx,
                                   int64_t bt_row_stride, int64_t bt_kv_stride, int32_t bt_cols,
                                   const int32_t *seq_lens, const int32_t *kv_page_indptr, int32_t batch_size,
                                   void *out_fp8, int64_t num_out_pages, int32_t *fp8_block_tables,
                                   int32_t max_pages_per_seq)
{
    kvfp4_status_t s = check_cache(cache);
    if (s != KVFP4_OK)
        return s;
    if (cache->layout != KVFP4_HND || cache->page_size % 4 != 0 || cache->head_dim % 64 != 0)
        return KVFP4_EINVAL;
    if (batch_size < 0 || num_out_pages < 1 || !out_fp8 || max_pages_per_seq < 0)
        return KVFP4_EINVAL;
    if (!aligned16(out_fp8))
        return KVFP4_EALIGN;
    if (batch_size > 0) {
        if (!block_tables || !seq_lens || !kv_page_indptr || !fp8_block_tables)
            return KVFP4_EINVAL;
        if (bt_cols < max_pages_per_seq)
            return KVFP4_EINVAL;
        if (uses_shared_paged_kv_idx) {
            if (bt_row_stride < bt_cols)
                return KVFP4_EINVAL;
        } else if (bt_kv_stride < bt_cols || bt_row_stride < bt_kv_stride + bt_cols) {
            return KVFP4_EINVAL;
        }
    }
    MaterializeRec &m = r->u.materialize;
    m.cache = *cache;
    m.block_tables = block_tables;
    m.bt_row_stride = bt_row_stride;
    m.bt_kv_stride = bt_kv_stride;
    m.seq_lens = seq_lens;
    m.kv_page_indptr = kv_page_indptr;
    m.out = out_fp8;
    m.num_out_pages = num_out_pages;
    m.fp8_block_tables = fp8_block_tables;
    m.interleaved = v_sf_interleaved != 0;
    m.shared = uses_shared_paged_kv_idx != 0;
    m.batch = batch_size;
    m.max_pages_per_seq = max_pages_per_seq;
    return KVFP4_OK;
}

// both calls' checks, exactly as each entry point runs them, plus one row per
// request (nnz == batch_size)
kvfp4_status_t prepare_append_dequant(CallRec *r, const kvfp4_paged_cache_t *cache, const void *append_key,
                                      const void *append_value, int32_t in_dtype, int64_t nnz,
                                      const int32_t *batch_indices, const int32_t *positions,
                                      const int32_t *kv_indices, const int32_t *kv_indptr,
                                      const int32_t *kv_last_page_len, float k_scale, float v_scale,
                                      const kvfp4_recipe_t *recipe, const void *block_tables, int32_t bt_dtype,
                                      int64_t bt_row_stride, int32_t bt_cols, const int32_t *seq_lens,
                                      int32_t batch_size, const float *dq_k_scale, const float *dq_v_scale,
                                      void *output_k, void *output_v, int32_t out_dtype, int32_t max_seq_len)
{
    CallRec ra, rd;
    memset(&ra, 0, sizeof(ra));
    memset(&rd, 0, sizeof(rd));
    kvfp4_status_t s = prepare_append(&ra, cache, append_key, append_value, in_dtype, nnz, batch_indices, positions,
                                      kv_indices, kv_indptr, kv_last_page_len, batch_size, k_scale, v_scale, recipe);
    if (s != KVFP4_OK)
        return s;
    s = prepare_dequant(&rd, cache, block_tables, bt_dtype, bt_row_stride, bt_cols, seq_lens, batch_size, dq_k_scale,
                        dq_v_scale, output_k, output_v, out_dtype, max_seq_len);
    if (s != KVFP4_OK)
        return s;
    if (nnz != batch_size)
        return KVFP4_EINVAL;
    if (ra.nothing_to_do && rd.nothing_to_do) {
        r->nothing_to_do = 1;
        return KVFP4_OK;
    }
    AppendDequantRec &x = r->u.append_dequant;
    x.cache = *cache;
    x.key = append_key;
    x.value = append_value;
    x.nnz = nnz;
    x.batch_indices = batch_indices;
    x.positions = positions;
    x.kv_indices = kv_indices;
    x.kv_indptr = kv_indptr;
    x.k_scale = k_scale;
    x.v_scale = v_scale;
    x.in_bf16 = in_dtype == KVFP4_BF16;
    x.has_recipe = recipe != nullptr;
    if (recipe)
        x.recipe = *recipe;
    x.block_tables = block_tables;
    x.bt_row_stride = bt_row_stride;
    x.seq_lens = seq_lens;
    x.dq_k_scale = dq_k_scale;
    x.dq_v_scale = dq_v_scale;
    x.out_k = output_k;
    x.out_v = output_v;
    x.bt64 = bt_dtype == KVFP4_I64;
    x.batch = batch_size;
    x.out_bf16 = out_dtype == KVFP4_BF16;
    x.max_seq_len = rd.nothing_to_do ? 0 : max_seq_len;
    return KVFP4_OK;
}

kvfp4_status_t launch_rec(const CallRec *r, hipStream_t st)
{
    if (r->nothing_to_do)
        return KVFP4_OK;
    switch (r->op) {
    case kOpAppend: {
        const AppendRec &a = r->u.append;
        return from_hip(launch_quantize_append(a.cache, a.key, a.value, a.bf16 != 0, a.nnz, a.batch_indices,
                                               a.positions, a.kv_indices, a.kv_indptr, a.k_scale, a.v_scale,
                                               a.has_recipe ? &a.recipe : nullptr, st));
    }
    case kOpDequant: {
        const DequantRec &d = r->u.dequant;
        return from_hip(launch_dequantize_paged(d.cache, d.block_tables, d.bt64 != 0, d.bt_row_stride, d.seq_lens,
                                                d.batch, d.k_scale, d.v_scale, d.out_k, d.out_v, d.out_bf16 != 0,
                                                d.max_seq_len, st));
    }
    case kOpMaterialize: {
        const MaterializeRec &m = r->u.materialize;
        return from_hip(launch_materialize_fp8(m.cache, m.interleaved != 0, m.block_tables, m.shared != 0,
                                               m.bt_row_stride, m.bt_kv_stride, m.seq_lens, m.kv_page_indptr,
                                               m.batch, m.out, m.num_out_pages, m.fp8_block_tables,
                                               m.max_pages_per_seq, st));
    }
    case kOpAppendDequant: {
        const AppendDequantRec &x = r->u.append_dequant;
        return from_hip(launch_append_dequantize_paged(
            x.cache, x.key, x.value, x.in_bf16 != 0, x.nnz, x.batch_indices, x.positions, x.kv_indices, x.kv_indptr,
            x.k_scale, x.v_scale, x.has_recipe ? &x.recipe : nullptr, x.block_tables, x.bt64 != 0, x.bt_row_stride,
            x.seq_lens, x.batch, x.dq_k_scale, x.dq_v_scale, x.out_k, x.out_v, x.out_bf16 != 0, x.max_seq_len, st));
    }
    default:
        return KVFP4_EINVAL;
    }
}

}  // namespace

extern "C" {

kvfp4_status_t kv_quantize_append_prepare(kvfp4_call_t *call, const kvfp4_paged_cache_t *cache,
                                          const void *append_key, const void *append_value, int32_t in_dtype,
                                          int64_t nnz, const int32_t *batch_indices, const int32_t *positions,
                                          const int32_t *kv_indices, const int32_t *kv_indptr,
                                          const int32_t *kv_last_page_len, int32_t batch_size, float k_scale,
                                          float v_scale, const kvfp4_recipe_t *recipe)
{
    if (!call)
        return KVFP4_EINVAL;
    CallRec *r = begin(call, kOpAppend);
    return finish(r, prepare_append(r, cache, append_key, append_value, in_dtype, nnz, batch_indices, positions,
                                    kv_indices, kv_indptr, kv_last_page_len, batch_size, k_scale, v_scale, recipe));
}

kvfp4_status_t kv_dequantize_paged_prepare(kvfp4_call_t *call, const kvfp4_paged_cache_t *cache,
                                           const void *block_tables, int32_t bt_dtype, int64_t bt_row_stride,
                                           int32_t bt_cols, const int32_t *seq_lens, int32_t batch_size,
                                           const float *k_scale, const float *v_scale, void *output_k,
                                           void *output_v, int32_t out_dtype, int32_t max_seq_len)
{
    if (!call)
        return KVFP4_EINVAL;
    CallRec *r = begin(call, kOpDequant);
    return finish(r, prepare_dequant(r, cache, block_tables, bt_dtype, bt_row_stride, bt_cols, seq_lens, batch_size,
                                     k_scale, v_scale, output_k, output_v, out_dtype, max_seq_len));
}

kvfp4_status_t kv_materialize_fp8_prepare(kvfp4_call_t *call, const kvfp4_paged_cache_t *cache,
                                          int32_t v_sf_interleaved, const int32_t *block_tables,
                                          int32_t uses_shared_paged_kv_idx, int64_t bt_row_stride,
                                          int64_t bt_kv_stride, int32_t bt_cols, const int32_t *seq_lens,
                                          const int32_t *kv_page_indptr, int32_t batch_size, void *out_fp8,
                                          int64_t num_out_pages, int32_t *fp8_block_tables,
                                          int32_t max_pages_per_seq)
{
    if (!call)
        return KVFP4_EINVAL;
    CallRec *r = begin(call, kOpMaterialize);
    return finish(r, prepare_materialize(r, cache, v_sf_interleaved, block_tables, uses_shared_paged_kv_idx,
                                         bt_row_stride, bt_kv_stride, bt_cols, seq_lens, kv_page_indptr, batch_size,
                                         out_fp8, num_out_pages, fp8_block_tables, max_pages_per_seq));
}

kvfp4_status_t kv_append_dequantize_paged_prepare(
    kvfp4_call_t *call, const kvfp4_paged_cache_t *cache, const void *append_key, const void *append_value,
    int32_t in_dtype, int64_t nnz, const int32_t *batch_indices, const int32_t *positions, const int32_t *kv_indices,
    const int32_t *kv_indptr, const int32_t *kv_last_page_len, float k_scale, float v_scale,
    const kvfp4_recipe_t *recipe, const void *block_tables, int32_t bt_dtype, int64_t bt_row_stride, int32_t bt_cols,
    const int32_t *seq_lens, int32_t batch_size, const float *dequant_k_scale, const float *dequant_v_scale,
    void *output_k, void *output_v, int32_t out_dtype, int32_t max_seq_len)
{
    if (!call)
        return KVFP4_EINVAL;
    CallRec *r = begin(call, kOpAppendDequant);
    return finish(r, prepare_append_dequant(r, cache, append_key, append_value, in_dtype, nnz, batch_indices,
                                            positions, kv_indices, kv_indptr, kv_last_page_len, k_scale, v_scale,
                                            recipe, block_tables, bt_dtype, bt_row_stride, bt_cols, seq_lens,
                                            batch_size, dequant_k_scale, dequant_v_scale, output_k, output_v,
                                            out_dtype, max_seq_len));
}

kvfp4_status_t kvfp4_launch(const kvfp4_call_t *call, void *stream)
{
    if (!call)
        return KVFP4_EINVAL;
    const CallRec *r = (const CallRec *)call;
    if (r->op == 0 || r->seal != seal_of(r))
        return KVFP4_EINVAL;
    return launch_rec(r, (hipStream_t)stream);
}

kvfp4_status_t kv_quantize_append(const kvfp4_paged_cache_t *cache, const void *append_key,
                                  const void *append_value, int32_t in_dtype, int64_t nnz,
                                  const int32_t *batch_indices, const int32_t *positions,
                                  const int32_t *kv_indices, const int32_t *kv_indptr,
                                  const int32_t *kv_last_page_len, int32_t batch_size, float k_scale,
                                  float v_scale, const kvfp4_recipe_t *recipe, void *stream)
{
    kvfp4_call_t call;
    CallRec *r = begin(&call, kOpAppend);
    const kvfp4_status_t s = prepare_append(r, cache, append_key, append_value, in_dtype, nnz, batch_indices,
                                            positions, kv_indices, kv_indptr, kv_last_page_len, batch_size, k_scale,
                                            v_scale, recipe);
    return s != KVFP4_OK ? s : launch_rec(r, (hipStream_t)stream);
}

kvfp4_status_t kv_dequantize_paged(const kvfp4_paged_cache_t *cache, const void *block_tables, int32_t bt_dtype,
                                   int64_t bt_row_stride, int32_t bt_cols, const int32_t *seq_lens,
                                   int32_t batch_size, const float *k_scale, const float *v_scale,
                                   void *output_k, void *output_v, int32_t out_dtype, int32_t max_seq_len,
                                   void *stream)
{
    kvfp4_call_t call;
    CallRec *r = begin(&call, kOpDequant);
    const kvfp4_status_t s = prepare_dequant(r, cache, block_tables, bt_dtype, bt_row_stride, bt_cols, seq_lens,
                                             batch_size, k_scale, v_scale, output_k, output_v, out_dtype,
                                             max_seq_len);
    return s != KVFP4_OK ? s : launch_rec(r, (hipStream_t)stream);
}

kvfp4_status_t kv_append_dequantize_paged(
    const kvfp4_paged_cache_t *cache, const void *append_key, const void *append_value, int32_t in_dtype, int64_t nnz,
    const int32_t *batch_indices, const int32_t *positions, const int32_t *kv_indices, const int32_t *kv_indptr,
    const int32_t *kv_last_page_len, float k_scale, float v_scale, const kvfp4_recipe_t *recipe,
    const void *block_tables, int32_t bt_dtype, int64_t bt_row_stride, int32_t bt_cols, const int32_t *seq_lens,
    int32_t batch_size, const float *dequant_k_scale, const float *dequant_v_scale, void *output_k, void *output_v,
    int32_t out_dtype, int32_t max_seq_len, void *stream)
{
    kvfp4_call_t call;
    CallRec *r = begin(&call, kOpAppendDequant);
    const kvfp4_status_t s = prepare_append_dequant(
        r, cache, append_key, append_value, in_dtype, nnz, batch_indices, positions, kv_indices, kv_indptr,
        kv_last_page_len, k_scale, v_scale, recipe, block_tables, bt_dtype, bt_row_stride, bt_cols, seq_lens,
        batch_size, dequant_k_scale, dequant_v_scale, output_k, output_v, out_dtype, max_seq_len);
    return s != KVFP4_OK ? s : launch_rec(r, (hipStream_t)stream);
}

kvfp4_status_t kv_materialize_fp8(const kvfp4_paged_cache_t *cache, int32_t v_sf_interleaved,
                                  const int32_t *block_tables, int32_t uses_shared_paged_kv_idx,
                                  int64_t bt_row_stride, int64_t bt_kv_stride, int32_t bt_cols,
                                  const int32_t *seq_lens, const int32_t *kv_page_indptr, int32_t batch_size,
                                  void *out_fp8, int64_t num_out_pages, int32_t *fp8_block_tables,
                                  int32_t max_pages_per_seq, void *stream)
{
    kvfp4_call_t call;
    CallRec *r = begin(&call, kOpMaterialize);
    const kvfp4_status_t s = prepare_materialize(r, cache, v_sf_interleaved, block_tables, uses_shared_paged_kv_idx,
                                                 bt_row_stride, bt_kv_stride, bt_cols, seq_lens, kv_page_indptr,
                                                 batch_size, out_fp8, num_out_pages, fp8_block_tables,
                                                 max_pages_per_seq);
    return s != KVFP4_OK ? s : launch_rec(r, (hipStream_t)stream);
}

kvfp4_status_t kv_global_scale(const void *x, int32_t dtype, int64_t n, float e4m3_max, float *g_out, void *stream)
{
    if (dtype != KVFP4_F16 && dtype != KVFP4_BF16)
        return KVFP4_EINVAL;
    if (n < 0 || !g_out || (n > 0 && !x))
        return KVFP4_EINVAL;
    if (!(e4m3_max > 0.0f && e4m3_max <= 448.0f) || !is_finite_e4m3_value(e4m3_max))
        return KVFP4_EINVAL;
    if (n > 0 && !aligned16(x))
        return KVFP4_EALIGN;
    if (((uintptr_t)g_out & 3u) != 0)
        return KVFP4_EALIGN;
    return from_hip(launch_global_scale(x, dtype == KVFP4_BF16, n, e4m3_max, g_out, (hipStream_t)stream));
}

kvfp4_status_t kv_quantize(const void *input, int32_t in_dtype, int64_t rows, int64_t cols,
                           const float *global_scale, const kvfp4_recipe_t *recipe,
                           void *fp4_data, void *block_scales, void *stream)
{
    if (in_dtype != KVFP4_F16 && in_dtype != KVFP4_BF16)
        return KVFP4_EINVAL;
    if (rows < 0 || cols < 0 || cols % 16 != 0)
        return KVFP4_EINVAL;
    kvfp4_status_t s = check_recipe(recipe);
    if (s != KVFP4_OK)
        return s;
    if (rows == 0 || cols == 0)
        return KVFP4_OK;
    if (!input || !global_scale || !fp4_data || !block_scales)
        return KVFP4_EINVAL;
    if (cols / 16 > kMaxBlocks / rows)
        return KVFP4_EUNSUPPORTED;
    if (!aligned16(input) || !aligned16(fp4_data))
        return KVFP4_EALIGN;
    return from_hip(launch_quantize_contiguous(input, in_dtype == KVFP4_BF16, rows, cols, global_scale, recipe,
                                               fp4_data, block_scales, (hipStream_t)stream));
}

kvfp4_status_t kv_dequantize(const void *fp4_data, const void *block_scales, int64_t rows, int64_t cols,
                             const float *global_scale, void *output, int32_t out_dtype, void *stream)
{
    if (out_dtype != KVFP4_F16 && out_dtype != KVFP4_BF16)
        return KVFP4_EINVAL;
    if (rows < 0 || cols < 0 || cols % 16 != 0)
        return KVFP4_EINVAL;
    if (rows == 0 || cols == 0)
        return KVFP4_OK;
    if (!fp4_data || !block_scales || !global_scale || !output)
        return KVFP4_EINVAL;
    if (cols / 8 > ((int64_t)1 << 40) / rows)
        return KVFP4_EUNSUPPORTED;
    if (!aligned16(fp4_data) || !aligned16(output))
        return KVFP4_EALIGN;
    return from_hip(launch_dequantize_contiguous(fp4_data, block_scales, rows, cols, global_scale, output,
                                                 out_dtype == KVFP4_BF16, (hipStream_t)stream));
}

kvfp4_status_t kv_quantize_paged_cache(const kvfp4_paged_cache_t *cache, const void *k_in, const void *v_in,
                                       int32_t in_dtype, const float *k_scale, const float *v_scale,
                                       const kvfp4_recipe_t *recipe, int32_t v_sf_interleaved, void *stream)
{
    kvfp4_status_t s = check_cache(cache);
    if (s != KVFP4_OK)
        return s;
    if (in_dtype != KVFP4_F16 && in_dtype != KVFP4_BF16)
        return KVFP4_EINVAL;
    s = check_recipe(recipe);
    if (s != KVFP4_OK)
        return s;
    if (v_sf_interleaved && (cache->layout != KVFP4_HND || cache->page_size % 4 != 0))
        return KVFP4_EINVAL;
    if (!k_in || !v_in || !k_scale || !v_scale)
        return KVFP4_EINVAL;
    const int64_t blocks_per_page = (int64_t)cache->page_size * cache->num_kv_heads * (cache->head_dim / 16);
    if (blocks_per_page > kMaxBlocks / cache->num_pages)
        return KVFP4_EUNSUPPORTED;
    if (!aligned16(k_in) || !aligned16(v_in))
        return KVFP4_EALIGN;
    return from_hip(launch_quantize_paged_cache(*cache, k_in, v_in, in_dtype == KVFP4_BF16, k_scale, v_scale,
                                                recipe, v_sf_interleaved != 0, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// the checks kv_decode_attention and kv_decode_attention_noalloc share (all
// but the workspace); KVFP4_OK with *nothing_to_do set for an empty batch
kvfp4_status_t check_attention(const kvfp4_paged_cache_t *cache, const void *q, int32_t q_dtype,
                               int32_t num_qo_heads, const int32_t *block_tables, int64_t bt_row_stride,
                               int32_t bt_cols, const int32_t *seq_lens, int32_t batch_size, const float *k_scale,
                               const float *v_scale, float sm_scale, const void *out, bool *nothing_to_do)
{
    *nothing_to_do = false;
    kvfp4_status_t s = check_cache(cache);
    if (s != KVFP4_OK)
        return s;
    if (q_dtype != KVFP4_F16 && q_dtype != KVFP4_BF16)
        return KVFP4_EINVAL;
    if (batch_size < 0 || num_qo_heads <= 0 || num_qo_heads % cache->num_kv_heads != 0)
        return KVFP4_EINVAL;
    if (bt_cols < 0 || bt_row_stride < bt_cols || !isfinite(sm_scale))
        return KVFP4_EINVAL;
    const int D = cache->head_dim;
    if (D != 64 && D != 128 && D != 256)
        return KVFP4_EUNSUPPORTED;
    if (batch_size == 0) {
        *nothing_to_do = true;
        return KVFP4_OK;
    }
    if (!q || !block_tables || !seq_lens || !k_scale || !v_scale || !out || bt_cols < 1)
        return KVFP4_EINVAL;
    if ((int64_t)batch_size * cache->num_kv_heads * decode_attention_splits(bt_cols, cache->page_size) > INT32_MAX)
        return KVFP4_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(out))
        return KVFP4_EALIGN;
    // a lane reads D / 64 K scale bytes of a row at once (head_dim 128: 2,
    // 256: 4)
    const uint64_t sf_align = D >= 128 ? (uint64_t)D / 64 - 1 : 0;
    if ((((uintptr_t)cache->k_sf | (uintptr_t)cache->v_sf) & sf_align) ||
        ((uint64_t)(cache->k_sf_page_stride | cache->v_sf_page_stride) & sf_align))
        return KVFP4_EALIGN;
    return KVFP4_OK;
}

}  // namespace

extern "C" {

kvfp4_status_t kv_decode_attention(const kvfp4_paged_cache_t *cache, const void *q, int32_t q_dtype,
                                   int32_t num_qo_heads, const int32_t *block_tables, int64_t bt_row_stride,
                                   int32_t bt_cols, const int32_t *seq_lens, int32_t batch_size,
                                   const float *k_scale, const float *v_scale, float sm_scale, void *out,
                                   void *workspace, int64_t workspace_bytes, void *stream)
{
    bool empty = false;
    kvfp4_status_t s = check_attention(cache, q, q_dtype, num_qo_heads, block_tables, bt_row_stride, bt_cols,
                                       seq_lens, batch_size, k_scale, v_scale, sm_scale, out, &empty);
    if (s != KVFP4_OK || empty)
        return s;
    if (!workspace)
        return KVFP4_EINVAL;
    if (workspace_bytes < decode_attention_workspace_bytes(batch_size, cache->num_kv_heads, num_qo_heads, bt_cols,
                                                           cache->page_size, cache->head_dim))
        return KVFP4_EINVAL;
    if (!aligned16(workspace))
        return KVFP4_EALIGN;
    return from_hip(launch_decode_attention(*cache, q, q_dtype == KVFP4_BF16, num_qo_heads, block_tables,
                                            bt_row_stride, bt_cols, seq_lens, batch_size, k_scale, v_scale,
                                            sm_scale, out, workspace, (hipStream_t)stream));
}

kvfp4_status_t kv_decode_attention_noalloc(const kvfp4_paged_cache_t *cache, const void *q, int32_t q_dtype,
                                           int32_t num_qo_heads, const int32_t *block_tables,
                                           int64_t bt_row_stride, int32_t bt_cols, const int32_t *seq_lens,
                                           int32_t batch_size, const float *k_scale, const float *v_scale,
                                           float sm_scale, void *out, void *stream)
{
    bool empty = false;
    kvfp4_status_t s = check_attention(cache, q, q_dtype, num_qo_heads, block_tables, bt_row_stride, bt_cols,
                                       seq_lens, batch_size, k_scale, v_scale, sm_scale, out, &empty);
    if (s != KVFP4_OK || empty)
        return s;
    if (decode_attention_workspace_bytes(batch_size, cache->num_kv_heads, num_qo_heads, bt_cols, cache->page_size,
                                         cache->head_dim) > kNoAllocScratchBytes)
        return KVFP4_ESCRATCH;
    void *ws = nullptr;
    hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess)
        return KVFP4_ELAUNCH;
    return from_hip(launch_decode_attention(*cache, q, q_dtype == KVFP4_BF16, num_qo_heads, block_tables,
                                            bt_row_stride, bt_cols, seq_lens, batch_size, k_scale, v_scale,
                                            sm_scale, out, ws, (hipStream_t)stream));
}

int64_t kv_decode_attention_workspace_size(int32_t batch_size, int32_t num_kv_heads, int32_t num_qo_heads,
                                           int32_t bt_cols, int32_t page_size, int32_t head_dim)
{
    if (batch_size < 0 || num_kv_heads <= 0 || num_qo_heads <= 0 || num_qo_heads % num_kv_heads != 0 ||
        bt_cols < 0 || page_size <= 0 || head_dim <= 0)
        return -1;
    return decode_attention_workspace_bytes(batch_size, num_kv_heads, num_qo_heads, bt_cols, page_size, head_dim);
}

const char *kvfp4_status_string(kvfp4_status_t status)
{
    switch (status) {
    case KVFP4_OK: return "ok";
    case KVFP4_EINVAL: return "invalid argument (null pointer, enum, extent, stride or scale)";
    case KVFP4_EALIGN: return "misaligned pointer or stride (16-byte alignment required)";
    case KVFP4_EUNSUPPORTED: return "unsupported request (sizes beyond the library's 32-bit index limits)";
    case KVFP4_ELAUNCH: return "HIP kernel launch failed (is the device gfx950?)";
    case KVFP4_EVALUE: return "a table value is out of range (see the check's report)";
    case KVFP4_ESCRATCH: return "the call needs more than the no-allocation entry point's fixed scratch "
                                "(KVFP4_NOALLOC_SCRATCH_BYTES); use the variant with a caller workspace";
    default: return "unknown status";
    }
}

}  // extern "C"

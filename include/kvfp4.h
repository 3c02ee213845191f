/*
 * kvfp4.h - C ABI of the paged NVFP4 KV-cache library for AMD MI355X (gfx950).
 *
 * Calls, all asynchronous on a caller-given HIP stream:
 *   kv_quantize_append   fp16/bf16 K/V rows -> packed E2M1 + E4M3 block scales
 *                        in paged NHD/HND caches addressed by a CSR page table
 *   kv_dequantize_paged  paged NVFP4 -> contiguous [B, T, H, D] fp16/bf16
 *   kv_append_dequantize_paged  a decode step: both of the above, one launch
 *   kv_materialize_fp8   active pages -> float8_e4m3fn page copy + block table
 *   kv_global_scale      per-tensor global decode scale amax / (6 * e4m3_max)
 *   kv_quantize          contiguous fp16/bf16 -> NVFP4 with linear scales
 *   kv_dequantize        contiguous NVFP4 with linear scales -> fp16/bf16
 *   kv_quantize_paged_cache  a whole 16-bit page pool -> NVFP4 cache, V
 *                        scales optionally 4-token interleaved
 *   kv_decode_attention  one-token-per-request attention read straight
 *                        from the NVFP4 pages
 *   *_prepare + kvfp4_launch  the first four calls checked once, then
 *                        launched many times without re-checking
 *
 * Sources (FlashInfer 0.7.4 documentation): the API pages
 * flashinfer.page.nvfp4_quantize_append_paged_kv_cache,
 * flashinfer.quantization.nvfp4_kv_dequantize_paged and
 * flashinfer.quantization.kernels.nvfp4_kv_materialize.nvfp4_kv_materialize_fp8,
 * and the flashinfer.quantization module page (sections "NVFP4 4over6
 * Recipes", "FP4 KV Cache Quantization", "NVFP4 KV Cache Materialization" with
 * NVFP4KVMaterializer.run()).
 *
 * Formats: E2M1 codes (OCP FP4: sign bit 3, magnitudes 0, .5, 1, 1.5, 2, 3, 4,
 * 6), two per byte, the even element in the low nibble; E4M3 block scales
 * (OCP float8_e4m3fn bytes), one per 16 consecutive elements of head_dim.
 * A decoded value is e2m1 * block_scale * global_scale.
 *
 * Ownership and threading: every buffer pointer is device memory owned by the
 * caller and must stay valid until the work queued on `stream` completes.
 * The library never allocates, frees or synchronizes; it only launches
 * kernels on `stream` (a hipStream_t passed as void*, NULL = the null
 * stream), so every call can be captured in a HIP graph. Calls keep no state
 * between them and may be made from several host threads.
 *
 * Errors: each call returns a status. Every argument check runs before any
 * launch, so a call that returns an error has queued nothing and written
 * nothing. Tensor *values* (page ids, positions, lengths, indptr entries) are
 * not checked, as on the pages; out-of-range values are undefined behaviour.
 * KVFP4_ELAUNCH reports a HIP launch failure (for instance a device that is
 * not gfx950).
 */
#ifndef KVFP4_H
#define KVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvfp4_status_t;
enum {
    KVFP4_OK = 0,
    KVFP4_EINVAL = 1,        /* null pointer, bad enum, bad extent or scale */
    KVFP4_EALIGN = 2,        /* a base pointer or stride is not 16-byte aligned */
    KVFP4_EUNSUPPORTED = 3,  /* a valid request the library does not implement */
    KVFP4_ELAUNCH = 4,       /* the HIP runtime refused a launch */
    KVFP4_ESCRATCH = 5,      /* a no-allocation call needs more than its fixed scratch */
    KVFP4_EVALUE = 6         /* a table check found a value out of range (see the report) */
};

enum { KVFP4_NHD = 0, KVFP4_HND = 1 };                /* cache layouts */
enum { KVFP4_F16 = 0, KVFP4_BF16 = 1 };               /* 16-bit float types */
enum { KVFP4_I32 = 0, KVFP4_I64 = 1 };                /* block-table index types */
enum { KVFP4_ERR_MSE = 0, KVFP4_ERR_MAE = 1 };        /* 4over6 error metrics */

/*
 * 4over6 block-scale recipe (module page, "NVFP4 4over6 Recipes",
 * NVFP44Over6Config): for every 16-element block the quantizer forms the
 * amax/6 scale (clamped at e4m3_max) and the 1.5x tighter amax/4 scale
 * (clamped at 448), quantizes and dequantizes with both, and keeps amax/4
 * only when its summed error (err_mode: squared or absolute, evaluated in
 * fp32, pairwise tree over the 16 elements) is strictly lower.
 * A NULL recipe pointer selects standard NVFP4: amax/6 clamped at 448.
 *   e4m3_max           a finite E4M3 value in (0, 448]; 256 is the page's knob
 *   err_mode           KVFP4_ERR_MSE or KVFP4_ERR_MAE
 *   err_use_fast_math  nonzero: the error is evaluated in IEEE fp16 (the
 *                      page's distinct "fast math" recipe): the input and the
 *                      fp32 reconstruction rounded to fp16, then the
 *                      difference, the square and every pairwise sum rounded
 *                      to fp16; an inf or NaN error never wins
 */
typedef struct {
    float e4m3_max;
    int32_t err_mode;
    int32_t err_use_fast_math;
} kvfp4_recipe_t;

/*
 * A paged NVFP4 cache (append and dequantize pages: paged_kv_cache and
 * kv_cache_sf, as a tuple or a stacked tensor). Per page, the data holds
 * [page_size, num_kv_heads, head_dim/2] bytes (NHD) or
 * [num_kv_heads, page_size, head_dim/2] (HND), compact inside the page; the
 * scales the same with head_dim/16 bytes per row. Page p of K data starts at
 * k_data + p * k_page_stride, and likewise for the other three. A tuple cache
 * passes two allocations; a stacked 5-D cache [pages, 2, ...] passes
 * v = k + page bytes and strides of twice the page bytes. Strides are in bytes
 * and may exceed the compact page (padded pages). The data bases and data
 * page strides must be multiples of 16 bytes (the launchers on the pages check
 * 16-byte alignment); scale bases and strides have no alignment requirement.
 */
typedef struct {
    void *k_data, *v_data;            /* uint8 packed E2M1 */
    void *k_sf, *v_sf;                /* uint8 E4M3 block scales, linear layout */
    int64_t k_page_stride, v_page_stride;        /* bytes */
    int64_t k_sf_page_stride, v_sf_page_stride;  /* bytes */
    int32_t num_pages;                /* pages addressable through each base */
    int32_t page_size;
    int32_t num_kv_heads;
    int32_t head_dim;                 /* multiple of 16 */
    int32_t layout;                   /* KVFP4_NHD or KVFP4_HND */
} kvfp4_paged_cache_t;

/*
 * kv_quantize_append - nvfp4_quantize_append_paged_kv_cache.
 * Quantizes nnz rows of append_key / append_value ([nnz, num_kv_heads,
 * head_dim] contiguous, in_dtype KVFP4_F16/KVFP4_BF16, 16-byte aligned) and
 * writes them in place into `cache`: row r belongs to request
 * b = batch_indices[r] at logical position p = positions[r]; its page is
 * kv_indices[kv_indptr[b] + p / page_size] and its slot p % page_size.
 * kv_indptr has batch_size + 1 entries, kv_last_page_len batch_size entries
 * (the space must already be reserved, as the page's note requires; the
 * table is not modified). All index arrays are int32 device arrays.
 * k_scale / v_scale are the positive finite global decode scales (host
 * floats). Only the addressed code and scale bytes change. recipe: NULL for
 * standard NVFP4, else a 4over6 recipe (the page lists no recipe argument for
 * this call; every other NVFP4 entry point takes one, so it is accepted here).
 * Rows with equal (b, p) race. nnz == 0 is a no-op.
 * append_key / append_value must be 16-byte aligned.
 */
kvfp4_status_t kv_quantize_append(const kvfp4_paged_cache_t *cache,
                                  const void *append_key, const void *append_value,
                                  int32_t in_dtype, int64_t nnz,
                                  const int32_t *batch_indices, const int32_t *positions,
                                  const int32_t *kv_indices, const int32_t *kv_indptr,
                                  const int32_t *kv_last_page_len, int32_t batch_size,
                                  float k_scale, float v_scale,
                                  const kvfp4_recipe_t *recipe, void *stream);

/*
 * kv_dequantize_paged - nvfp4_kv_dequantize_paged.
 * For every request b < batch_size and position t < min(seq_lens[b],
 * max_seq_len): page = block_tables[b * bt_row_stride + t / page_size]
 * (int32 or int64 per bt_dtype), slot t % page_size, and for every head h and
 * element e: output[b, t, h, e] = RNE_16(fp32(fp32(E4M3(s) * g) * e2m1(c)))
 * with g = *k_scale for output_k and *v_scale for output_v (device fp32
 * scalars). Outputs are caller-owned contiguous [batch_size, max_seq_len,
 * num_kv_heads, head_dim] fp16/bf16 (out_dtype), 16-byte aligned. Positions
 * t >= seq_lens[b] are left unchanged. bt_cols is the number of columns of
 * the table (each row needs ceil(min(seq_len, max_seq_len) / page_size)).
 */
kvfp4_status_t kv_dequantize_paged(const kvfp4_paged_cache_t *cache,
                                   const void *block_tables, int32_t bt_dtype,
                                   int64_t bt_row_stride, int32_t bt_cols,
                                   const int32_t *seq_lens, int32_t batch_size,
                                   const float *k_scale, const float *v_scale,
                                   void *output_k, void *output_v, int32_t out_dtype,
                                   int32_t max_seq_len, void *stream);

/*
 * kv_append_dequantize_paged - one decode step over a paged cache: the
 * nvfp4_quantize_append_paged_kv_cache page's append of each request's newest
 * token, then the nvfp4_kv_dequantize_paged page's dequantize of every
 * request's context, including that token. The arguments are those of
 * kv_quantize_append (cache through k_scale / v_scale / recipe: host global
 * scales for the quantization) followed by those of kv_dequantize_paged
 * (dequant_k_scale / dequant_v_scale: device fp32 scalars for the decode),
 * with one batch_size for both and the same checks, plus nnz == batch_size
 * (KVFP4_EINVAL otherwise). The cache and both outputs end exactly as after
 * kv_quantize_append followed by kv_dequantize_paged on the same stream,
 * provided the values follow the decode-step pattern (not checked, like
 * every value): each request b has exactly one row r (batch_indices[r] ==
 * b), at position positions[r] == seq_lens[b] - 1, and no other request of
 * the call reaches the slot that row writes within its first seq_lens - 1
 * tokens (requests that share pages read them, they do not append to them).
 * For the standard recipe it is one launch, on every layout: the leading
 * workgroups quantize the rows, store them in the cache and write their
 * dequantized values into the outputs straight from the codes they
 * computed, while the others dequantize every request without its newest
 * token, so no workgroup reads a byte another writes. With a 4over6 recipe it
 * queues the two calls' kernels in sequence.
 */
kvfp4_status_t kv_append_dequantize_paged(const kvfp4_paged_cache_t *cache,
                                          const void *append_key, const void *append_value,
                                          int32_t in_dtype, int64_t nnz,
                                          const int32_t *batch_indices, const int32_t *positions,
                                          const int32_t *kv_indices, const int32_t *kv_indptr,
                                          const int32_t *kv_last_page_len,
                                          float k_scale, float v_scale, const kvfp4_recipe_t *recipe,
                                          const void *block_tables, int32_t bt_dtype,
                                          int64_t bt_row_stride, int32_t bt_cols,
                                          const int32_t *seq_lens, int32_t batch_size,
                                          const float *dequant_k_scale, const float *dequant_v_scale,
                                          void *output_k, void *output_v, int32_t out_dtype,
                                          int32_t max_seq_len, void *stream);

/*
 * kv_materialize_fp8 - nvfp4_kv_materialize_fp8 / NVFP4KVMaterializer.run().
 * cache must be HND with page_size % 4 == 0 and head_dim % 64 == 0 (the
 * materializer's constraints); data page strides may exceed the compact
 * page. For every request b and page j < ceil(seq_lens[b] / page_size):
 *   dst = kv_page_indptr[b] + j + 1,
 *   K page = block_tables[b * bt_row_stride + j],
 *   V page = the same entry (uses_shared_paged_kv_idx != 0) or
 *            block_tables[b * bt_row_stride + bt_kv_stride + j],
 *   out[dst, 0 | 1, h, t, e] = E4M3_satfinite(E2M1(c) * E4M3(s)) for the
 *   whole page (all page_size slots), K into half 0 and V into half 1,
 *   fp8_block_tables[b * max_pages_per_seq + j] = dst.
 * Page 0 of out (both halves) is set to zero. Only E2M1 and block scales are
 * multiplied: the global scales belong to the consumer. The product is exact
 * and rounds once to nearest-even, saturating at +-448 with its sign. K
 * scales are linear; V scales are read 4-token interleaved when
 * v_sf_interleaved != 0 (inside a (page, head) tile the scale of token t,
 * block c sits at byte ((t / 4) * (head_dim / 16) + c) * 4 + t % 4), linear
 * otherwise. out is float8_e4m3fn [num_out_pages, 2, num_kv_heads,
 * page_size, head_dim], contiguous, 16-byte aligned, num_out_pages >=
 * kv_page_indptr[batch_size] + 1; pages past kv_page_indptr[batch_size] and
 * pages of a request past its length are neither written nor read, and no
 * other table entry is written (zero the table first if a consumer reads
 * them). Requests must satisfy seq_lens[b] <= max_pages_per_seq * page_size
 * and reserve at least ceil(seq_lens[b] / page_size) pages.
 * block_tables, seq_lens, kv_page_indptr and fp8_block_tables are int32.
 */
kvfp4_status_t kv_materialize_fp8(const kvfp4_paged_cache_t *cache, int32_t v_sf_interleaved,
                                  const int32_t *block_tables, int32_t uses_shared_paged_kv_idx,
                                  int64_t bt_row_stride, int64_t bt_kv_stride, int32_t bt_cols,
                                  const int32_t *seq_lens, const int32_t *kv_page_indptr,
                                  int32_t batch_size, void *out_fp8, int64_t num_out_pages,
                                  int32_t *fp8_block_tables, int32_t max_pages_per_seq,
                                  void *stream);

/*
 * Validate once, launch many (the NVFP4KVMaterializer pattern of the module
 * page's "NVFP4 KV Cache Materialization" section: its functional form checks
 * every tensor on every call, which costs more host time than the launch,
 * so the class checks at construction and run() only launches). A
 * kvfp4_call_t is caller-owned memory. A *_prepare call runs every check of
 * the entry point of the same name, exactly as that entry point does, and
 * on success stores the checked arguments in *call; on failure it returns the
 * same status and leaves a record that kvfp4_launch refuses. kvfp4_launch
 * then queues that call's kernels on `stream` without checking anything
 * again, as often as wanted (each launch reads the buffers' contents at the
 * time it runs: caches, tables and lengths may change between launches, the
 * pointers and sizes may not - prepare again for those). A record that no
 * prepare call wrote, or that was modified since, gives KVFP4_EINVAL (the
 * record carries a seal over its contents). Launches are graph-capturable
 * and, like the entry points, allocate and synchronize nothing.
 */
typedef struct {
    uint64_t opaque[40];
} kvfp4_call_t;

kvfp4_status_t kv_quantize_append_prepare(kvfp4_call_t *call, const kvfp4_paged_cache_t *cache,
                                          const void *append_key, const void *append_value, int32_t in_dtype,
                                          int64_t nnz, const int32_t *batch_indices, const int32_t *positions,
                                          const int32_t *kv_indices, const int32_t *kv_indptr,
                                          const int32_t *kv_last_page_len, int32_t batch_size, float k_scale,
                                          float v_scale, const kvfp4_recipe_t *recipe);

kvfp4_status_t kv_dequantize_paged_prepare(kvfp4_call_t *call, const kvfp4_paged_cache_t *cache,
                                           const void *block_tables, int32_t bt_dtype, int64_t bt_row_stride,
                                           int32_t bt_cols, const int32_t *seq_lens, int32_t batch_size,
                                           const float *k_scale, const float *v_scale, void *output_k,
                                           void *output_v, int32_t out_dtype, int32_t max_seq_len);

kvfp4_status_t kv_materialize_fp8_prepare(kvfp4_call_t *call, const kvfp4_paged_cache_t *cache,
                                          int32_t v_sf_interleaved, const int32_t *block_tables,
                                          int32_t uses_shared_paged_kv_idx, int64_t bt_row_stride,
                                          int64_t bt_kv_stride, int32_t bt_cols, const int32_t *seq_lens,
                                          const int32_t *kv_page_indptr, int32_t batch_size, void *out_fp8,
                                          int64_t num_out_pages, int32_t *fp8_block_tables,
                                          int32_t max_pages_per_seq);

kvfp4_status_t kv_append_dequantize_paged_prepare(kvfp4_call_t *call, const kvfp4_paged_cache_t *cache,
                                                  const void *append_key, const void *append_value,
                                                  int32_t in_dtype, int64_t nnz, const int32_t *batch_indices,
                                                  const int32_t *positions, const int32_t *kv_indices,
                                                  const int32_t *kv_indptr, const int32_t *kv_last_page_len,
                                                  float k_scale, float v_scale, const kvfp4_recipe_t *recipe,
                                                  const void *block_tables, int32_t bt_dtype,
                                                  int64_t bt_row_stride, int32_t bt_cols,
                                                  const int32_t *seq_lens, int32_t batch_size,
                                                  const float *dequant_k_scale, const float *dequant_v_scale,
                                                  void *output_k, void *output_v, int32_t out_dtype,
                                                  int32_t max_seq_len);

kvfp4_status_t kvfp4_launch(const kvfp4_call_t *call, void *stream);

/*
 * kv_global_scale - make_nvfp4_global_scale(x, per_token_activation=False,
 * recipe) (module page, "NVFP4 4over6 Recipes" and its precedence note): the
 * per-tensor global decode scale g = amax|x| / fp32(6 * e4m3_max), one IEEE
 * fp32 division, and 1 for an all-zero tensor. x is n contiguous fp16/bf16
 * values (16-byte aligned); g_out is one device fp32, written in place (it is
 * also used as the running maximum while the call runs). e4m3_max must match
 * the quantizer's recipe: 448 for standard NVFP4, the recipe's value (256)
 * for 4over6 - the page warns that a mismatch silently rescales the tensor.
 */
kvfp4_status_t kv_global_scale(const void *x, int32_t dtype, int64_t n, float e4m3_max,
                               float *g_out, void *stream);

/*
 * kv_quantize - nvfp4_kv_quantize(input, global_scale) (module page, "FP4 KV
 * Cache Quantization": the NVFP4 KV-cache format with the linear block-scale
 * layout). input is [rows, cols] row-major fp16/bf16 (in_dtype), cols a
 * multiple of 16; blocks of 16 run along each row. fp4_data receives
 * [rows, cols/2] packed codes (even element in the low nibble), block_scales
 * [rows, cols/16] E4M3 bytes. global_scale points to one device fp32, the
 * global decode scale g (as make_nvfp4_global_scale returns it). The block
 * arithmetic is the append's: amax / (6 g) clamped at 448, or at the recipe's
 * e4m3_max with the two-candidate 4over6 search (recipe non-NULL). input and
 * fp4_data must be 16-byte aligned; rows * cols / 16 < 2^31. rows == 0 is a
 * no-op.
 */
kvfp4_status_t kv_quantize(const void *input, int32_t in_dtype, int64_t rows, int64_t cols,
                           const float *global_scale, const kvfp4_recipe_t *recipe,
                           void *fp4_data, void *block_scales, void *stream);

/*
 * kv_dequantize - nvfp4_kv_dequantize(fp4_data, block_scales, ...) (module
 * page, "FP4 KV Cache Quantization"): the inverse layout of kv_quantize.
 * out[r, e] = RNE_{f16|bf16}(fp32(fp32(E4M3(s) * g) * e2m1(c))), the paged
 * dequant's arithmetic. fp4_data [rows, cols/2], block_scales [rows, cols/16],
 * output [rows, cols] of out_dtype; global_scale points to one device fp32.
 * fp4_data and output must be 16-byte aligned, cols a multiple of 16.
 */
kvfp4_status_t kv_dequantize(const void *fp4_data, const void *block_scales, int64_t rows, int64_t cols,
                             const float *global_scale, void *output, int32_t out_dtype, void *stream);

/*
 * kv_quantize_paged_cache - nvfp4_quantize_paged_kv_cache(k_cache, v_cache)
 * (module page, "FP4 KV Cache Quantization"; the materialize page names it as
 * the producer of 4-token-interleaved V scales): quantizes every slot of every
 * page of two 16-bit page pools into `cache`. k_in / v_in are contiguous
 * [cache->num_pages, page_size, H, D] (NHD) or [num_pages, H, page_size, D]
 * (HND) fp16/bf16 pools in the cache's layout; page p of the pool lands in
 * page p of the cache (page strides as in the descriptor; padding bytes are
 * not written). k_scale / v_scale point to one device fp32 each (global
 * decode scales, e.g. from kv_global_scale). K scales are written linear; V
 * scales 4-token interleaved when v_sf_interleaved != 0 (HND and
 * page_size % 4 == 0 required), linear otherwise. recipe as for append.
 * k_in, v_in must be 16-byte aligned; num_pages * page_size * H * D / 16 <
 * 2^31.
 */
kvfp4_status_t kv_quantize_paged_cache(const kvfp4_paged_cache_t *cache, const void *k_in, const void *v_in,
                                       int32_t in_dtype, const float *k_scale, const float *v_scale,
                                       const kvfp4_recipe_t *recipe, int32_t v_sf_interleaved, void *stream);

/*
 * kv_decode_attention - the NVFP4 attention consumer of the paged cache
 * (flashinfer.quantization.nvfp4_kv_dequantize_paged page, which names
 * FlashInfer's NVFP4 attention kernels as users of its global decode scales
 * k_scale and v_scale; values e2m1 * block_scale * global_scale). For each request b
 * and query head hq (kv head hq / (num_qo_heads / num_kv_heads)):
 *   out[b, hq, :] = sum_t softmax_t(sm_scale * q[b, hq, :] . K[b, t, h, :]) V[b, t, h, :]
 * over t < seq_lens[b], K and V decoded from the cache (page
 * block_tables[b * bt_row_stride + t / page_size], slot t % page_size) times
 * *k_scale / *v_scale (device fp32). A request of length 0 gives zeros.
 * Lengths are values and are not checked on the host; the kernels cut a
 * length to the bt_cols * page_size tokens its table row addresses and treat
 * a negative one as 0, so no access leaves the caller's buffers and a bad
 * length changes only its own request's output.
 * q and out are [batch_size, num_qo_heads, head_dim] of q_dtype (bf16 or
 * fp16), contiguous, 16-byte aligned; block_tables and seq_lens int32.
 * head_dim must be 64, 128 or 256 (KVFP4_EUNSUPPORTED otherwise); any number
 * of query heads per kv head (beyond 16 they run in passes of 16, each
 * reading the cache again); scale bases and scale page strides must be
 * even for head_dim 128 and multiples of 4 for head_dim 256. Scores and the
 * softmax are fp32. The products run in fp16: decoded
 * K and V are exact there; a bf16 query row is scaled by a power of two that
 * puts its largest magnitude in [2^14, 2^15) and converted (exact except for
 * components more than 2^38 below that largest one); the probabilities are
 * rounded to fp16 for the value product; out is rounded once to q_dtype.
 * The sequence is split into 256-token pieces whose partial softmax results
 * go to `workspace` (caller-owned device memory, 16-byte aligned, at least
 * kv_decode_attention_workspace_size(batch_size, num_kv_heads, num_qo_heads,
 * bt_cols, page_size, head_dim) bytes, no initial contents needed; it is scratch for the
 * duration of the call's stream work, so concurrent calls need their own).
 */
kvfp4_status_t kv_decode_attention(const kvfp4_paged_cache_t *cache, const void *q, int32_t q_dtype,
                                   int32_t num_qo_heads, const int32_t *block_tables, int64_t bt_row_stride,
                                   int32_t bt_cols, const int32_t *seq_lens, int32_t batch_size,
                                   const float *k_scale, const float *v_scale, float sm_scale, void *out,
                                   void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of workspace kv_decode_attention needs for these sizes (-1 for
 * invalid sizes): batch_size * num_kv_heads * ceil(bt_cols * page_size / 256)
 * partials of (2 + head_dim) * min(num_qo_heads / num_kv_heads, 16) floats. */
int64_t kv_decode_attention_workspace_size(int32_t batch_size, int32_t num_kv_heads, int32_t num_qo_heads,
                                           int32_t bt_cols, int32_t page_size, int32_t head_dim);

/*
 * kv_decode_attention_noalloc - kv_decode_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc): the same arguments, kernels and result,
 * without the workspace. The split partials go to a fixed device array of
 * KVFP4_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; the call allocates and frees nothing. Calls whose partials
 * (kv_decode_attention_workspace_size of the same sizes) exceed that size
 * return KVFP4_ESCRATCH before anything is queued. Every call on a GPU uses
 * that GPU's one array: calls whose stream work overlaps on the same GPU
 * (other streams, other host threads) race and must be serialized by the
 * caller; calls in order on one stream are safe. The array needs no initial
 * contents (each call writes every partial it reads).
 */
#define KVFP4_NOALLOC_SCRATCH_BYTES (32ll << 20)
kvfp4_status_t kv_decode_attention_noalloc(const kvfp4_paged_cache_t *cache, const void *q, int32_t q_dtype,
                                           int32_t num_qo_heads, const int32_t *block_tables,
                                           int64_t bt_row_stride, int32_t bt_cols, const int32_t *seq_lens,
                                           int32_t batch_size, const float *k_scale, const float *v_scale,
                                           float sm_scale, void *out, void *stream);

/*
 * Host-side table checks: a debugging aid for the values the calls above
 * never check (the module page's materializer note: lengths, page indices
 * and indptr are not checked by the launchers). Each function reads HOST
 * copies of the index arrays (plain host pointers, not device memory), with
 * the same meaning as the corresponding call's arguments, and returns
 * KVFP4_OK when every value the call would use is in range, KVFP4_EVALUE with
 * *report set to the first problem found, or KVFP4_EINVAL for bad arguments.
 * Nothing is launched and no device memory is touched.
 *   problem  one of KVFP4_TABLE_* below
 *   index    the offending element: the row (append rows), the request, or
 *            the flat index into kv_indices / block_tables / indptr
 *   value    that element's value
 */
enum {
    KVFP4_TABLE_OK = 0,
    KVFP4_TABLE_INDPTR_START = 1,    /* kv_indptr / kv_page_indptr[0] != 0 */
    KVFP4_TABLE_INDPTR_ORDER = 2,    /* the indptr array decreases */
    KVFP4_TABLE_PAGE_RANGE = 3,      /* a page id the call reads is outside [0, num_pages) */
    KVFP4_TABLE_BATCH_RANGE = 4,     /* batch_indices[r] outside [0, batch_size) */
    KVFP4_TABLE_POSITION_RANGE = 5,  /* positions[r] outside the request's reserved space */
    KVFP4_TABLE_LAST_PAGE_LEN = 6,   /* kv_last_page_len[b] outside [1, page_size] (0 without pages) */
    KVFP4_TABLE_DUPLICATE_ROW = 7,   /* two rows write the same (request, position): they race */
    KVFP4_TABLE_LENGTH_RANGE = 8,    /* a length below 0 or longer than the table row addresses */
    KVFP4_TABLE_RESERVATION = 9,     /* kv_page_indptr reserves fewer pages than a request needs */
    KVFP4_TABLE_OUT_PAGES = 10,      /* out has fewer than kv_page_indptr[batch_size] + 1 pages */
    KVFP4_TABLE_STEP_POSITION = 11   /* a decode-step row's position is not seq_lens[b] - 1 */
};
typedef struct {
    int32_t problem;
    int64_t index;
    int64_t value;
} kvfp4_table_report_t;

/* kv_quantize_append's tables: kv_indptr starts at 0 and never decreases,
 * every kv_indices entry is a page id, kv_last_page_len[b] is in
 * [1, page_size] for a request with pages (0 otherwise), every row's request
 * is in range and its position inside (pages - 1) * page_size +
 * kv_last_page_len[b]. With `scratch` (host memory for nnz int64 values,
 * overwritten) rows that write the same (request, position) are reported
 * too; NULL skips that check. */
kvfp4_status_t kvfp4_check_append_tables(const int32_t *batch_indices, const int32_t *positions, int64_t nnz,
                                         const int32_t *kv_indices, const int32_t *kv_indptr,
                                         const int32_t *kv_last_page_len, int32_t batch_size, int32_t page_size,
                                         int32_t num_pages, int64_t *scratch, kvfp4_table_report_t *report);

/* kv_append_dequantize_paged's rows (on top of the two checks above and
 * below, which its append and dequant tables need as well): nnz ==
 * batch_size (KVFP4_EINVAL otherwise), every row's request in range and its
 * position seq_lens[b] - 1, and, with `scratch` (host memory for batch_size
 * int64 values, overwritten), no request named by two rows. Whether another
 * request reads a row's slot is not checked. */
kvfp4_status_t kvfp4_check_step_rows(const int32_t *batch_indices, const int32_t *positions, int64_t nnz,
                                     const int32_t *seq_lens, int32_t batch_size, int64_t *scratch,
                                     kvfp4_table_report_t *report);

/* kv_dequantize_paged's (max_seq_len as given) and kv_decode_attention's
 * (max_seq_len = INT32_MAX, bt_dtype KVFP4_I32) tables: every length is
 * >= 0 and needs at most bt_cols pages, and the page ids of the pages a
 * request uses are in range. */
kvfp4_status_t kvfp4_check_paged_tables(const void *block_tables, int32_t bt_dtype, int64_t bt_row_stride,
                                        int32_t bt_cols, const int32_t *seq_lens, int32_t batch_size,
                                        int32_t page_size, int32_t num_pages, int32_t max_seq_len,
                                        kvfp4_table_report_t *report);

/* kv_materialize_fp8's tables: kv_page_indptr starts at 0 and never
 * decreases, reserves at least ceil(seq_lens[b] / page_size) pages per
 * request and fits num_out_pages - 1 pages; 0 <= seq_lens[b] <=
 * max_pages_per_seq * page_size; the K (and V) page ids of every page used
 * are in range. */
kvfp4_status_t kvfp4_check_materialize_tables(const int32_t *block_tables, int32_t uses_shared_paged_kv_idx,
                                              int64_t bt_row_stride, int64_t bt_kv_stride, int32_t bt_cols,
                                              const int32_t *seq_lens, const int32_t *kv_page_indptr,
                                              int32_t batch_size, int32_t page_size, int32_t num_pages,
                                              int32_t max_pages_per_seq, int64_t num_out_pages,
                                              kvfp4_table_report_t *report);

/* Static description of a KVFP4_TABLE_* problem. */
const char *kvfp4_table_problem_string(int32_t problem);

/* Static description of a status code. */
const char *kvfp4_status_string(kvfp4_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* KVFP4_H */

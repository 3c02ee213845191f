// kvfp4_internal.h - launchers shared between the C-ABI layer and the kernel
// translation units. Arguments reaching these functions are already checked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvfp4.h"

namespace kvfp4 {

// Persistent grids: 256 CUs x 8 resident 256-thread workgroups.
constexpr int kPersistentWorkgroups = 2048;

hipError_t launch_quantize_append(const kvfp4_paged_cache_t &c, const void *key, const void *value,
                                  bool in_bf16, int64_t nnz, const int32_t *batch_indices,
                                  const int32_t *positions, const int32_t *kv_indices,
                                  const int32_t *kv_indptr, float k_scale, float v_scale,
                                  const kvfp4_recipe_t *recipe, hipStream_t st);

hipError_t launch_dequantize_paged(const kvfp4_paged_cache_t &c, const void *block_tables, bool bt64,
                                   int64_t bt_row_stride, const int32_t *seq_lens, int32_t batch,
                                   const float *k_scale, const float *v_scale, void *out_k, void *out_v,
                                   bool out_bf16, int32_t max_seq_len, hipStream_t st);

// the append then the dequantize of a decode step (each request's newest
// token is one appended row, at position seq_lens[b] - 1), in one launch
// where the recipe and layout allow it
hipError_t launch_append_dequantize_paged(const kvfp4_paged_cache_t &c, const void *key, const void *value,
                                          bool in_bf16, int64_t nnz, const int32_t *batch_indices,
                                          const int32_t *positions, const int32_t *kv_indices,
                                          const int32_t *kv_indptr, float k_g, float v_g,
                                          const kvfp4_recipe_t *recipe, const void *block_tables, bool bt64,
                                          int64_t bt_row_stride, const int32_t *seq_lens, int32_t batch,
                                          const float *k_scale, const float *v_scale, void *out_k, void *out_v,
                                          bool out_bf16, int32_t max_seq_len, hipStream_t st);

hipError_t launch_materialize_fp8(const kvfp4_paged_cache_t &c, bool v_interleaved, const int32_t *bt,
                                  bool shared, int64_t bt_row_stride, int64_t bt_kv_stride,
                                  const int32_t *seq_lens, const int32_t *indptr, int32_t batch,
                                  void *out, int64_t num_out_pages, int32_t *table, int32_t maxp,
                                  hipStream_t st);

hipError_t launch_global_scale(const void *x, bool bf16, int64_t n, float e4m3_max, float *g_out,
                               hipStream_t st);

hipError_t launch_quantize_contiguous(const void *x, bool in_bf16, int64_t rows, int64_t cols, const float *g,
                                      const kvfp4_recipe_t *recipe, void *codes, void *scales, hipStream_t st);

hipError_t launch_dequantize_contiguous(const void *codes, const void *scales, int64_t rows, int64_t cols,
                                        const float *g, void *out, bool out_bf16, hipStream_t st);

hipError_t launch_quantize_paged_cache(const kvfp4_paged_cache_t &c, const void *k_in, const void *v_in,
                                       bool in_bf16, const float *k_scale, const float *v_scale,
                                       const kvfp4_recipe_t *recipe, bool v_interleaved, hipStream_t st);

hipError_t launch_decode_attention(const kvfp4_paged_cache_t &c, const void *q, bool bf16, int32_t num_qo_heads,
                                   const int32_t *bt, int64_t bt_row_stride, int32_t bt_cols,
                                   const int32_t *seq_lens, int32_t batch, const float *k_scale,
                                   const float *v_scale, float sm_scale, void *out, void *workspace,
                                   hipStream_t st);
int64_t decode_attention_splits(int32_t bt_cols, int32_t page_size);
// the current device's address of the no-allocation entry point's scratch
// array (kNoAllocScratchBytes), looked up on the first call on each device
constexpr int64_t kNoAllocScratchBytes = KVFP4_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void **addr);
int64_t decode_attention_workspace_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_qo_heads, int32_t bt_cols,
                                         int32_t page_size, int32_t head_dim);

}  // namespace kvfp4

/*
 * kvfp4_oracle.h - interface of the plain CPU oracle for the paged NVFP4
 * KV-cache path (quantize-append, gather-dequantize, materialize-FP8).
 *
 * TEST INFRASTRUCTURE. This library is a checker: only the test-suite, the
 * package smoke check and the benchmark's CPU-baseline leg load it. The GPU
 * library neither includes this header nor links this code, and this code
 * includes nothing of the GPU library.
 *
 * Every pointer is host memory owned by the caller. Every function returns 0
 * on success and a negative number when an argument or a tensor value breaks
 * the contract stated at that function (the oracle checks values that the
 * GPU library, like the pages' launchers, does not check).
 */
#ifndef KVFP4_ORACLE_H
#define KVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar codecs (all defined by nearest-value scans) ---------------- */
double orc_e2m1_value(int code);                 /* code 0..15 */
int    orc_e2m1_encode(float v);                 /* RNE onto the grid, saturating at 6 */
double orc_e4m3_value(int byte);                 /* byte 0..255, NaN for 0x7F/0xFF */
int    orc_e4m3_encode_scale(float sf, float e4m3_max);   /* sf >= 0 */
int    orc_e4m3_encode_satfinite(float p);       /* sign kept, saturates to +-448 */
double orc_half_value(uint16_t bits, int is_bf16);
uint16_t orc_round_half(float x, int is_bf16);   /* fp32 -> fp16/bf16, RNE */

/* array forms of the codecs, for exhaustive checks from Python */
void orc_e2m1_encode_array(const float *v, int64_t n, uint8_t *out);
void orc_e4m3_encode_scale_array(const float *sf, int64_t n, float e4m3_max, uint8_t *out);
void orc_e4m3_encode_satfinite_array(const float *p, int64_t n, uint8_t *out);
void orc_round_half_array(const float *x, int64_t n, int is_bf16, uint16_t *out);

/* ---- recipe ------------------------------------------------------------ */
/* four_over_six = 0: standard amax/6 block scale clamped at e4m3_max.
 * four_over_six = 1: two-candidate search, err_mode 0 = MSE, 1 = MAE;
 * err_fp16 = 1 evaluates the error in fp16 ("err_use_fast_math").       */
typedef struct {
    int   four_over_six;
    float e4m3_max;
    int   err_mode;
    int   err_fp16;
} orc_recipe_t;

/* One 16-element block. Writes the 16 codes and the chosen scale byte.
 * err6/err4/chose4 report the 4over6 search (zeros for the standard recipe). */
int orc_quantize_block(const float *x16, float g, const orc_recipe_t *recipe,
                       uint8_t *codes16, uint8_t *scale_byte,
                       float *err6, float *err4, int *chose4);

/* Per-tensor global decode scale: amax(|x|) / (6 * e4m3_max), 1 when all zero. */
float orc_global_scale(const uint16_t *x, int64_t n, int is_bf16, float e4m3_max);

/* ---- paged cache description ------------------------------------------- */
typedef struct {
    uint8_t *k_data, *v_data;         /* packed E2M1, head_dim/2 bytes per (token, head) */
    uint8_t *k_sf, *v_sf;             /* E4M3 bytes, head_dim/16 per (token, head) */
    int64_t k_page_stride, v_page_stride;        /* bytes between pages */
    int64_t k_sf_page_stride, v_sf_page_stride;  /* bytes between pages */
    int32_t num_pages, page_size, num_heads, head_dim;
    int32_t layout;                   /* 0 = NHD [ps,H,*], 1 = HND [H,ps,*] */
} orc_cache_t;

int orc_quantize_append(const orc_cache_t *cache,
                        const uint16_t *key, const uint16_t *value, int in_is_bf16, int64_t nnz,
                        const int32_t *batch_indices, const int32_t *positions,
                        const int32_t *kv_indices, const int32_t *kv_indptr,
                        const int32_t *kv_last_page_len, int32_t batch_size,
                        float k_scale, float v_scale, const orc_recipe_t *recipe, int threads);

int orc_dequantize_paged(const orc_cache_t *cache,
                         const void *block_tables, int bt_is_int64, int64_t bt_row_stride, int32_t bt_cols,
                         const int32_t *seq_lens, int32_t batch_size,
                         float k_scale, float v_scale,
                         uint16_t *out_k, uint16_t *out_v, int out_is_bf16, int32_t max_seq_len,
                         int threads);

int orc_materialize_fp8(const orc_cache_t *cache, int v_sf_interleaved,
                        const int32_t *block_tables, int shared, int64_t bt_row_stride,
                        int64_t bt_kv_stride, int32_t bt_cols,
                        const int32_t *seq_lens, const int32_t *kv_page_indptr, int32_t batch_size,
                        uint8_t *out, int64_t num_out_pages,
                        int32_t *fp8_block_tables, int32_t max_pages_per_seq, int threads);

/* ---- contiguous codec with linear block scales ------------------------- */
/* x is [rows, cols] row-major fp16/bf16 with cols % 16 == 0; blocks of 16
 * run along each row. codes [rows, cols/2] (low nibble = even element),
 * scales [rows, cols/16]; g is the global decode scale. */
int orc_quantize_contiguous(const uint16_t *x, int in_is_bf16, int64_t rows, int64_t cols, float g,
                            const orc_recipe_t *recipe, uint8_t *codes, uint8_t *scales, int threads);
int orc_dequantize_contiguous(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                              float g, uint16_t *out, int out_is_bf16, int threads);

/* ---- whole-pool quantizer ---------------------------------------------- */
/* k_in / v_in are contiguous fp16/bf16 pools of cache->num_pages pages, each
 * page [ps, H, D] (NHD) or [H, ps, D] (HND) as cache->layout; every slot of
 * every page is quantized into the cache (same layout, the cache's page
 * strides). V scales are written 4-token interleaved when v_sf_interleaved
 * (HND and page_size % 4 == 0 only), K scales always linear. */
int orc_quantize_paged_cache(const orc_cache_t *cache, const uint16_t *k_in, const uint16_t *v_in,
                             int in_is_bf16, float k_scale, float v_scale, const orc_recipe_t *recipe,
                             int v_sf_interleaved, int threads);

/* ---- decode attention over the paged NVFP4 cache ------------------------ */
/* One query token per request: for query head hq (kv head hq / (Hq / H)),
 *   s_t = sm_scale * sum_e q[b, hq, e] * K[b, t, e],  t < seq_lens[b]
 *   out[b, hq, :] = sum_t softmax(s)_t * V[b, t, :]
 * with K, V the exact dequantized values e2m1 * E4M3(s) * g (no rounding).
 * q is [B, Hq, D] fp16/bf16 bits; out [B, Hq, D] double. A request of length
 * 0 gives zeros. Computed in double. */
int orc_decode_attention(const orc_cache_t *cache, const uint16_t *q, int q_is_bf16, int32_t num_qo_heads,
                         const int32_t *block_tables, int64_t bt_row_stride, int32_t bt_cols,
                         const int32_t *seq_lens, int32_t batch_size, float k_scale, float v_scale,
                         float sm_scale, double *out, int threads);

#ifdef __cplusplus
}
#endif
#endif

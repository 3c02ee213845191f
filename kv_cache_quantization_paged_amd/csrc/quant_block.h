// quant_block.h - the NVFP4 block quantizer shared by the paged append, the
// contiguous quantize and the whole-pool quantize kernels (FlashInfer
// pages: flashinfer.page.nvfp4_quantize_append_paged_kv_cache; the "NVFP4
// 4over6 Recipes" and "FP4 KV Cache Quantization" sections of the
// flashinfer.quantization page).
//
// fp32 order (bit-exact with the reference reading):
//   sf  = amax / fp32(C * g)                 (IEEE division)
//   s   = E4M3_RNE(min(sf, clamp_C))
//   dec = fp32(E4M3(s) * g),  inv = dec ? fp32(1 / dec) : 0
//   c_i = E2M1_RNE_sat(fp32(x_i * inv))
//   4over6: d_i = x_i - fp32(dec * e2m1(c_i)); MSE d_i*d_i or MAE |d_i|;
//   pairwise tree over the 16 terms; amax/4 kept only when strictly lower.
// dec and inv depend only on (tensor, scale byte): callers tabulate them for
// the 127 finite non-negative scale bytes (in LDS) and pass the table.
#pragma once

#include "nvfp4_device.h"

namespace kvfp4 {

template <bool BF16>
__device__ __forceinline__ void load_block(const uint8_t *p, float x[16])
{
    const uint4 a = *(const uint4 *)p;
    const uint4 b = *(const uint4 *)(p + 16);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[2 * i] = BF16 ? bf16_lo(w[i]) : f16_lo(w[i]);
        x[2 * i + 1] = BF16 ? bf16_hi(w[i]) : f16_hi(w[i]);
    }
}

// E2M1 codes of fp32(x_i * inv), packed two per byte, element 0 lowest
__device__ __forceinline__ uint2 encode16(const float x[16], float inv)
{
    uint32_t w0 = 0u, w1 = 0u;
    w0 = f32x2_to_fp4x2<0>(w0, x[0] * inv, x[1] * inv);
    w0 = f32x2_to_fp4x2<1>(w0, x[2] * inv, x[3] * inv);
    w0 = f32x2_to_fp4x2<2>(w0, x[4] * inv, x[5] * inv);
    w0 = f32x2_to_fp4x2<3>(w0, x[6] * inv, x[7] * inv);
    w1 = f32x2_to_fp4x2<0>(w1, x[8] * inv, x[9] * inv);
    w1 = f32x2_to_fp4x2<1>(w1, x[10] * inv, x[11] * inv);
    w1 = f32x2_to_fp4x2<2>(w1, x[12] * inv, x[13] * inv);
    w1 = f32x2_to_fp4x2<3>(w1, x[14] * inv, x[15] * inv);
    return make_uint2(w0, w1);
}

// terms of one packed dword (8 elements starting at x[0])
template <bool MSE>
__device__ __forceinline__ void terms8(const float *x, uint32_t w, float dec, float t[8])
{
    const f32x2 v0 = fp4x2_to_f32x2<0>(w), v1 = fp4x2_to_f32x2<1>(w);
    const f32x2 v2 = fp4x2_to_f32x2<2>(w), v3 = fp4x2_to_f32x2<3>(w);
    const float v[8] = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float d = x[i] - dec * v[i];
        t[i] = MSE ? d * d : fabsf(d);
    }
}

// summed error of a candidate: pairwise tree over the 16 terms in index order
template <bool MSE>
__device__ __forceinline__ float block_error(const float x[16], uint2 codes, float dec)
{
    float t[16];
    terms8<MSE>(x, codes.x, dec, t);
    terms8<MSE>(x + 8, codes.y, dec, t + 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = t[2 * i] + t[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = t[2 * i] + t[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0] + t[1];
}

// RECIPE: 0 standard, 1 4over6 MSE, 2 4over6 MAE. x holds the block, amax
// its largest magnitude; returns the packed codes and sets the scale byte.
template <int RECIPE>
__device__ __forceinline__ uint2 quantize_block(const float x[16], float amax, float g, float clamp6,
                                                const float *dec_tab, const float *inv_tab, uint32_t &s_out)
{
    const float sf6 = amax / (6.0f * g);
    uint32_t s = f32_to_e4m3_hw(fminf(sf6, clamp6));
    uint2 codes = encode16(x, inv_tab[s]);
    if (RECIPE != 0) {
        const float dec = dec_tab[s];
        const float sf4 = amax / (4.0f * g);
        const uint32_t s4 = f32_to_e4m3_hw(fminf(sf4, 448.0f));
        const float dec4 = dec_tab[s4];
        const uint2 codes4 = encode16(x, inv_tab[s4]);
        const float e6 = block_error<RECIPE == 1>(x, codes, dec);
        const float e4 = block_error<RECIPE == 1>(x, codes4, dec4);
        if (e4 < e6) {
            s = s4;
            codes = codes4;
        }
    }
    s_out = s;
    return codes;
}

}  // namespace kvfp4

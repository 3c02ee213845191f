// quant_block.h - the NVFP4 block quantizer shared by the paged append, the
// contiguous quantize and the whole-pool quantize kernels (FlashInfer
// pages: flashinfer.page.nvfp4_quantize_append_paged_kv_cache; the "NVFP4
// 4over6 Recipes" and "FP4 KV Cache Quantization" sections of the
// flashinfer.quantization page).
//
// fp32 order (bit-exact with the reference reading):
//   sf  = amax / fp32(C * g)                 (IEEE division; scale_code
//                                             reaches the same code faster)
//   s   = E4M3_RNE(min(sf, clamp_C))
//   dec = fp32(E4M3(s) * g),  inv = dec ? fp32(1 / dec) : 0
//   c_i = E2M1_RNE_sat(fp32(x_i * inv))
//   4over6: d_i = x_i - fp32(dec * e2m1(c_i)); MSE d_i*d_i or MAE |d_i|;
//   pairwise tree over the 16 terms; amax/4 kept only when strictly lower.
// dec and inv depend only on (tensor, scale byte): callers tabulate them for
// the 127 finite non-negative scale bytes (in LDS) and pass the table.
#pragma once

#include "../../include/kvfp4.h"
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

// A quick stand-in for a candidate's error, to decide the 4over6 choice
// without the exact tree in almost every block: each difference is one fused
// x_i - dec * e2m1_i (rounded once) and the terms (its square for MSE, its
// magnitude for MAE) are accumulated by a chain of fused multiply-adds /
// adds. With u = 2^-24, S the exact sum of the exact terms and q_i = dec *
// e2m1_i (|q_i| <= 6 dec):
//   MSE: pairwise tree vs S within 5.0001u S; the fused differences move the
//        sum by at most 10.001u S + 1.0001u sum(q_i^2) <= ... + 576.06u dec^2;
//        the chain adds 16.0001u S': in all within 31.01u S + 577u dec^2.
//   MAE: tree within 4.0001u S, the differences within 2.0001u S + 96.01u
//        dec, the chain 15.001u S': in all within 21.01u S + 97u dec.
// Results in fp32's subnormal range add at most 2^-140 of absolute error.
template <bool MSE>
__device__ __forceinline__ float error_chain(const float x[16], uint2 codes, float dec)
{
    float acc = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint32_t w = half ? codes.y : codes.x;
        const f32x2 v0 = fp4x2_to_f32x2<0>(w), v1 = fp4x2_to_f32x2<1>(w);
        const f32x2 v2 = fp4x2_to_f32x2<2>(w), v3 = fp4x2_to_f32x2<3>(w);
        const float v[8] = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float d = __builtin_fmaf(-dec, v[i], x[8 * half + i]);
            acc = MSE ? __builtin_fmaf(d, d, acc) : acc + fabsf(d);
        }
    }
    return acc;
}

// 4over6 choice for the fp32 MSE / MAE recipes: amax/4 iff its pairwise-tree
// error is strictly lower. The chains decide it whenever they are further
// apart than m, which is at least the sum of both chains' worst distances to
// their trees above (the constants are generous: 2^-18 >= 64u covers 31.01u
// with room for m's own roundings, 2^-14 >= 1024u covers 577u, 2^-19 >= 32u
// covers 21.01u, 2^-17 >= 128u covers 97u; the 2^-126 floor covers the
// subnormal term). Both chains zero means every difference is zero, so both
// trees are zero: a tie, amax/6 stays. Anything closer, and an inf on either
// side (m is then inf or NaN and neither test passes), is decided by the
// trees themselves, so the choice is always the trees' choice.
template <bool MSE>
__device__ __forceinline__ bool chain_takes_amax4(const float x[16], uint2 codes6, float dec6, uint2 codes4,
                                                  float dec4)
{
    const float f6 = error_chain<MSE>(x, codes6, dec6);
    const float f4 = error_chain<MSE>(x, codes4, dec4);
    if (f4 == 0.0f && f6 == 0.0f)
        return false;
    const float m = MSE ? fmaxf(0x1p-18f * (f4 + f6) + 0x1p-14f * (dec4 * dec4 + dec6 * dec6), 0x1p-126f)
                        : fmaxf(0x1p-19f * (f4 + f6) + 0x1p-17f * (dec4 + dec6), 0x1p-126f);
    if (f6 - f4 > m)
        return true;
    if (f4 - f6 > m)
        return false;
    return block_error<MSE>(x, codes4, dec4) < block_error<MSE>(x, codes6, dec6);
}

// fp32 value -> nearest fp16 value (ties to even), back in fp32 (exact)
__device__ __forceinline__ float round_f16(float v) { return (float)(_Float16)v; }

// the same error in IEEE fp16 ("err_use_fast_math"): the input and the fp32
// reconstruction are rounded to fp16, then the difference, the square and
// every sum of the tree are fp16 operations (each rounds to nearest-even,
// overflowing to inf). Each fp16 operation is done in fp32 and rounded once
// to fp16: fp32 carries 24 >= 2 * 11 + 2 significant bits, so for +, - and *
// that double rounding gives exactly the correctly rounded fp16 result.
// the input in fp16, as pairs xh[j] = (x_j, x_{j+8}): this pairing puts
// every level of the index-order tree except the last in packed fp16 adds
// (the empty asm pins the converted pairs, so that the subtraction below
// cannot be folded back into the conversions: that rewrite trips an
// instruction-selection failure when packed fp32 instructions are disabled)
__device__ __forceinline__ void inputs_fp16(const float x[16], f16x2 xh[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[j], x[j + 8]}, f16x2));
        asm volatile("" : "+v"(b));
        xh[j] = __builtin_bit_cast(f16x2, b);
    }
}

// the same error in IEEE fp16 ("err_use_fast_math"): the input and the fp32
// reconstruction are rounded to fp16, then the difference, the square and
// every sum of the tree are fp16 operations, each rounding to nearest-even
// (overflow gives inf). Lane pairs (j, j+8) go through packed fp16 math:
// V_j = (d_j, d_{j+8}), then V_{2k} + V_{2k+1} = (p_k, p_{k+4}) are the
// first-level sums, (q_m, q_{m+2}) the second, (r_0, r_1) the third.
template <bool MSE>
__device__ __forceinline__ float block_error_fp16(const f16x2 xh[8], uint2 codes, float dec)
{
    f16x2 t[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x2 lo = k == 0 ? fp4x2_to_f32x2<0>(codes.x) : k == 1 ? fp4x2_to_f32x2<1>(codes.x)
                       : k == 2 ? fp4x2_to_f32x2<2>(codes.x) : fp4x2_to_f32x2<3>(codes.x);
        const f32x2 hi = k == 0 ? fp4x2_to_f32x2<0>(codes.y) : k == 1 ? fp4x2_to_f32x2<1>(codes.y)
                       : k == 2 ? fp4x2_to_f32x2<2>(codes.y) : fp4x2_to_f32x2<3>(codes.y);
        // elements 2k, 2k+1 (lo) and 2k+8, 2k+9 (hi). The fp32 reconstruction
        // is rounded to fp32 first: the empty asm keeps the compiler from
        // fusing multiply and conversion into one v_fma_mix, whose single
        // rounding of the exact product to fp16 differs from rounding the
        // fp32 product (a 26-bit value).
        float r0 = dec * lo.x, r1 = dec * lo.y, r8 = dec * hi.x, r9 = dec * hi.y;
        asm volatile("" : "+v"(r0), "+v"(r1), "+v"(r8), "+v"(r9));
        const f16x2 ra = __builtin_convertvector((f32x2){r0, r8}, f16x2);
        const f16x2 rb = __builtin_convertvector((f32x2){r1, r9}, f16x2);
        // reconstruction minus input: the negated difference, same square and |d|
        const f16x2 da = ra - xh[2 * k], db = rb - xh[2 * k + 1];
        t[2 * k] = MSE ? da * da : __builtin_elementwise_abs(da);
        t[2 * k + 1] = MSE ? db * db : __builtin_elementwise_abs(db);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = t[2 * k] + t[2 * k + 1];       // (p_k, p_{k+4})
    t[0] = t[0] + t[1];                                                // (q_0, q_2)
    t[1] = t[2] + t[3];                                                // (q_1, q_3)
    t[0] = t[0] + t[1];                                                // (r_0, r_1)
    const _Float16 e = t[0].x + t[0].y;
    return (float)e;
}

// RECIPE: 0 standard, 1 4over6 MSE, 2 4over6 MAE, 3 MSE in fp16, 4 MAE in
// fp16. x holds the block, amax its largest magnitude; returns the packed
// codes and sets the scale byte.
// E4M3_RNE(min(fp32(amax / t), clamp)), the block-scale code, for amax >= 0
// and t = fp32(C * g) > 0 (rt = fp32(1 / t)). q = fp32(amax * rt) is within
// 3.0001u (amax / t) of the quotient, so fp32(amax / t) and q are at most 4
// bit patterns apart, and they round to the same E4M3 code unless an E4M3
// rounding midpoint lies between them. Normal E4M3 midpoints (1.mmm1 x 2^e)
// have bit 19 set and bits 18..0 clear in fp32, so a q whose low 20 bits are
// more than 16 away from 0x80000 has none within reach; below 2^-6 (the
// subnormal E4M3 range, where midpoints fall elsewhere) only q < 2^-11, where
// both give code 0, is taken directly. Everything else divides in IEEE fp32,
// which is then exactly the quotient the arithmetic defines. Clamping cannot
// separate the two either: the clamp is itself an E4M3 value.
__device__ __forceinline__ uint32_t scale_code(float amax, float t, float rt, float clamp)
{
    const float q = amax * rt;
    const uint32_t low = __float_as_uint(q) & 0xFFFFFu;
    const bool direct = q < 0x1p-11f || (q >= 0x1p-6f && low - 0x7FFF0u > 32u);
    float sf = q;
    if (__builtin_expect(!direct, 0))
        sf = amax / t;
    return f32_to_e4m3_hw(fminf(sf, clamp));
}

template <int RECIPE>
__device__ __forceinline__ uint2 quantize_block(const float x[16], float amax, float g, float clamp6,
                                                const float *dec_tab, const float *inv_tab, uint32_t &s_out)
{
    const float t6 = 6.0f * g, t4 = 4.0f * g;
    uint32_t s = scale_code(amax, t6, 1.0f / t6, clamp6);
    uint2 codes = encode16(x, inv_tab[s]);
    if (RECIPE != 0) {
        const float dec = dec_tab[s];
        const uint32_t s4 = scale_code(amax, t4, 1.0f / t4, 448.0f);
        const float dec4 = dec_tab[s4];
        const uint2 codes4 = encode16(x, inv_tab[s4]);
        constexpr bool kMse = RECIPE == 1 || RECIPE == 3;
        bool take4;
        if (RECIPE >= 3) {
            f16x2 xh[8];
            inputs_fp16(x, xh);
            take4 = block_error_fp16<kMse>(xh, codes4, dec4) < block_error_fp16<kMse>(xh, codes, dec);
        } else {
            take4 = chain_takes_amax4<kMse>(x, codes, dec, codes4, dec4);
        }
        if (take4) {                       // an inf or NaN error never wins
            s = s4;
            codes = codes4;
        }
    }
    s_out = s;
    return codes;
}

// kernel recipe index of a (checked) recipe: 0 standard, 1/2 MSE/MAE in
// fp32, 3/4 MSE/MAE in fp16
inline int recipe_kind(const kvfp4_recipe_t *recipe)
{
    if (recipe == nullptr)
        return 0;
    return (recipe->err_mode == KVFP4_ERR_MSE ? 1 : 2) + (recipe->err_use_fast_math ? 2 : 0);
}

}  // namespace kvfp4

// nvfp4_device.h - device-side number-format helpers for the gfx950 kernels.
//
// E2M1 (OCP FP4): sign bit 3, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for
// codes 0..7. E4M3 (OCP float8_e4m3fn): bias 7, subnormal step 2^-9, largest
// finite 448, 0x7F/0xFF NaN. Rounding is always to nearest, ties to even,
// as the FlashInfer KV-cache pages' formats require of a quantizer; every
// helper here is exact integer or single-rounding fp32 work so that the
// results are reproducible bit for bit. Build with -ffp-contract=off: no step
// below may be fused with a neighbouring multiply or add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- E4M3 ----
// byte -> fp32 (exact; NaN bytes give NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b)
{
    const uint32_t mag = b & 0x7Fu;
    float v = (mag >= 8u) ? __uint_as_float((mag << 20) + (120u << 23))   // (1+m/8) 2^(e-7)
                          : (float)mag * 0x1p-9f;                          // m 2^-9
    v = (mag == 0x7Fu) ? __uint_as_float(0x7FC00000u) : v;
    return (b & 0x80u) ? -v : v;
}

// x in [0, 448] -> nearest E4M3 byte (ties to the even code).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float x)
{
    if (x < 0x1p-6f)                                          // subnormal range: step 2^-9
        return (uint32_t)__builtin_rintf(x * 512.0f);         // 8 here is 2^-6, the first normal
    const uint32_t u = __float_as_uint(x);
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);       // keep 3 mantissa bits, RNE
    return (r >> 20) - (120u << 3);
}

// |p| of an exact product, any magnitude -> E4M3 byte with saturation to 448;
// the sign comes from `sign` (0 or 0x80). NaN -> 0x7F | sign.
__device__ __forceinline__ uint32_t f32_to_e4m3_satfinite(float a, uint32_t sign)
{
    if (!(a == a))
        return 0x7Fu | sign;
    return f32_to_e4m3_rne(fminf(a, 448.0f)) | sign;
}

// ---------------------------------------------------------------- E2M1 ----
// |v| (finite) -> nearest E2M1 magnitude as fp32, ties to even, saturating at
// 6. The grid has step 0.5 below 2 and doubles every binade above, so adding
// c = 2^(E+22), whose ulp is that step (E = exponent of max(|v|, 1)), lets
// the fp32 adder do the round-to-nearest-even; subtracting c gives the value.
__device__ __forceinline__ float e2m1_round_mag(float a)
{
    const uint32_t u = __float_as_uint(a);
    // exponent of |v| clamped to [1, 8]: below 1 the step stays 0.5, above 8
    // everything saturates anyway (and c stays a finite power of two)
    const uint32_t clamped = u < 0x3F800000u ? 0x3F800000u : (u > 0x41000000u ? 0x41000000u : u);
    const float c = __uint_as_float((clamped & 0x7F800000u) + (22u << 23));
    const float q = (a + c) - c;
    return fminf(q, 6.0f);
}

// nearest-E2M1 magnitude (0, 0.5, 1, ..., 6) -> its 3-bit code.
__device__ __forceinline__ uint32_t e2m1_mag_to_code(float q)
{
    const uint32_t hi = (__float_as_uint(q) >> 22);          // 252 for 0.5, 254.. for >= 1
    const uint32_t k = hi >= 254u ? hi - 252u : 0u;
    return q == 0.5f ? 1u : k;
}

// E2M1 magnitude code 0..7 -> value (exact).
__device__ __forceinline__ float e2m1_code_to_mag(uint32_t k)
{
    const uint32_t bits = (k >= 2u) ? ((k + 252u) << 22) : (k ? 0x3F000000u : 0u);
    return __uint_as_float(bits);
}

// ------------------------------------------------ gfx950 conversions ----
// These conversion instructions are used only in the forms that reproduce
// the definitions above bit for bit (checked exhaustively per input class on
// the device): the FP4 and FP8 decodes are exact; the FP4 encode with a unit
// scale rounds to nearest-even onto the E2M1 grid, saturates at +-6 and keeps
// the sign of zero; the FP8 encode rounds to nearest-even for |x| <= 448 (it
// is only given clamped values). Their scale operand applies only its
// exponent, so it is always 1.0 here.

// byte SEL of `packed` (two E2M1 codes, low nibble first) -> two fp32 values
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32x2(uint32_t packed)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, SEL);
}

// two fp32 -> two E2M1 codes written into byte SEL of `old`, `lo` in the low
// nibble; the other bytes of `old` are kept
template <int SEL>
__device__ __forceinline__ uint32_t f32x2_to_fp4x2(uint32_t old, float lo, float hi)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, SEL);
}

// E4M3 byte (low 8 bits) -> fp32, exact
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t b)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// x in [0, 448] -> nearest E4M3 byte, ties to even
__device__ __forceinline__ uint32_t f32_to_e4m3_hw(float x)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFFu;
}

// ------------------------------------------------------ buffer access ----
// Raw buffer loads/stores: a wave-uniform base in scalar registers plus a
// 32-bit per-lane byte offset (no 64-bit address arithmetic per lane). An
// access whose offset lies at or beyond `bytes` reads zero and a store there
// is dropped by the hardware range check; the kernels only rely on that for
// whole 4- or 16-byte accesses at aligned offsets, never for partial ones.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferFlags = 0x00020000;   // gfx9 raw-buffer dword 3 (32-bit data format)

// `base` and `bytes` must be the same in every lane of the wavefront; they are
// moved to scalar registers here so that no per-lane descriptor is ever built
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t v = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    void *p = (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// a value known to be equal in every lane of the wavefront, in a scalar register
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t buf_load_u8(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u32(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load_u32x2(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_load_u32x4(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_u8(uint32_t v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x2(u32x2 v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x4(u32x4 v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
// streaming store for outputs no later kernel in the same pass reads back:
// non-temporal (nt) with system scope (sc1), so the lines go on to HBM instead
// of sitting dirty in the caches (and being written back inside whatever runs
// next). Measured 1-2% faster than nt alone on the dequant and materialize
// streams.
constexpr int kStreamStore = 2 | 16;     // cache-policy bits: nt | sc1
__device__ __forceinline__ void buf_store_u32x4_nt(u32x4 v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStreamStore);
}
// non-temporal loads of bytes read once. Measured on the materialize loads
// (+0.6%) and on the gather dequant's code bytes (+1.8%); the same hint on the
// dequant's scale bytes (whose lines several lanes and items share) cost
// 2.5%, and on the LDS-staged HND dequant 6%, so those keep the default.
constexpr int kStreamLoad = 2;           // cache-policy bits: nt
__device__ __forceinline__ uint32_t buf_load_u32_nt(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kStreamLoad);
}
__device__ __forceinline__ uint32_t buf_load_u8_nt(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, kStreamLoad);
}
__device__ __forceinline__ u32x2 buf_load_u32x2_nt(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kStreamLoad);
}

// ------------------------------------------------------- 16-bit floats ----
// RNE fp32 -> bf16 / fp16 bit patterns, two at a time (gfx950 converts with
// round-to-nearest-even; fp16 keeps subnormals).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    const bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    const f16x2 r = __builtin_convertvector(v, f16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// bf16 / fp16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

}  // namespace kvfp4

// global_scale.hip - per-tensor NVFP4 global decode scale for gfx950
// (make_nvfp4_global_scale with per_token_activation=False, flashinfer.
// quantization page, "NVFP4 4over6 Recipes" and its precedence note):
// g = amax|x| / fp32(6 * e4m3_max), and 1 for an all-zero tensor.
//
// Three short launches on the caller's stream, no scratch memory: the output
// word first holds 0, then the running maximum of |x| as an unsigned bit
// pattern (non-negative floats order like their bits, so an integer atomic max
// is exact), and finally g. Each workgroup reduces its strided share of 16-byte
// loads in registers and across the wavefront before one atomic.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;

__global__ void clear_word(uint32_t *w) { *w = 0u; }

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint4 *x, int64_t n_vec, const uint16_t *tail,
                                                       int64_t n_tail, uint32_t *amax_bits)
{
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_vec; i += (int64_t)gridDim.x * kThreads) {
        const uint4 v = x[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = fmaxf(m, fabsf(BF16 ? bf16_lo(w[k]) : f16_lo(w[k])));
            m = fmaxf(m, fabsf(BF16 ? bf16_hi(w[k]) : f16_hi(w[k])));
        }
    }
    if (blockIdx.x == 0) {
        for (int64_t i = threadIdx.x; i < n_tail; i += kThreads) {
            const uint32_t w = tail[i];
            m = fmaxf(m, fabsf(BF16 ? bf16_lo(w) : f16_lo(w)));
        }
    }
    // wavefront maximum
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0 && m > 0.0f)
        atomicMax(amax_bits, __float_as_uint(m));
}

__global__ void finish_scale(uint32_t *w, float denom)
{
    const float amax = __uint_as_float(*w);
    ((float *)w)[0] = (amax == 0.0f) ? 1.0f : amax / denom;
}

}  // namespace

hipError_t launch_global_scale(const void *x, bool bf16, int64_t n, float e4m3_max, float *g_out, hipStream_t st)
{
    uint32_t *w = (uint32_t *)g_out;
    hipLaunchKernelGGL(clear_word, dim3(1), dim3(1), 0, st, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t n_vec = n / 8;
    const int64_t n_tail = n - n_vec * 8;
    const uint16_t *tail = (const uint16_t *)x + n_vec * 8;
    int64_t wgs = (n_vec + kThreads - 1) / kThreads;
    if (wgs < 1)
        wgs = 1;
    const int grid = (int)(wgs < kPersistentWorkgroups ? wgs : kPersistentWorkgroups);
    if (bf16)
        hipLaunchKernelGGL((amax_kernel<true>), dim3(grid), dim3(kThreads), 0, st, (const uint4 *)x, n_vec, tail,
                           n_tail, w);
    else
        hipLaunchKernelGGL((amax_kernel<false>), dim3(grid), dim3(kThreads), 0, st, (const uint4 *)x, n_vec, tail,
                           n_tail, w);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const float denom = 6.0f * e4m3_max;
    hipLaunchKernelGGL(finish_scale, dim3(1), dim3(1), 0, st, w, denom);
    return hipGetLastError();
}

}  // namespace kvfp4

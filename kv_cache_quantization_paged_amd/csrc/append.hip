// append.hip - NVFP4 quantize-append into paged NHD/HND caches for gfx950
// (FlashInfer page flashinfer.page.nvfp4_quantize_append_paged_kv_cache, and
// the "NVFP4 4over6 Recipes" section of the flashinfer.quantization page).
//
// One lane owns one 16-element block of one (row, head) of K or V: it loads
// the block's 32 input bytes, reduces amax in registers, derives the E4M3
// block scale, encodes 16 E2M1 codes and stores 8 packed bytes plus the scale
// byte at (page, slot) from the CSR table. The 4over6 recipe evaluates both
// candidates in the same lane: no cross-lane traffic.
//
// fp32 order (bit-exact with the reference reading):
//   sf  = amax / fp32(C * g)                 (IEEE division)
//   s   = E4M3_RNE(min(sf, clamp_C))
//   dec = fp32(E4M3(s) * g),  inv = dec ? fp32(1 / dec) : 0
//   c_i = E2M1_RNE_sat(fp32(x_i * inv))
//   4over6: d_i = x_i - fp32(dec * e2m1(c_i)); MSE d_i*d_i or MAE |d_i|;
//   pairwise tree over the 16 terms; amax/4 kept only when strictly lower.
// dec and inv depend only on (tensor, scale byte): each workgroup tabulates
// them for the 127 finite non-negative scale bytes in LDS at start, so a block
// pays one IEEE division (for sf) per candidate and two LDS reads. The E2M1
// encode / decode and the E4M3 encode use gfx950's conversion instructions.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;

struct AppendArgs {
    uint8_t *data[2];
    uint8_t *sf[2];
    int64_t stride[2];
    int64_t sf_stride[2];
    const uint8_t *in[2];
    const int32_t *batch_indices, *positions, *kv_indices, *kv_indptr;
    float g[2];
    int32_t ps, H, D;
    int64_t nnz;
    float clamp6;      // E4M3 clamp of the amax/6 candidate (recipe e4m3_max, or 448)
    int32_t err_mode;  // 0 MSE, 1 MAE
};

struct ScaleTables {
    float dec[2][128];
    float inv[2][128];
};

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

// RECIPE: 0 standard, 1 4over6 MSE, 2 4over6 MAE
template <bool BF16, int RECIPE>
__device__ __forceinline__ void quantize_one(const AppendArgs &a, const ScaleTables &tab, int kv, int64_t r, int h,
                                             int c, int64_t page, int slot, bool hnd)
{
    const int nb = a.D >> 4;
    float x[16];
    load_block<BF16>(a.in[kv] + (((r * a.H + h) * a.D) + c * 16) * 2, x);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const float g = a.g[kv];

    const float sf6 = amax / (6.0f * g);
    uint32_t s = f32_to_e4m3_hw(fminf(sf6, a.clamp6));
    float dec = tab.dec[kv][s];
    uint2 codes = encode16(x, tab.inv[kv][s]);
    if (RECIPE != 0) {
        const float sf4 = amax / (4.0f * g);
        const uint32_t s4 = f32_to_e4m3_hw(fminf(sf4, 448.0f));
        const float dec4 = tab.dec[kv][s4];
        const uint2 codes4 = encode16(x, tab.inv[kv][s4]);
        const float e6 = block_error<RECIPE == 1>(x, codes, dec);
        const float e4 = block_error<RECIPE == 1>(x, codes4, dec4);
        if (e4 < e6) {
            s = s4;
            codes = codes4;
        }
    }
    const int64_t row = hnd ? ((int64_t)h * a.ps + slot) : ((int64_t)slot * a.H + h);
    const u32x2 cv = {codes.x, codes.y};
    __builtin_nontemporal_store(cv, (u32x2 *)(a.data[kv] + page * a.stride[kv] + row * (a.D >> 1) + c * 8));
    a.sf[kv][page * a.sf_stride[kv] + row * nb + c] = (uint8_t)s;
}

// At least 6 workgroups (24 waves) per CU: caps the 4over6 kernels at 80
// VGPRs without spilling, which hides more memory latency than the default
// allocation (98 VGPRs, 4 waves per SIMD) does.
template <bool BF16, int RECIPE, bool HND>
__global__ __launch_bounds__(kThreads, 6) void append_kernel(AppendArgs a)
{
    __shared__ ScaleTables tab;
    const int tid = threadIdx.x;
    {
        // decode factor and its reciprocal for (tensor, scale byte)
        const int kv = tid >> 7, s = tid & 127;
        const float dec = e4m3_byte_to_f32((uint32_t)s) * a.g[kv];
        tab.dec[kv][s] = dec;
        tab.inv[kv][s] = (dec == 0.0f) ? 0.0f : 1.0f / dec;
    }
    __syncthreads();

    const int nb = a.D >> 4;
    const int bpr = a.H * nb;                         // blocks per row (all heads)
    if (bpr <= kThreads) {
        const int rows_per_iter = kThreads / bpr;
        const int row_off = tid / bpr;
        if (row_off >= rows_per_iter)
            return;
        const int hc = tid - row_off * bpr;
        const int h = hc / nb, c = hc - (hc / nb) * nb;
        for (int64_t r = (int64_t)blockIdx.x * rows_per_iter + row_off; r < a.nnz;
             r += (int64_t)gridDim.x * rows_per_iter) {
            const int b = a.batch_indices[r];
            const int p = a.positions[r];
            const int64_t page = a.kv_indices[a.kv_indptr[b] + p / a.ps];
            const int slot = p % a.ps;
            quantize_one<BF16, RECIPE>(a, tab, 0, r, h, c, page, slot, HND);
            quantize_one<BF16, RECIPE>(a, tab, 1, r, h, c, page, slot, HND);
        }
    } else {
        for (int64_t r = blockIdx.x; r < a.nnz; r += gridDim.x) {
            const int b = a.batch_indices[r];
            const int p = a.positions[r];
            const int64_t page = a.kv_indices[a.kv_indptr[b] + p / a.ps];
            const int slot = p % a.ps;
            for (int hc = tid; hc < bpr; hc += kThreads) {
                const int h = hc / nb, c = hc - (hc / nb) * nb;
                quantize_one<BF16, RECIPE>(a, tab, 0, r, h, c, page, slot, HND);
                quantize_one<BF16, RECIPE>(a, tab, 1, r, h, c, page, slot, HND);
            }
        }
    }
}

template <bool BF16, int RECIPE>
hipError_t launch2(bool hnd, const AppendArgs &a, int grid, hipStream_t st)
{
    if (hnd)
        hipLaunchKernelGGL((append_kernel<BF16, RECIPE, true>), dim3(grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((append_kernel<BF16, RECIPE, false>), dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch1(int recipe, bool hnd, const AppendArgs &a, int grid, hipStream_t st)
{
    if (recipe == 1)
        return launch2<BF16, 1>(hnd, a, grid, st);
    if (recipe == 2)
        return launch2<BF16, 2>(hnd, a, grid, st);
    return launch2<BF16, 0>(hnd, a, grid, st);
}

}  // namespace

hipError_t launch_quantize_append(const kvfp4_paged_cache_t &c, const void *key, const void *value,
                                  bool in_bf16, int64_t nnz, const int32_t *batch_indices,
                                  const int32_t *positions, const int32_t *kv_indices,
                                  const int32_t *kv_indptr, float k_scale, float v_scale,
                                  const kvfp4_recipe_t *recipe, hipStream_t st)
{
    AppendArgs a;
    a.data[0] = (uint8_t *)c.k_data;
    a.data[1] = (uint8_t *)c.v_data;
    a.sf[0] = (uint8_t *)c.k_sf;
    a.sf[1] = (uint8_t *)c.v_sf;
    a.stride[0] = c.k_page_stride;
    a.stride[1] = c.v_page_stride;
    a.sf_stride[0] = c.k_sf_page_stride;
    a.sf_stride[1] = c.v_sf_page_stride;
    a.in[0] = (const uint8_t *)key;
    a.in[1] = (const uint8_t *)value;
    a.batch_indices = batch_indices;
    a.positions = positions;
    a.kv_indices = kv_indices;
    a.kv_indptr = kv_indptr;
    a.g[0] = k_scale;
    a.g[1] = v_scale;
    a.ps = c.page_size;
    a.H = c.num_kv_heads;
    a.D = c.head_dim;
    a.nnz = nnz;
    a.clamp6 = recipe ? recipe->e4m3_max : 448.0f;
    a.err_mode = recipe ? recipe->err_mode : 0;
    if (nnz == 0)
        return hipSuccess;
    const int bpr = a.H * (a.D >> 4);
    const int64_t rows_per_wg = bpr <= kThreads ? kThreads / bpr : 1;
    const int64_t wgs = (nnz + rows_per_wg - 1) / rows_per_wg;
    // The standard recipe is memory-bound: one workgroup per group of rows
    // balances best. The 4over6 recipes are VALU-bound: a persistent grid
    // builds the LDS tables once per workgroup and overlaps a row's loads
    // with the previous row's arithmetic.
    const int64_t cap = recipe == nullptr ? ((int64_t)1 << 24) : kPersistentWorkgroups;
    const int grid = (int)(wgs < cap ? wgs : cap);
    const bool hnd = c.layout == KVFP4_HND;
    const int rk = recipe == nullptr ? 0 : (recipe->err_mode == KVFP4_ERR_MSE ? 1 : 2);
    return in_bf16 ? launch1<true>(rk, hnd, a, grid, st) : launch1<false>(rk, hnd, a, grid, st);
}

}  // namespace kvfp4

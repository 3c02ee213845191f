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
// The block arithmetic (fp32 operation order, both 4over6 candidates) is
// quant_block.h's quantize_block.
// dec and inv depend only on (tensor, scale byte): each workgroup tabulates
// them for the 127 finite non-negative scale bytes in LDS at start, so a block
// pays one IEEE division (for sf) per candidate and two LDS reads. The E2M1
// encode / decode and the E4M3 encode use gfx950's conversion instructions.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"
#include "quant_block.h"

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
    uint32_t s;
    const uint2 codes = quantize_block<RECIPE>(x, amax, a.g[kv], a.clamp6, tab.dec[kv], tab.inv[kv], s);
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
    switch (recipe) {
    case 1: return launch2<BF16, 1>(hnd, a, grid, st);
    case 2: return launch2<BF16, 2>(hnd, a, grid, st);
    case 3: return launch2<BF16, 3>(hnd, a, grid, st);
    case 4: return launch2<BF16, 4>(hnd, a, grid, st);
    default: return launch2<BF16, 0>(hnd, a, grid, st);
    }
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
    const int rk = recipe_kind(recipe);
    return in_bf16 ? launch1<true>(rk, hnd, a, grid, st) : launch1<false>(rk, hnd, a, grid, st);
}

}  // namespace kvfp4

// append.hip - NVFP4 quantize-append into paged NHD/HND caches for gfx950
// (FlashInfer page flashinfer.page.nvfp4_quantize_append_paged_kv_cache, and
// the "NVFP4 4over6 Recipes" section of the flashinfer.quantization page).
//
// One lane owns one 16-element block of one (row, head) of K or V: it loads
// the block's 32 input bytes (two 16-byte loads, consecutive lanes read
// consecutive blocks of a row), reduces amax in registers, derives the E4M3
// block scale, encodes 16 E2M1 codes and stores 8 packed bytes plus the scale
// byte at (page, slot) from the CSR table. The 4over6 recipe evaluates both
// candidates in the same lane: no cross-lane traffic at all.
//
// fp32 order (bit-exact with the reference reading):
//   sf  = amax / fp32(C * g)                 (IEEE division)
//   s   = E4M3_RNE(min(sf, clamp_C))
//   dec = fp32(E4M3(s) * g),  inv = dec ? fp32(1 / dec) : 0
//   q_i = nearest E2M1 magnitude of |x_i| * inv, sign from x_i
//   4over6: d_i = |x_i| - fp32(dec * q_i); MSE d_i*d_i or MAE |d_i|; pairwise
//   tree over the 16 terms; amax/4 kept only when strictly lower.
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

struct Candidate {
    uint32_t s;
    float dec, inv;
};

__device__ __forceinline__ Candidate make_candidate(float amax, float t, float clamp, float g)
{
    Candidate c;
    const float sf = amax / t;
    c.s = f32_to_e4m3_rne(fminf(sf, clamp));
    c.dec = e4m3_to_f32(c.s) * g;
    c.inv = (c.dec == 0.0f) ? 0.0f : 1.0f / c.dec;
    return c;
}

// 16 magnitudes + the signs of x -> two packed code dwords
__device__ __forceinline__ uint2 pack_codes(const float q[16], const float x[16])
{
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t k = e2m1_mag_to_code(q[i]) | ((__float_as_uint(x[i]) >> 28) & 8u);
        w[i >> 3] |= k << (4 * (i & 7));
    }
    return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ float tree16(float t[16])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = t[2 * i] + t[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = t[2 * i] + t[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0] + t[1];
}

template <bool BF16, bool FOUR_OVER_SIX>
__device__ __forceinline__ void quantize_one(const AppendArgs &a, int kv, int64_t r, int h, int c,
                                             int64_t page, int slot, bool hnd, int err_mode)
{
    const int nb = a.D >> 4;
    float x[16];
    load_block<BF16>(a.in[kv] + (((r * a.H + h) * a.D) + c * 16) * 2, x);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const float g = a.g[kv];

    uint32_t s;
    float q[16];
    const Candidate c6 = make_candidate(amax, 6.0f * g, a.clamp6, g);
    if (!FOUR_OVER_SIX) {
        s = c6.s;
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = e2m1_round_mag(fabsf(x[i]) * c6.inv);
    } else {
        const Candidate c4 = make_candidate(amax, 4.0f * g, 448.0f, g);
        float q6[16], q4[16], t6[16], t4[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float ax = fabsf(x[i]);
            q6[i] = e2m1_round_mag(ax * c6.inv);
            q4[i] = e2m1_round_mag(ax * c4.inv);
            const float d6 = ax - c6.dec * q6[i];
            const float d4 = ax - c4.dec * q4[i];
            t6[i] = err_mode == 0 ? d6 * d6 : fabsf(d6);
            t4[i] = err_mode == 0 ? d4 * d4 : fabsf(d4);
        }
        const float e6 = tree16(t6);
        const float e4 = tree16(t4);
        const bool take4 = e4 < e6;
        s = take4 ? c4.s : c6.s;
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = take4 ? q4[i] : q6[i];
    }
    const uint2 packed = pack_codes(q, x);
    const int64_t row = hnd ? ((int64_t)h * a.ps + slot) : ((int64_t)slot * a.H + h);
    *(uint2 *)(a.data[kv] + page * a.stride[kv] + row * (a.D >> 1) + c * 8) = packed;
    a.sf[kv][page * a.sf_stride[kv] + row * nb + c] = (uint8_t)s;
}

template <bool BF16, bool FOUR_OVER_SIX, bool HND>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a)
{
    const int nb = a.D >> 4;
    const int bpr = a.H * nb;                         // blocks per row (all heads)
    const int tid = threadIdx.x;
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
            quantize_one<BF16, FOUR_OVER_SIX>(a, 0, r, h, c, page, slot, HND, a.err_mode);
            quantize_one<BF16, FOUR_OVER_SIX>(a, 1, r, h, c, page, slot, HND, a.err_mode);
        }
    } else {
        for (int64_t r = blockIdx.x; r < a.nnz; r += gridDim.x) {
            const int b = a.batch_indices[r];
            const int p = a.positions[r];
            const int64_t page = a.kv_indices[a.kv_indptr[b] + p / a.ps];
            const int slot = p % a.ps;
            for (int hc = tid; hc < bpr; hc += kThreads) {
                const int h = hc / nb, c = hc - (hc / nb) * nb;
                quantize_one<BF16, FOUR_OVER_SIX>(a, 0, r, h, c, page, slot, HND, a.err_mode);
                quantize_one<BF16, FOUR_OVER_SIX>(a, 1, r, h, c, page, slot, HND, a.err_mode);
            }
        }
    }
}

template <bool BF16, bool F46>
hipError_t launch2(bool hnd, const AppendArgs &a, int grid, hipStream_t st)
{
    if (hnd)
        hipLaunchKernelGGL((append_kernel<BF16, F46, true>), dim3(grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((append_kernel<BF16, F46, false>), dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
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
    const int grid = (int)(wgs < kPersistentWorkgroups ? wgs : kPersistentWorkgroups);
    const bool hnd = c.layout == KVFP4_HND;
    const bool f46 = recipe != nullptr;
    if (in_bf16)
        return f46 ? launch2<true, true>(hnd, a, grid, st) : launch2<true, false>(hnd, a, grid, st);
    return f46 ? launch2<false, true>(hnd, a, grid, st) : launch2<false, false>(hnd, a, grid, st);
}

}  // namespace kvfp4

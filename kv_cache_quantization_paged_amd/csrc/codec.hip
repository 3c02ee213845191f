// codec.hip - NVFP4 quantize / dequantize of contiguous tensors and whole
// page pools for gfx950 (the "FP4 KV Cache Quantization" section of the
// FlashInfer flashinfer.quantization page: nvfp4_kv_quantize,
// nvfp4_kv_dequantize and nvfp4_quantize_paged_kv_cache).
//
// Both quantizers see their input as units of `bpu` consecutive 16-element
// blocks: a row of a contiguous [rows, cols] tensor, or a page of a 16-bit
// page pool. One lane owns one block (of K and, for a pool, of V): 32 input
// bytes in, 8 code bytes and one scale byte out, the block arithmetic of
// quant_block.h. Lanes follow the blocks in memory order, so the loads and
// the code stores are contiguous across a wavefront. Codes go to
// data + unit * stride + 8 q; the scale of block q goes to
// sf + unit * sf_stride + q, or, for the V scales of an HND pool written
// 4-token interleaved, to the byte of token t, block column c inside the
// (page, head) tile: ((t / 4) * (D / 16) + c) * 4 + t % 4.
//
// The contiguous dequantize is a flat stream: 8 outputs per lane and chunk
// (4 code bytes and the block's scale byte in, 16 bytes out), each
// workgroup on its own contiguous range, whose base sits in scalar registers.
// value = RNE16(fp32(fp32(E4M3(s) * g) * e2m1(c))), as in the paged dequant.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"
#include "quant_block.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;

struct BlockQuantArgs {
    const uint8_t *in[2];      // 16-bit elements, blocks contiguous in unit order
    uint8_t *data[2];
    uint8_t *sf[2];
    int64_t stride[2];         // bytes between units' codes
    int64_t sf_stride[2];      // bytes between units' scales
    int32_t bpu;               // blocks per unit
    int32_t n_blocks;          // units * bpu (per tensor)
    float clamp6;
    int32_t ps, nb;            // pool geometry, for the interleaved V scales
};

// LDS tables of the decode factor and its reciprocal for (tensor, scale byte)
struct CodecTables {
    float dec[2][128];
    float inv[2][128];
};

template <int NT>
__device__ __forceinline__ void build_tables(CodecTables &tab, const float *g0, const float *g1)
{
    const int tid = threadIdx.x;
    const int kv = tid >> 7, s = tid & 127;
    if (kv < NT) {
        const float g = kv ? *g1 : *g0;
        const float dec = e4m3_byte_to_f32((uint32_t)s) * g;
        tab.dec[kv][s] = dec;
        tab.inv[kv][s] = (dec == 0.0f) ? 0.0f : 1.0f / dec;
    }
    __syncthreads();
}

// NT tensors (1: contiguous, 2: K and V of a pool); V_ILV: tensor 1's scales
// 4-token interleaved. The global scales are read-only for the launch.
template <bool BF16, int RECIPE, int NT, bool V_ILV>
__global__ __launch_bounds__(kThreads) void block_quant_kernel(BlockQuantArgs a, const float *__restrict__ g0,
                                                               const float *__restrict__ g1)
{
    __shared__ CodecTables tab;
    build_tables<NT>(tab, g0, g1);
    const float g[2] = {*g0, NT > 1 ? *g1 : 0.0f};
    const int gi = blockIdx.x * kThreads + threadIdx.x;
    if (gi >= a.n_blocks)
        return;
    const int u = gi / a.bpu;
    const int q = gi - u * a.bpu;
#pragma unroll
    for (int kv = 0; kv < NT; ++kv) {
        float x[16];
        load_block<BF16>(a.in[kv] + (int64_t)gi * 32, x);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
        uint32_t s;
        const uint2 codes = quantize_block<RECIPE>(x, amax, g[kv], a.clamp6, tab.dec[kv], tab.inv[kv], s);
        const u32x2 cv = {codes.x, codes.y};
        __builtin_nontemporal_store(cv, (u32x2 *)(a.data[kv] + u * a.stride[kv] + (int64_t)q * 8));
        int sidx = q;
        if (V_ILV && kv == 1) {
            const int row = q / a.nb, c = q - row * a.nb;      // row = h * ps + t
            const int h = row / a.ps, t = row - h * a.ps;
            sidx = h * a.ps * a.nb + ((t >> 2) * a.nb + c) * 4 + (t & 3);
        }
        a.sf[kv][u * a.sf_stride[kv] + sidx] = (uint8_t)s;
    }
}

template <bool BF16, int RECIPE>
void launch_bq(int nt, bool v_ilv, const BlockQuantArgs &a, const float *g0, const float *g1, int grid,
               hipStream_t st)
{
    if (nt == 1)
        hipLaunchKernelGGL((block_quant_kernel<BF16, RECIPE, 1, false>), dim3(grid), dim3(kThreads), 0, st, a, g0, g1);
    else if (v_ilv)
        hipLaunchKernelGGL((block_quant_kernel<BF16, RECIPE, 2, true>), dim3(grid), dim3(kThreads), 0, st, a, g0, g1);
    else
        hipLaunchKernelGGL((block_quant_kernel<BF16, RECIPE, 2, false>), dim3(grid), dim3(kThreads), 0, st, a, g0, g1);
}

template <bool BF16>
void launch_bq_recipe(int rk, int nt, bool v_ilv, const BlockQuantArgs &a, const float *g0, const float *g1,
                      int grid, hipStream_t st)
{
    switch (rk) {
    case 1: launch_bq<BF16, 1>(nt, v_ilv, a, g0, g1, grid, st); break;
    case 2: launch_bq<BF16, 2>(nt, v_ilv, a, g0, g1, grid, st); break;
    case 3: launch_bq<BF16, 3>(nt, v_ilv, a, g0, g1, grid, st); break;
    case 4: launch_bq<BF16, 4>(nt, v_ilv, a, g0, g1, grid, st); break;
    default: launch_bq<BF16, 0>(nt, v_ilv, a, g0, g1, grid, st); break;
    }
}

hipError_t run_block_quant(bool bf16, const kvfp4_recipe_t *recipe, int nt, bool v_ilv, const BlockQuantArgs &a,
                           const float *g0, const float *g1, hipStream_t st)
{
    if (a.n_blocks == 0)
        return hipSuccess;
    const int grid = (int)(((int64_t)a.n_blocks + kThreads - 1) / kThreads);
    const int rk = recipe_kind(recipe);
    if (bf16)
        launch_bq_recipe<true>(rk, nt, v_ilv, a, g0, g1, grid, st);
    else
        launch_bq_recipe<false>(rk, nt, v_ilv, a, g0, g1, grid, st);
    return hipGetLastError();
}

// ------------------------------------------------------------ dequantize --
constexpr int kBatch = 8;                  // chunks per lane
constexpr int kUnit = kBatch * kThreads;   // chunks per workgroup

template <bool BF16>
__device__ __forceinline__ u32x4 decode8(uint32_t codes, float dec)
{
    const f32x2 v0 = fp4x2_to_f32x2<0>(codes);
    const f32x2 v1 = fp4x2_to_f32x2<1>(codes);
    const f32x2 v2 = fp4x2_to_f32x2<2>(codes);
    const f32x2 v3 = fp4x2_to_f32x2<3>(codes);
    u32x4 r;
    if (BF16) {
        r.x = pack_bf16x2(dec * v0.x, dec * v0.y);
        r.y = pack_bf16x2(dec * v1.x, dec * v1.y);
        r.z = pack_bf16x2(dec * v2.x, dec * v2.y);
        r.w = pack_bf16x2(dec * v3.x, dec * v3.y);
    } else {
        r.x = pack_f16x2(dec * v0.x, dec * v0.y);
        r.y = pack_f16x2(dec * v1.x, dec * v1.y);
        r.z = pack_f16x2(dec * v2.x, dec * v2.y);
        r.w = pack_f16x2(dec * v3.x, dec * v3.y);
    }
    return r;
}

// chunk ci (8 elements): codes at 4 ci, scale at ci / 2, output at 16 ci
template <bool BF16>
__global__ __launch_bounds__(kThreads) void contig_dequant_kernel(const uint8_t *codes, const uint8_t *scales,
                                                                  const float *__restrict__ gp, uint8_t *out,
                                                                  int64_t n_chunks)
{
    const float g = *gp;
    const int64_t first = (int64_t)blockIdx.x * kUnit;
    const int64_t left = n_chunks - first;
    const uint32_t n = (uint32_t)(left < kUnit ? left : kUnit);     // chunks of this workgroup (even)
    const rsrc_t src = make_rsrc(codes + first * 4, n * 4u);
    const rsrc_t sfs = make_rsrc(scales + first / 2, n / 2u);
    const rsrc_t dst = make_rsrc(out + first * 16, n * 16u);
    uint32_t c[kBatch], s[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        const uint32_t ci = (uint32_t)(k * kThreads) + threadIdx.x;
        c[k] = buf_load_u32(src, ci * 4u);
        s[k] = buf_load_u8(sfs, ci >> 1);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
        const uint32_t ci = (uint32_t)(k * kThreads) + threadIdx.x;
        buf_store_u32x4_nt(decode8<BF16>(c[k], e4m3_byte_to_f32(s[k]) * g), dst, ci * 16u);
    }
}

}  // namespace

hipError_t launch_quantize_contiguous(const void *x, bool in_bf16, int64_t rows, int64_t cols, const float *g,
                                      const kvfp4_recipe_t *recipe, void *codes, void *scales, hipStream_t st)
{
    BlockQuantArgs a = {};
    a.in[0] = (const uint8_t *)x;
    a.data[0] = (uint8_t *)codes;
    a.sf[0] = (uint8_t *)scales;
    a.stride[0] = cols / 2;
    a.sf_stride[0] = cols / 16;
    a.bpu = (int32_t)(cols / 16);
    a.n_blocks = (int32_t)(rows * (cols / 16));
    a.clamp6 = recipe ? recipe->e4m3_max : 448.0f;
    a.ps = 1;
    a.nb = a.bpu;
    return run_block_quant(in_bf16, recipe, 1, false, a, g, g, st);
}

hipError_t launch_quantize_paged_cache(const kvfp4_paged_cache_t &c, const void *k_in, const void *v_in,
                                       bool in_bf16, const float *k_scale, const float *v_scale,
                                       const kvfp4_recipe_t *recipe, bool v_interleaved, hipStream_t st)
{
    BlockQuantArgs a = {};
    a.in[0] = (const uint8_t *)k_in;
    a.in[1] = (const uint8_t *)v_in;
    a.data[0] = (uint8_t *)c.k_data;
    a.data[1] = (uint8_t *)c.v_data;
    a.sf[0] = (uint8_t *)c.k_sf;
    a.sf[1] = (uint8_t *)c.v_sf;
    a.stride[0] = c.k_page_stride;
    a.stride[1] = c.v_page_stride;
    a.sf_stride[0] = c.k_sf_page_stride;
    a.sf_stride[1] = c.v_sf_page_stride;
    a.nb = c.head_dim / 16;
    a.ps = c.page_size;
    a.bpu = c.page_size * c.num_kv_heads * a.nb;
    a.n_blocks = (int32_t)((int64_t)c.num_pages * a.bpu);
    a.clamp6 = recipe ? recipe->e4m3_max : 448.0f;
    return run_block_quant(in_bf16, recipe, 2, v_interleaved, a, k_scale, v_scale, st);
}

hipError_t launch_dequantize_contiguous(const void *codes, const void *scales, int64_t rows, int64_t cols,
                                        const float *g, void *out, bool out_bf16, hipStream_t st)
{
    const int64_t n_chunks = rows * cols / 8;
    if (n_chunks == 0)
        return hipSuccess;
    const int64_t grid = (n_chunks + kUnit - 1) / kUnit;
    if (out_bf16)
        hipLaunchKernelGGL((contig_dequant_kernel<true>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                           (const uint8_t *)codes, (const uint8_t *)scales, g, (uint8_t *)out, n_chunks);
    else
        hipLaunchKernelGGL((contig_dequant_kernel<false>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                           (const uint8_t *)codes, (const uint8_t *)scales, g, (uint8_t *)out, n_chunks);
    return hipGetLastError();
}

}  // namespace kvfp4

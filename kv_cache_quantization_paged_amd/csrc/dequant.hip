// dequant.hip - paged NVFP4 gather-dequantize for gfx950
// (FlashInfer page flashinfer.quantization.nvfp4_kv_dequantize_paged).
//
// Work item ("tile"): one logical page j of one request b for K or for V.
// Its output rows out[b, j*ps + t, h, :] (t < tokens of the page, every head)
// are one contiguous run of n_tok*H*D 16-bit values, so every wavefront store
// is a coalesced 16-byte-per-lane stream whatever the cache layout; the NHD/HND
// difference is only where a lane reads its 8 code bytes and scale byte.
// A persistent grid walks the B * ceil(T/ps) * 2 tiles; tiles past a request's
// length cost a few scalar instructions and are skipped.
//
// Per lane and per 16-element block: 8 code bytes + 1 scale byte in, 32 bytes
// out. value = RNE16(fp32(fp32(E4M3(s) * g) * e2m1(c))); the product order is
// the one the oracle states (scale times global first).
#include "kvfp4_internal.h"
#include "nvfp4_device.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct DequantArgs {
    const uint8_t *data[2];
    const uint8_t *sf[2];
    int64_t stride[2];
    int64_t sf_stride[2];
    const void *block_tables;
    int64_t bt_row_stride;
    const int32_t *seq_lens;
    const float *scale[2];
    uint16_t *out[2];
    int32_t ps, H, D, T;
    int32_t pages_per_req;   // ceil(T / ps)
    int64_t num_tiles;       // B * pages_per_req * 2
};

// 8 code bytes (16 elements) -> 8 packed 16-bit pairs
template <bool BF16>
__device__ __forceinline__ void decode_block(uint32_t c0, uint32_t c1, float dec, uint32_t out[8])
{
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t c = w ? c1 : c0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (c >> (8 * i)) & 0xFu;
            const uint32_t hi = (c >> (8 * i + 4)) & 0xFu;
            float ylo = dec * e2m1_code_to_mag(lo & 7u);
            float yhi = dec * e2m1_code_to_mag(hi & 7u);
            ylo = __uint_as_float(__float_as_uint(ylo) ^ ((lo & 8u) << 28));
            yhi = __uint_as_float(__float_as_uint(yhi) ^ ((hi & 8u) << 28));
            out[w * 4 + i] = BF16 ? pack_bf16x2(ylo, yhi) : pack_f16x2(ylo, yhi);
        }
    }
}

template <bool HND, bool BF16, bool BT64>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs a)
{
    const int nb = a.D >> 4;                       // blocks per (token, head) row
    const int rows_per_iter = kThreads / nb;       // rows the workgroup covers per step
    const int tid = threadIdx.x;
    const bool lane_active = tid < rows_per_iter * nb;
    const int c = tid % nb;
    const int row0 = tid / nb;
    const int t_step = rows_per_iter / a.H, h_step = rows_per_iter % a.H;
    const float g0 = *a.scale[0], g1 = *a.scale[1];

    for (int64_t tile = blockIdx.x; tile < a.num_tiles; tile += gridDim.x) {
        const int kv = (int)(tile & 1);
        const int64_t bj = tile >> 1;
        const int b = (int)(bj / a.pages_per_req);
        const int j = (int)(bj - (int64_t)b * a.pages_per_req);
        const int len = min(a.seq_lens[b], a.T);
        const int t_first = j * a.ps;
        if (t_first >= len)
            continue;
        const int n_tok = min(a.ps, len - t_first);
        const int64_t page = BT64 ? ((const int64_t *)a.block_tables)[b * a.bt_row_stride + j]
                                  : (int64_t)((const int32_t *)a.block_tables)[b * a.bt_row_stride + j];
        const uint8_t *src = a.data[kv] + page * a.stride[kv];
        const uint8_t *sfs = a.sf[kv] + page * a.sf_stride[kv];
        uint16_t *dst = a.out[kv] + ((int64_t)b * a.T + t_first) * a.H * a.D;
        const float g = kv ? g1 : g0;
        const int n_rows = n_tok * a.H;
        if (!lane_active)
            continue;

        // (t, h) of this lane's first row, advanced incrementally
        int t = row0 / a.H, h = row0 - (row0 / a.H) * a.H;
        for (int row = row0; row < n_rows; row += kUnroll * rows_per_iter) {
            uint2 codes[kUnroll];
            uint32_t sbyte[kUnroll];
            int rows[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                rows[u] = row + u * rows_per_iter;
                const int in_row = HND ? (h * a.ps + t) : rows[u];
                if (rows[u] < n_rows) {
                    codes[u] = *(const uint2 *)(src + (int64_t)in_row * (a.D >> 1) + c * 8);
                    sbyte[u] = sfs[(int64_t)in_row * nb + c];
                }
                h += h_step;
                t += t_step;
                if (h >= a.H) {
                    h -= a.H;
                    t += 1;
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (rows[u] < n_rows) {
                    const float dec = e4m3_to_f32(sbyte[u]) * g;
                    uint32_t o[8];
                    decode_block<BF16>(codes[u].x, codes[u].y, dec, o);
                    uint4 *p = (uint4 *)(dst + (int64_t)rows[u] * a.D + c * 16);
                    p[0] = make_uint4(o[0], o[1], o[2], o[3]);
                    p[1] = make_uint4(o[4], o[5], o[6], o[7]);
                }
            }
        }
    }
}

template <bool HND, bool BF16>
hipError_t launch3(bool bt64, const DequantArgs &a, int grid, hipStream_t st)
{
    if (bt64)
        hipLaunchKernelGGL((dequant_kernel<HND, BF16, true>), dim3(grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((dequant_kernel<HND, BF16, false>), dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize_paged(const kvfp4_paged_cache_t &c, const void *block_tables, bool bt64,
                                   int64_t bt_row_stride, const int32_t *seq_lens, int32_t batch,
                                   const float *k_scale, const float *v_scale, void *out_k, void *out_v,
                                   bool out_bf16, int32_t max_seq_len, hipStream_t st)
{
    DequantArgs a;
    a.data[0] = (const uint8_t *)c.k_data;
    a.data[1] = (const uint8_t *)c.v_data;
    a.sf[0] = (const uint8_t *)c.k_sf;
    a.sf[1] = (const uint8_t *)c.v_sf;
    a.stride[0] = c.k_page_stride;
    a.stride[1] = c.v_page_stride;
    a.sf_stride[0] = c.k_sf_page_stride;
    a.sf_stride[1] = c.v_sf_page_stride;
    a.block_tables = block_tables;
    a.bt_row_stride = bt_row_stride;
    a.seq_lens = seq_lens;
    a.scale[0] = k_scale;
    a.scale[1] = v_scale;
    a.out[0] = (uint16_t *)out_k;
    a.out[1] = (uint16_t *)out_v;
    a.ps = c.page_size;
    a.H = c.num_kv_heads;
    a.D = c.head_dim;
    a.T = max_seq_len;
    a.pages_per_req = (max_seq_len + c.page_size - 1) / c.page_size;
    a.num_tiles = (int64_t)batch * a.pages_per_req * 2;
    if (a.num_tiles == 0)
        return hipSuccess;
    const int grid = (int)(a.num_tiles < (int64_t)kPersistentWorkgroups ? a.num_tiles : kPersistentWorkgroups);
    const bool hnd = c.layout == KVFP4_HND;
    if (hnd)
        return out_bf16 ? launch3<true, true>(bt64, a, grid, st) : launch3<true, false>(bt64, a, grid, st);
    return out_bf16 ? launch3<false, true>(bt64, a, grid, st) : launch3<false, false>(bt64, a, grid, st);
}

}  // namespace kvfp4

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
// pays two LDS reads per candidate, and its scale code a multiply (an IEEE
// division only near an E4M3 rounding midpoint). The E2M1 encode / decode and
// the E4M3 encode use gfx950's conversion instructions.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"
#include "quant_block.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;

// Row-kernel shape per recipe, as measured on the 4over6 workload (65,536
// rows of 8 x 128 bf16): the fp32-error recipes need their 96 VGPRs (5
// workgroups per CU) and copy the prefetched slice into place; the
// fp16-error recipes fit 80 VGPRs (6 per CU) with two slice buffers that
// trade roles, which took them from about 77-80 us to 74-75 us.
constexpr int row_workgroups_per_cu(int recipe) { return recipe >= 3 ? 6 : 5; }
constexpr bool row_ping_pong(int recipe) { return recipe >= 3; }

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

// Rows whose blocks fill whole wavefronts (H * D / 16 a multiple of 64: 8
// heads of 128, 4 of 256, 16 of 64, ...): each wavefront takes a 64-block
// slice of one row, so the row's request, position, page and slot are
// wave-uniform scalar loads, and every address is a scalar base plus a
// per-lane constant (no per-lane 64-bit address arithmetic). The index arrays
// are read-only for the launch: as __restrict__ kernel parameters their
// uniform reads are scalar loads.
template <bool BF16, int RECIPE, bool HND>
__global__ __launch_bounds__(kThreads, row_workgroups_per_cu(RECIPE)) void append_rows_kernel(AppendArgs a,
                                                                  const int32_t *__restrict__ batch_indices,
                                                                  const int32_t *__restrict__ positions,
                                                                  const int32_t *__restrict__ kv_indices,
                                                                  const int32_t *__restrict__ kv_indptr)
{
    __shared__ ScaleTables tab;
    const int tid = threadIdx.x;
    {
        const int kv = tid >> 7, s = tid & 127;
        const float dec = e4m3_byte_to_f32((uint32_t)s) * a.g[kv];
        tab.dec[kv][s] = dec;
        tab.inv[kv][s] = (dec == 0.0f) ? 0.0f : 1.0f / dec;
    }
    __syncthreads();

    const int nb = a.D >> 4;
    const int slices = (a.H * nb) >> 6;                     // wavefronts per row
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const uint32_t row_in = (uint32_t)a.H * a.D * 2;        // input bytes per row
    const uint32_t page_bytes = (uint32_t)(a.ps * a.H * (a.D >> 1));
    const uint32_t page_sf_bytes = (uint32_t)(a.ps * a.H * nb);
    // wavefront w of the grid takes row slices w, w + step, ... in (row,
    // slice) order, advanced by additions (no division per slice)
    const int step = (int)gridDim.x * (kThreads / 64);
    const int step_rows = step / slices, step_slices = step - step_rows * slices;
    // one row slice: its destination (scalar) and its input words (per lane)
    struct Slice {
        int64_t page;
        int slot, hc;
        u32x4 in[2][2];
    };
    // the input loads first: they need only the row, so they are in flight
    // while the request -> indptr -> page chain of scalar loads resolves
    auto fetch = [&](int64_t r, int slice, Slice &sl) {
        sl.hc = slice * 64 + lane;                           // this lane's block of the row
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            const rsrc_t in = make_rsrc(a.in[kv] + r * row_in, row_in);
            sl.in[kv][0] = buf_load_u32x4(in, (uint32_t)sl.hc * 32u);
            sl.in[kv][1] = buf_load_u32x4(in, (uint32_t)sl.hc * 32u + 16u);
        }
        const int b = batch_indices[r];
        const int p = positions[r];
        sl.page = kv_indices[kv_indptr[b] + p / a.ps];
        sl.slot = p % a.ps;
    };
    auto quantize = [&](const Slice &cur) {
        const int h = cur.hc / nb, c = cur.hc - (cur.hc / nb) * nb;
        // byte offsets of the block's codes and scale inside the page
        const uint32_t off_c = HND ? (uint32_t)((h * a.ps + cur.slot) * (a.D >> 1) + c * 8)
                                   : (uint32_t)(cur.slot * a.H * (a.D >> 1) + cur.hc * 8);
        const uint32_t off_s = HND ? (uint32_t)((h * a.ps + cur.slot) * nb + c)
                                   : (uint32_t)(cur.slot * a.H * nb + cur.hc);
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            const uint32_t w[8] = {cur.in[kv][0].x, cur.in[kv][0].y, cur.in[kv][0].z, cur.in[kv][0].w,
                                   cur.in[kv][1].x, cur.in[kv][1].y, cur.in[kv][1].z, cur.in[kv][1].w};
            float x[16];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[2 * i] = BF16 ? bf16_lo(w[i]) : f16_lo(w[i]);
                x[2 * i + 1] = BF16 ? bf16_hi(w[i]) : f16_hi(w[i]);
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
            uint32_t sc;
            const uint2 codes = quantize_block<RECIPE>(x, amax, a.g[kv], a.clamp6, tab.dec[kv], tab.inv[kv], sc);
            const rsrc_t dd = make_rsrc(a.data[kv] + cur.page * a.stride[kv], page_bytes);
            const rsrc_t ds = make_rsrc(a.sf[kv] + cur.page * a.sf_stride[kv], page_sf_bytes);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{codes.x, codes.y}, dd, (int)off_c, 0, kStreamStore);
            buf_store_u8(sc, ds, off_s);
        }
    };
    // the slice after (r, slice) in this wavefront's sequence
    auto advance = [&](int64_t &r, int &slice) {
        r += step_rows;
        slice += step_slices;
        if (slice >= slices) {
            slice -= slices;
            ++r;
        }
    };
    // software pipeline: the next slice's index lookups and input loads are
    // in flight while the current slice is quantized (a wait for the current
    // loads does not wait for the stores issued after them)
    const int first = (int)blockIdx.x * (kThreads / 64) + wave;
    int64_t r = uniform(first / slices);
    int slice = uniform(first - (first / slices) * slices);
    if (r >= a.nnz)
        return;
    Slice s0, s1;
    fetch(r, slice, s0);
    if constexpr (row_ping_pong(RECIPE)) {
        // two slice buffers that trade roles: no copy of the prefetched words
        for (;;) {
            advance(r, slice);
            const bool more1 = r < a.nnz;
            if (more1)
                fetch(r, slice, s1);
            quantize(s0);
            if (!more1)
                break;
            advance(r, slice);
            const bool more0 = r < a.nnz;
            if (more0)
                fetch(r, slice, s0);
            quantize(s1);
            if (!more0)
                break;
        }
    } else {
        // the prefetched slice is copied into place (unrolling this loop
        // spills the fp32-error recipes at their register budget)
        for (;;) {
            advance(r, slice);
            const bool more = r < a.nnz;
            if (more)
                fetch(r, slice, s1);
            quantize(s0);
            if (!more)
                break;
            s0 = s1;
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

template <bool BF16, int RECIPE>
hipError_t launch2_rows(bool hnd, const AppendArgs &a, int grid, hipStream_t st)
{
    if (hnd)
        hipLaunchKernelGGL((append_rows_kernel<BF16, RECIPE, true>), dim3(grid), dim3(kThreads), 0, st, a,
                           a.batch_indices, a.positions, a.kv_indices, a.kv_indptr);
    else
        hipLaunchKernelGGL((append_rows_kernel<BF16, RECIPE, false>), dim3(grid), dim3(kThreads), 0, st, a,
                           a.batch_indices, a.positions, a.kv_indices, a.kv_indptr);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch1(int recipe, bool hnd, bool rows, const AppendArgs &a, int grid, hipStream_t st)
{
    if (rows) {
        switch (recipe) {
        case 1: return launch2_rows<BF16, 1>(hnd, a, grid, st);
        case 2: return launch2_rows<BF16, 2>(hnd, a, grid, st);
        case 3: return launch2_rows<BF16, 3>(hnd, a, grid, st);
        case 4: return launch2_rows<BF16, 4>(hnd, a, grid, st);
        default: return launch2_rows<BF16, 0>(hnd, a, grid, st);
        }
    }
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
    // 4over6 rows that fill whole wavefronts take the pipelined,
    // scalar-addressed kernel (a row's input and a page must then stay within
    // 32-bit buffer offsets). The standard recipe keeps the flat kernel: on
    // the 4over6 workload's rows it measured 63.4 us against 65.9 us for the
    // row kernel, whose pipelining has nothing to overlap at one row per wave.
    const bool rows = recipe != nullptr && bpr % 64 == 0 && (int64_t)a.H * a.D * 2 < ((int64_t)1 << 31) &&
                      (int64_t)a.ps * a.H * a.D < ((int64_t)1 << 31);
    const int64_t rows_per_wg = bpr <= kThreads ? kThreads / bpr : 1;
    const int64_t wgs = rows ? (nnz * (bpr / 64) + 3) / 4 : (nnz + rows_per_wg - 1) / rows_per_wg;
    // The standard recipe is memory-bound: one workgroup per group of rows
    // balances best. The 4over6 recipes are VALU-bound: a persistent grid
    // builds the LDS tables once per workgroup and overlaps a row's loads
    // with the previous row's arithmetic. The row kernel's grid is what stays
    // resident (its occupancy bound per CU): on the 4over6 workload a larger
    // grid, which runs in a second partial round, measured 3-5 us slower for
    // the fp16-error recipes.
    int64_t cap = recipe == nullptr ? ((int64_t)1 << 24) : kPersistentWorkgroups;
    if (rows) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        cap = (int64_t)(cus > 0 ? cus : 1) * row_workgroups_per_cu(recipe_kind(recipe));
    }
    const int grid = (int)(wgs < cap ? wgs : cap);
    const bool hnd = c.layout == KVFP4_HND;
    const int rk = recipe_kind(recipe);
    return in_bf16 ? launch1<true>(rk, hnd, rows, a, grid, st) : launch1<false>(rk, hnd, rows, a, grid, st);
}

}  // namespace kvfp4

// materialize.hip - paged NVFP4 -> float8_e4m3fn page copy for gfx950
// (FlashInfer page flashinfer.quantization.kernels.nvfp4_kv_materialize.
// nvfp4_kv_materialize_fp8 and NVFP4KVMaterializer.run() on the
// flashinfer.quantization page).
//
// An HND page [H, ps, D/2] codes + [H, ps, D/16] scales maps element for
// element, in the same (h, t, e) order, onto the K or V half [H, ps, D] of an
// FP8 output page, so each lane streams one 16-element block: 8 code bytes and
// one scale byte in, 16 FP8 bytes out, with consecutive lanes on consecutive
// blocks. The output byte depends only on (scale byte, code): every
// workgroup first tabulates, in LDS, the 8 output magnitudes of each of the
// 256 scale bytes (the product E2M1 x E4M3 is exact in fp32 and is rounded
// once, saturating at 448); a block then needs one 8-byte LDS read and a few
// v_perm byte selects per 8 elements. The sign is code sign XOR scale sign.
//
// Work list: the output pages 1 .. kv_page_indptr[B] the requests reserve,
// walked by a persistent grid (the table above is built once per workgroup).
// Output page p + 1 belongs to the request b with indptr[b] <= p <
// indptr[b + 1] (a binary search over the indptr, in scalar registers) and is
// its page j = p - indptr[b]; it is written only when j < ceil(seq_len / ps),
// so reserved-but-unused pages and everything past kv_page_indptr[B] stay
// untouched. Walking reserved pages rather than the B x max_pages_per_seq
// table keeps the work per workgroup even when lengths differ widely.
// Workgroup 0 also zeroes output page 0.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;

struct MatArgs {
    const uint8_t *data[2];
    const uint8_t *sf[2];
    int64_t stride[2];
    int64_t sf_stride[2];
    const int32_t *bt;
    int64_t bt_row_stride, bt_kv_stride;
    const int32_t *seq_lens, *indptr;
    uint8_t *out;
    int32_t *table;
    int32_t ps, H, D;
    int32_t maxp;          // max_pages_per_seq: columns of the FP8 block table
    int32_t batch;
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 8 codes in `w` (element 2i in the low nibble of byte i) -> 8 FP8 bytes
__device__ __forceinline__ uint2 convert8(uint32_t w, uint2 lut, uint32_t smask)
{
    const uint32_t even = perm(lut.y, lut.x, w & 0x07070707u) ^ (((w << 4) & 0x80808080u) ^ smask);
    const uint32_t odd = perm(lut.y, lut.x, (w >> 4) & 0x07070707u) ^ ((w & 0x80808080u) ^ smask);
    return make_uint2(perm(odd, even, 0x05010400u), perm(odd, even, 0x07030602u));
}

template <bool INTERLEAVED, bool SHARED>
__global__ __launch_bounds__(kThreads) void materialize_kernel(MatArgs a)
{
    __shared__ uint2 lut[256];
    const int tid = threadIdx.x;
    {
        // output magnitude byte for (scale byte = tid, code magnitude k)
        const float sv = e4m3_to_f32((uint32_t)tid & 0x7Fu);
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float p = e2m1_code_to_mag((uint32_t)k) * sv;
            const uint32_t byte = f32_to_e4m3_satfinite(p, 0u);
            if (k < 4)
                lo |= byte << (8 * k);
            else
                hi |= byte << (8 * (k - 4));
        }
        lut[tid] = make_uint2(lo, hi);
    }
    __syncthreads();

    const int nb = a.D >> 4;
    const int blocks_per_half = a.H * a.ps * nb;
    const int64_t half_bytes = (int64_t)a.H * a.ps * a.D;

    if (blockIdx.x == 0) {
        uint4 *z = (uint4 *)a.out;
        for (int64_t i = tid; i < 2 * half_bytes / 16; i += kThreads)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    // block q = tid + k * kThreads of a half page is (h, t, c) with
    // q = (h * ps + t) * nb + c; the thread advances it by kThreads blocks
    const int c_step = kThreads % nb;
    const int t_all = kThreads / nb;
    const int t_step = t_all % a.ps, h_step = t_all / a.ps;
    const int c0 = tid % nb, t0 = (tid / nb) % a.ps, h0 = tid / (nb * a.ps);

    const int n_work = a.batch > 0 ? a.indptr[a.batch] : 0;
    for (int p = blockIdx.x; p < n_work; p += gridDim.x) {
        int lo = 0, hi = a.batch;              // indptr[lo] <= p < indptr[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.indptr[mid] <= p)
                lo = mid;
            else
                hi = mid;
        }
        const int b = lo;
        const int j = p - a.indptr[b];
        const int n_pages = (a.seq_lens[b] + a.ps - 1) / a.ps;
        if (j < 0 || j >= n_pages || j >= a.maxp)
            continue;
        const int64_t dst = (int64_t)p + 1;
        const int32_t *row = a.bt + b * a.bt_row_stride;
        const int64_t pk = row[j];
        const int64_t pv = SHARED ? pk : row[a.bt_kv_stride + j];
        if (tid == 0)
            a.table[(int64_t)b * a.maxp + j] = (int32_t)dst;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            const int64_t page = kv ? pv : pk;
            const uint8_t *src = a.data[kv] + page * a.stride[kv];
            const uint8_t *sfs = a.sf[kv] + page * a.sf_stride[kv];
            uint4 *o = (uint4 *)(a.out + (dst * 2 + kv) * half_bytes);
            int c = c0, t = t0, h = h0;
            for (int q = tid; q < blocks_per_half; q += kThreads) {
                const uint2 codes = *(const uint2 *)(src + (int64_t)q * 8);
                const int sidx = (INTERLEAVED && kv == 1) ? (h * a.ps + (t & ~3)) * nb + c * 4 + (t & 3) : q;
                const uint32_t sb = sfs[sidx];
                const uint2 l = lut[sb];
                const uint32_t smask = (sb & 0x80u) ? 0x80808080u : 0u;
                const uint2 lo = convert8(codes.x, l, smask);
                const uint2 hi = convert8(codes.y, l, smask);
                const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
                __builtin_nontemporal_store(v, (u32x4 *)&o[q]);   // the FP8 copy is read by a later kernel only
                c += c_step;
                int carry = c >= nb;
                c -= carry ? nb : 0;
                t += t_step + carry;
                h += h_step;
                if (t >= a.ps) {
                    t -= a.ps;
                    h += 1;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_materialize_fp8(const kvfp4_paged_cache_t &c, bool v_interleaved, const int32_t *bt,
                                  bool shared, int64_t bt_row_stride, int64_t bt_kv_stride,
                                  const int32_t *seq_lens, const int32_t *indptr, int32_t batch,
                                  void *out, int32_t *table, int32_t maxp, hipStream_t st)
{
    MatArgs a;
    a.data[0] = (const uint8_t *)c.k_data;
    a.data[1] = (const uint8_t *)c.v_data;
    a.sf[0] = (const uint8_t *)c.k_sf;
    a.sf[1] = (const uint8_t *)c.v_sf;
    a.stride[0] = c.k_page_stride;
    a.stride[1] = c.v_page_stride;
    a.sf_stride[0] = c.k_sf_page_stride;
    a.sf_stride[1] = c.v_sf_page_stride;
    a.bt = bt;
    a.bt_row_stride = bt_row_stride;
    a.bt_kv_stride = bt_kv_stride;
    a.seq_lens = seq_lens;
    a.indptr = indptr;
    a.out = (uint8_t *)out;
    a.table = table;
    a.ps = c.page_size;
    a.H = c.num_kv_heads;
    a.D = c.head_dim;
    a.maxp = maxp;
    a.batch = batch;
    // the number of reserved pages lives on the device: a fixed persistent
    // grid (at least one workgroup, which zeroes page 0 for an empty batch)
    const int64_t pairs = (int64_t)batch * maxp;
    const int64_t want = pairs > 0 ? pairs : 1;
    const int grid = (int)(want < kPersistentWorkgroups ? want : kPersistentWorkgroups);
    if (v_interleaved) {
        if (shared)
            hipLaunchKernelGGL((materialize_kernel<true, true>), dim3(grid), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((materialize_kernel<true, false>), dim3(grid), dim3(kThreads), 0, st, a);
    } else {
        if (shared)
            hipLaunchKernelGGL((materialize_kernel<false, true>), dim3(grid), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((materialize_kernel<false, false>), dim3(grid), dim3(kThreads), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace kvfp4

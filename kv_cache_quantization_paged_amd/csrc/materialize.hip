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
// Work list: the B x max_pages_per_seq (request, page) pairs, walked by a
// persistent grid; pairs past a request's ceil(seq_len / ps) pages are
// skipped, so no page beyond kv_page_indptr[B] is touched. Workgroup 0 also
// zeroes output page 0.
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
    int64_t num_pairs;     // B * maxp
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
    const int blocks_per_head = a.ps * nb;
    const int blocks_per_half = a.H * blocks_per_head;
    const int64_t half_bytes = (int64_t)a.H * a.ps * a.D;

    if (blockIdx.x == 0) {
        uint4 *z = (uint4 *)a.out;
        for (int64_t i = tid; i < 2 * half_bytes / 16; i += kThreads)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    // per-thread (h, t, c) of block q = tid + k * kThreads, advanced incrementally
    const int q_step_h = kThreads / blocks_per_head;
    const int q_step_r = kThreads - q_step_h * blocks_per_head;

    for (int64_t pair = blockIdx.x; pair < a.num_pairs; pair += gridDim.x) {
        const int b = (int)(pair / a.maxp);
        const int j = (int)(pair - (int64_t)b * a.maxp);
        const int n_pages = (a.seq_lens[b] + a.ps - 1) / a.ps;
        if (j >= n_pages)
            continue;
        const int64_t dst = (int64_t)a.indptr[b] + j + 1;
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
            uint8_t *o = a.out + (dst * 2 + kv) * half_bytes;
            int hh = tid / blocks_per_head;
            int rem = tid - hh * blocks_per_head;
            for (int q = tid; q < blocks_per_half; q += kThreads) {
                const uint2 codes = *(const uint2 *)(src + (int64_t)q * 8);
                uint32_t sidx = (uint32_t)q;
                if (INTERLEAVED && kv == 1) {
                    const int t = rem / nb, c = rem - (rem / nb) * nb;
                    sidx = (uint32_t)(hh * blocks_per_head + ((t >> 2) * nb + c) * 4 + (t & 3));
                }
                const uint32_t s = sfs[sidx];
                const uint2 l = lut[s];
                const uint32_t smask = (s & 0x80u) ? 0x80808080u : 0u;
                const uint2 lo = convert8(codes.x, l, smask);
                const uint2 hi = convert8(codes.y, l, smask);
                *(uint4 *)(o + (int64_t)q * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
                hh += q_step_h;
                rem += q_step_r;
                if (rem >= blocks_per_head) {
                    rem -= blocks_per_head;
                    hh += 1;
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
    a.num_pairs = (int64_t)batch * maxp;
    // at least one workgroup, which zeroes page 0 even for an empty batch
    const int64_t want = a.num_pairs > 0 ? a.num_pairs : 1;
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

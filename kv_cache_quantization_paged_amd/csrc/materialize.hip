// materialize.hip - paged NVFP4 -> float8_e4m3fn page copy for gfx950
// (FlashInfer page flashinfer.quantization.kernels.nvfp4_kv_materialize.
// nvfp4_kv_materialize_fp8 and NVFP4KVMaterializer.run() on the
// flashinfer.quantization page).
//
// An HND page [H, ps, D/2] codes + [H, ps, D/16] scales maps element for
// element, in the same (h, t, e) order, onto the K or V half [H, ps, D] of an
// FP8 output page, so each lane streams 16-element blocks: 8 code bytes and
// one scale byte in, 16 FP8 bytes out, with consecutive lanes on consecutive
// blocks (a wavefront store writes 1 KiB of contiguous output). A wavefront
// fetches the scale bytes of its 128 blocks per tensor as 32 dwords and hands
// each lane its byte with ds_bpermute: per lane and tensor one dword load
// instead of two byte loads, measured 2.4% faster on the whole call. The output
// byte depends only on (scale byte, code): every workgroup tabulates, in LDS,
// the 8 output magnitudes of each of the 256 scale bytes (the product
// E2M1 x E4M3 is exact in fp32 and is rounded once, saturating at 448); a
// block then needs one 8-byte LDS read and a few v_perm byte selects per 8
// elements. The sign is code sign XOR scale sign.
//
// Work item: a part of output page p + 1 for p < kv_page_indptr[B], one per
// workgroup. The page belongs to the request b with
// indptr[b] <= p < indptr[b + 1] (a binary search over the indptr in scalar
// registers) and is that request's page j = p - indptr[b]; it is written only when j < ceil(seq_len / ps), so
// reserved-but-unused pages and everything past kv_page_indptr[B] stay
// untouched. Indexing reserved pages rather than the B x max_pages_per_seq
// table gives every workgroup the same work however lengths are spread. An
// item issues all its loads (K and V) before its first store and builds the
// table while the loads are in flight. Workgroup 0 also zeroes output page 0.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;
// blocks per lane and tensor in one work item: half a page (8 KiB of FP8
// output per tensor) at 16 tokens x 8 heads x 128. With the non-temporal
// loads, half pages measured 1.3% faster than whole pages; larger pages
// split into more items.
constexpr int kRound = 2;
constexpr uint32_t kSpan = kRound * 64;    // blocks per wavefront and tensor
constexpr int64_t kMaxGrid = 1 << 20;      // work items past the grid loop round

struct MatArgs {
    const uint8_t *data[2];
    const uint8_t *sf[2];
    int64_t stride[2];
    int64_t sf_stride[2];
    int64_t bt_row_stride, bt_kv_stride;
    uint8_t *out;
    int32_t *table;
    int32_t ps, H, D;
    int32_t maxp;          // max_pages_per_seq: columns of the FP8 block table
    int32_t batch;
    int32_t parts;         // work items per page: ceil(blocks per half page / (kRound * kThreads))
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 8 codes in `w` (element 2i in the low nibble of byte i) -> 8 FP8 bytes
__device__ __forceinline__ uint2 convert8(uint32_t w, u32x2 lut, uint32_t smask)
{
    const uint32_t even = perm(lut.y, lut.x, w & 0x07070707u) ^ (((w << 4) & 0x80808080u) ^ smask);
    const uint32_t odd = perm(lut.y, lut.x, (w >> 4) & 0x07070707u) ^ ((w & 0x80808080u) ^ smask);
    return make_uint2(perm(odd, even, 0x05010400u), perm(odd, even, 0x07030602u));
}

// byte offset of block q's V scale in a page whose scales are 4-token
// interleaved: block q is (row, c) with row = q / nb = h ps + t (ps % 4 == 0,
// so row % 4 = t % 4), and its scale sits at (row - row % 4) nb + 4 c + row % 4.
// When nb divides 32, these offsets for a wavefront's kSpan blocks (whole
// groups of 4 rows) are the same kSpan bytes as for linear scales; nb is then
// a power of two (2^nbs).
__device__ __forceinline__ uint32_t v_scale_index(uint32_t q, uint32_t nb)
{
    const uint32_t row = q / nb, c = q - row * nb;
    return (row & ~3u) * nb + 4u * c + (row & 3u);
}
__device__ __forceinline__ uint32_t v_scale_index_pow2(uint32_t q, uint32_t nbs)
{
    const uint32_t row = q >> nbs, c = q & ((1u << nbs) - 1u);
    return ((row & ~3u) << nbs) + 4u * c + (row & 3u);
}

// the index arrays are read-only for the whole launch: as __restrict__ kernel
// parameters their wave-uniform reads are scalar loads
template <bool INTERLEAVED, bool SHARED, bool V_BYTES>
__global__ __launch_bounds__(kThreads) void materialize_kernel(MatArgs a, const int32_t *__restrict__ bt,
                                                               const int32_t *__restrict__ seq_lens,
                                                               const int32_t *__restrict__ indptr)
{
    __shared__ u32x2 lut[256];
    const int tid = threadIdx.x;
    const int nb = a.D >> 4;
    const int bph = a.H * a.ps * nb;                       // blocks per half page
    const uint32_t half_bytes = (uint32_t)bph * 16u;       // FP8 bytes per half page

    if (blockIdx.x == 0) {
        const rsrc_t z = make_rsrc(a.out, 2u * half_bytes);
        for (uint32_t i = tid; i < 2u * (uint32_t)bph; i += kThreads)
            buf_store_u32x4(u32x4{0u, 0u, 0u, 0u}, z, i * 16u);
    }

    bool have_lut = false;
    const int64_t n_work = a.batch > 0 ? indptr[a.batch] : 0;
    const int64_t n_items = n_work * a.parts;
    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int p = (int)(item / a.parts);
        const int part = (int)(item - (int64_t)p * a.parts);
        int lo = 0, hi = a.batch;              // indptr[lo] <= p < indptr[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (indptr[mid] <= p)
                lo = mid;
            else
                hi = mid;
        }
        const int b = lo;
        const int j = p - indptr[b];
        const int n_pages = (seq_lens[b] + a.ps - 1) / a.ps;
        if (j >= n_pages || j >= a.maxp)
            continue;
        const int64_t dst = (int64_t)p + 1;
        const int32_t *row = bt + b * a.bt_row_stride;
        const int64_t pg[2] = {row[j], SHARED ? row[j] : row[a.bt_kv_stride + j]};
        if (part == 0 && tid == 0)
            a.table[(int64_t)b * a.maxp + j] = (int32_t)dst;
        rsrc_t src[2], sfs[2], dsts[2];
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            src[kv] = make_rsrc(a.data[kv] + pg[kv] * a.stride[kv], (uint32_t)bph * 8u);
            sfs[kv] = make_rsrc(a.sf[kv] + pg[kv] * a.sf_stride[kv], (uint32_t)bph);
            dsts[kv] = make_rsrc(a.out + (dst * 2 + kv) * (int64_t)half_bytes, half_bytes);
        }
        // a wavefront takes kSpan consecutive blocks of each tensor, 64 per round
        const int base = part * kRound * kThreads;
        const int lane = tid & 63;
        const uint32_t nbs = (uint32_t)__builtin_ctz((unsigned)nb);
        const uint32_t qw = (uint32_t)base + (uint32_t)(tid >> 6) * kSpan;
        // every load of the item first: a wait for a load also waits for all
        // earlier stores. Blocks past the page read zeros and their stores
        // are dropped by the range checks. The wavefront's kSpan scale bytes
        // of a tensor come in as one dword per lane (lanes past kSpan / 4
        // fetch the same dwords again) and reach their blocks' lanes by
        // ds_bpermute; the byte-wise fallback reads V scales one by one.
        const uint32_t sdo = qw + 4u * ((uint32_t)lane % (kSpan / 4));
        const uint32_t sdw0 = buf_load_u32_nt(sfs[0], sdo);
        const uint32_t sdw1 = V_BYTES ? 0u : buf_load_u32_nt(sfs[1], sdo);
        uint32_t vsb[kRound];
        u32x2 code[2][kRound];
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            const uint32_t q = qw + u * 64 + lane;
            if (V_BYTES)
                vsb[u] = buf_load_u8_nt(sfs[1], v_scale_index(q, (uint32_t)nb));
            code[0][u] = buf_load_u32x2_nt(src[0], q * 8u);
            code[1][u] = buf_load_u32x2_nt(src[1], q * 8u);
        }
        if (!have_lut) {
            // output magnitude byte for (scale byte = tid, code magnitude k),
            // computed while this item's loads are in flight
            const float sv = e4m3_to_f32((uint32_t)tid & 0x7Fu);
            uint32_t lo4 = 0u, hi4 = 0u;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float prod = e2m1_code_to_mag((uint32_t)k) * sv;
                const uint32_t byte = f32_to_e4m3_satfinite(prod, 0u);
                if (k < 4)
                    lo4 |= byte << (8 * k);
                else
                    hi4 |= byte << (8 * (k - 4));
            }
            lut[tid] = u32x2{lo4, hi4};
            __syncthreads();
            have_lut = true;
        }
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
            for (int u = 0; u < kRound; ++u) {
                const uint32_t q = qw + u * 64 + lane;
                uint32_t s;
                if (kv == 1 && V_BYTES) {
                    s = vsb[u];
                } else {
                    // the block's scale byte, relative to the wavefront's first
                    const uint32_t rel = (INTERLEAVED && kv == 1 ? v_scale_index_pow2(q, nbs) : q) - qw;
                    const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(rel & ~3u),
                                                                              (int)(kv ? sdw1 : sdw0));
                    s = (w >> (8 * (rel & 3))) & 0xFFu;
                }
                const u32x2 l = lut[s];
                const uint32_t smask = (s & 0x80u) ? 0x80808080u : 0u;
                const uint2 lo8 = convert8(code[kv][u].x, l, smask);
                const uint2 hi8 = convert8(code[kv][u].y, l, smask);
                // the FP8 copy is read by a later kernel only
                buf_store_u32x4_nt(u32x4{lo8.x, lo8.y, hi8.x, hi8.y}, dsts[kv], q * 16u);
            }
        }
    }
}

template <bool INTERLEAVED, bool SHARED, bool V_BYTES = false>
void launch2(const MatArgs &a, const int32_t *bt, const int32_t *seq_lens, const int32_t *indptr, int grid,
             hipStream_t st)
{
    hipLaunchKernelGGL((materialize_kernel<INTERLEAVED, SHARED, V_BYTES>), dim3(grid), dim3(kThreads), 0, st, a,
                       bt, seq_lens, indptr);
}

}  // namespace

hipError_t launch_materialize_fp8(const kvfp4_paged_cache_t &c, bool v_interleaved, const int32_t *bt,
                                  bool shared, int64_t bt_row_stride, int64_t bt_kv_stride,
                                  const int32_t *seq_lens, const int32_t *indptr, int32_t batch,
                                  void *out, int64_t num_out_pages, int32_t *table, int32_t maxp,
                                  hipStream_t st)
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
    a.bt_row_stride = bt_row_stride;
    a.bt_kv_stride = bt_kv_stride;
    a.out = (uint8_t *)out;
    a.table = table;
    a.ps = c.page_size;
    a.H = c.num_kv_heads;
    a.D = c.head_dim;
    a.maxp = maxp;
    a.batch = batch;
    // kv_page_indptr[B] lives on the device; num_out_pages - 1 bounds it. At
    // least one workgroup runs, which zeroes page 0 for an empty batch.
    const int bph = c.num_kv_heads * c.page_size * (c.head_dim / 16);
    a.parts = (bph + kRound * kThreads - 1) / (kRound * kThreads);
    const int64_t want = num_out_pages - 1 > 0 ? (num_out_pages - 1) * a.parts : 1;
    const int grid = (int)(want < kMaxGrid ? want : kMaxGrid);
    // interleaved V scales stay inside a wavefront's kSpan bytes only when
    // D / 16 divides 32 (head_dim 64, 128, 256, 512); other head dims read
    // them byte by byte
    const bool v_bytes = v_interleaved && 32 % (c.head_dim / 16) != 0;
    if (v_bytes) {
        if (shared)
            launch2<true, true, true>(a, bt, seq_lens, indptr, grid, st);
        else
            launch2<true, false, true>(a, bt, seq_lens, indptr, grid, st);
    } else if (v_interleaved) {
        if (shared)
            launch2<true, true>(a, bt, seq_lens, indptr, grid, st);
        else
            launch2<true, false>(a, bt, seq_lens, indptr, grid, st);
    } else {
        if (shared)
            launch2<false, true>(a, bt, seq_lens, indptr, grid, st);
        else
            launch2<false, false>(a, bt, seq_lens, indptr, grid, st);
    }
    return hipGetLastError();
}

}  // namespace kvfp4

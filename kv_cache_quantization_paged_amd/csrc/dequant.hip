// dequant.hip - paged NVFP4 gather-dequantize for gfx950
// (FlashInfer page flashinfer.quantization.nvfp4_kv_dequantize_paged).
//
// Work item: up to kBatch * 256 chunks (kBatch per lane) of one logical page j of
// one request b, K and V together (one block-table lookup for both). The
// page's output rows out[b, j*ps + t, h, :] (t < tokens of the page, every
// head) are one contiguous run of n_tok*H*D 16-bit values, so lane l of a
// wavefront always stores the 16 bytes right after lane l-1: each store
// instruction writes 1 KiB of contiguous HBM whatever the cache layout. A
// lane owns 8 consecutive outputs per chunk: 4 code bytes and its block's
// scale byte in, 16 bytes out. NHD vs HND only changes where a chunk's code
// bytes are read (HND pages whose geometry allows it are staged through LDS
// instead, see dequant_hnd_lds_kernel). The grid has one workgroup per
// (request, page, part) of the B * ceil(T/ps) table, so large pages still
// spread over many workgroups;
// workgroups past a request's length exit at once. Active pages are scattered
// through that table when lengths differ, and a persistent loop over it
// leaves some workgroups with several times the work of others; one
// workgroup per item lets the dispatcher keep every CU busy. The lengths, the
// table and the global scales are read-only for the whole launch: as
// __restrict__ kernel parameters their wave-uniform reads are scalar loads.
//
// value = RNE16(fp32(fp32(E4M3(s) * g) * e2m1(c))): the scale and the codes
// are decoded by gfx950's conversion instructions (exact: E4M3 -> fp32, and
// FP4 -> fp32 with a unit scale), then two fp32 multiplies in that order and
// one round-to-nearest-even conversion per value.
//
// append_dequant_kernel and append_dequant_lds_kernel (at the end) run a
// decode step's append and this gather in one launch.
#include "kvfp4_internal.h"
#include "nvfp4_device.h"
#include "quant_block.h"

namespace kvfp4 {

namespace {

constexpr int kThreads = 256;
// chunks in flight per lane and tensor. Smaller work items keep the output
// window that the resident workgroups write at any moment narrower, which
// the write stream rewards (NHD: 8 KiB of each output per item; 4 KiB items
// are too short to cover their own latency); HND pages are read as H
// separate head runs, which longer items keep whole.
constexpr int kBatchNhd = 2;
constexpr int kBatchHnd = 8;
template <bool HND>
constexpr int batch_of() { return HND ? kBatchHnd : kBatchNhd; }
constexpr int64_t kMaxGrid = 1 << 24;  // workgroups per launch (grid size in work-items stays below 2^32)
// Workgroups are dealt to the 8 XCDs in turn. Giving each XCD runs of 4
// consecutive pages (all their parts) instead of spreading a page's parts
// over 4 XCDs measured 4-5% faster on 64 full 4096-token requests with
// shuffled pages (228 vs 238 us) and the same on the decode workload.
// Ordering the items page-major (page j of every request, then page j + 1)
// was 30% slower: the output is written best in request order.
constexpr int kXcdChunk = 4;

struct DequantArgs {
    const uint8_t *data[2];
    const uint8_t *sf[2];
    int64_t stride[2];
    int64_t sf_stride[2];
    int64_t bt_row_stride;
    uint16_t *out[2];
    int32_t ps, H, D, T;
    int32_t pages_per_req;   // ceil(T / ps)
    int32_t parts;           // work items per page: ceil(ps * H * D / 8 / (kBatch * kThreads))
    int32_t num_items;       // B * pages_per_req * parts
    int32_t xcd_chunk;       // items per XCD run (0: workgroup i takes item i)
};

// workgroup -> first item. Workgroups are dealt to the 8 XCDs in turn (XCD
// = blockIdx % 8); with xcd_chunk C, the k-th workgroup of XCD x takes item
// (k / C) * 8C + x * C + k % C, so each XCD works through runs of C
// consecutive items. A bijection on [0, grid) when the grid is a multiple of
// 8C.
__device__ __forceinline__ int first_item(int bid, int chunk)
{
    if (chunk == 0)
        return bid;
    const int x = bid & 7, k = bid >> 3;
    return (k / chunk) * 8 * chunk + x * chunk + k % chunk;
}


template <bool BF16>
__device__ __forceinline__ u32x4 decode_chunk(uint32_t codes, float dec)
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

// the gather dequant's items item0, item0 + step, ... of the launch; a
// request's length counts as seq_lens[b] - len_sub (len_sub 1: its last token
// is written by someone else)
template <bool HND, bool BF16, bool BT64>
__device__ __forceinline__ void dequant_items(const DequantArgs &a, int item0, int step,
                                              const void *__restrict__ block_tables,
                                              const int32_t *__restrict__ seq_lens, const float g[2], int len_sub)
{
    constexpr int kBatch = batch_of<HND>();
    constexpr int kUnit = kBatch * kThreads;   // chunks per work item
    const int cpr = a.D >> 3;                  // chunks per (token, head) row
    const int nb = a.D >> 4;
    const int tid = threadIdx.x;
    // mixed-radix position of chunk (c + 256 k): the row advances by r_step
    // (+1 on a carry from cc), and the row's (t, h) follow
    const int r_step = kThreads / cpr, c_step = kThreads - r_step * cpr;
    const int rt_step = r_step / a.H, rh_step = r_step - rt_step * a.H;
    // HND offset steps for kThreads chunks: base step, extra on a chunk-column
    // carry (next head row of the same token), extra on a head wrap (head 0 of
    // the next token)
    const int hb = a.ps * (a.D >> 1), hbs = a.ps * nb;
    const int k0_c = (rh_step * a.ps + rt_step) * (a.D >> 1) + c_step * 4;
    const int kc_c = hb - cpr * 4;
    const int kw_c = -(a.H * a.ps - 1) * (a.D >> 1);
    const int k0_s = (rh_step * a.ps + rt_step) * nb + c_step / 2;
    const int kc_s = hbs - nb;
    const int kw_s = -(a.H * a.ps - 1) * nb;
    const uint32_t page_bytes = (uint32_t)(a.ps * a.H * (a.D >> 1));
    const uint32_t page_sf_bytes = (uint32_t)(a.ps * a.H * nb);

    // one item per workgroup (the loop only repeats for more than kMaxGrid)
    for (int item = item0; item < a.num_items; item += step) {
        const int pair = item / a.parts;
        const int part = item - pair * a.parts;
        const int b = pair / a.pages_per_req;
        const int j = pair - b * a.pages_per_req;
        const int len = min(seq_lens[b] - len_sub, a.T);
        const int t_first = j * a.ps;
        if (t_first >= len)
            continue;
        const int n_tok = min(a.ps, len - t_first);
        const int n_chunks = n_tok * a.H * cpr;
        const int first = part * kUnit;
        if (first >= n_chunks)
            continue;
        const int64_t page = BT64 ? ((const int64_t *)block_tables)[b * a.bt_row_stride + j]
                                  : (int64_t)((const int32_t *)block_tables)[b * a.bt_row_stride + j];
        const int64_t out_off = ((int64_t)b * a.T + t_first) * a.H * a.D;
        // chunks past the page's valid tokens read zeros or in-page bytes and
        // their stores fall outside the outputs' ranges: no per-chunk branch
        const rsrc_t src[2] = {make_rsrc(a.data[0] + page * a.stride[0], page_bytes),
                               make_rsrc(a.data[1] + page * a.stride[1], page_bytes)};
        const rsrc_t sfs[2] = {make_rsrc(a.sf[0] + page * a.sf_stride[0], page_sf_bytes),
                               make_rsrc(a.sf[1] + page * a.sf_stride[1], page_sf_bytes)};
        const rsrc_t dst[2] = {make_rsrc(a.out[0] + out_off, (uint32_t)n_chunks * 16u),
                               make_rsrc(a.out[1] + out_off, (uint32_t)n_chunks * 16u)};
        // byte offsets of this lane's chunk in a code / scale page (K and V
        // pages share the geometry). NHD pages hold rows in output order, so
        // chunk ci sits at 4 ci / ci / 2. HND rows are (h, t): the offsets
        // follow the chunk's (h, cc) counters by additions only.
        const int ci0 = first + tid;
        const int row0 = ci0 / cpr;
        int cc = ci0 - row0 * cpr, h = row0 - (row0 / a.H) * a.H;
        const int t0 = row0 / a.H;
        uint32_t off_c = (uint32_t)((h * a.ps + t0) * (a.D >> 1) + cc * 4);
        uint32_t off_s = (uint32_t)((h * a.ps + t0) * nb + (cc >> 1));
        // every load of the item is issued before its first store: a wait
        // for a load also waits for all earlier stores
        uint32_t code[2][kBatch], sbyte[2][kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            uint32_t oc, os;
            if (!HND) {
                const uint32_t ci = (uint32_t)(ci0 + u * kThreads);
                oc = ci * 4u;
                os = ci >> 1;
            } else {
                oc = off_c;
                os = off_s;
                // advance (h, cc) by kThreads chunks; cc keeps its parity
                // (cpr and c_step are even), so the scale offset moves by
                // exactly half the chunk-column step
                cc += c_step;
                const int carry = cc >= cpr;
                cc -= carry ? cpr : 0;
                h += rh_step + carry;
                const int wrap = h >= a.H;
                h -= wrap ? a.H : 0;
                off_c += (uint32_t)(k0_c + (carry ? kc_c : 0) + (wrap ? kw_c : 0));
                off_s += (uint32_t)(k0_s + (carry ? kc_s : 0) + (wrap ? kw_s : 0));
            }
#pragma unroll
            for (int kv = 0; kv < 2; ++kv) {
                code[kv][u] = buf_load_u32_nt(src[kv], oc);
                sbyte[kv][u] = buf_load_u8(sfs[kv], os);
            }
        }
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const uint32_t ci = (uint32_t)(ci0 + u * kThreads);
                const float dec = e4m3_byte_to_f32(sbyte[kv][u]) * g[kv];
                buf_store_u32x4_nt(decode_chunk<BF16>(code[kv][u], dec), dst[kv], ci * 16u);
            }
        }
    }
}

template <bool HND, bool BF16, bool BT64>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs a, const void *__restrict__ block_tables,
                                                           const int32_t *__restrict__ seq_lens,
                                                           const float *__restrict__ k_scale,
                                                           const float *__restrict__ v_scale)
{
    const float g[2] = {*k_scale, *v_scale};
    dequant_items<HND, BF16, BT64>(a, first_item((int)blockIdx.x, a.xcd_chunk), (int)gridDim.x, block_tables,
                                   seq_lens, g, 0);
}

// HND pages through LDS. When a token's H * D / 8 chunks divide the item
// (kBatchLds * 256 chunks: then H, D / 8 and the item's tokens ti are powers
// of two) and ti divides the page, an item is tokens [t_a, t_a + ti) of one
// page for every head. The workgroup reads each head's run of ti rows (ti * D / 2
// code bytes, ti * D / 16 scale bytes, contiguous in the page) with 16- and
// 4-byte loads in address order, parks them in LDS, and each lane then takes
// its chunks in output order from there: reads as contiguous as the writes.
// Each head's code block in LDS is padded by kLdsPad bytes so that the four
// 16-lane groups of a wave, which read four heads, start on different banks.
constexpr int kLdsPad = 64;
// chunks per lane and tensor in an LDS-staged item: 1024-chunk items (8
// tokens of 8 heads x 128) measured fastest on the prefill workload, ahead
// of 512, 2048 and 4096
constexpr int kBatchLds = 4;

struct HndLdsShape {
    int32_t ti;                  // tokens per item
    int32_t s_cpt, s_cpr;        // log2 of chunks per token (H * D / 8) and per row (D / 8)
};

// the LDS-staged items item0, item0 + step, ... (len_sub as in dequant_items)
template <bool BF16, bool BT64>
__device__ __forceinline__ void dequant_lds_items(const DequantArgs &a, const HndLdsShape &sh, int item0, int step,
                                                  const void *__restrict__ block_tables,
                                                  const int32_t *__restrict__ seq_lens, const float g[2],
                                                  int len_sub, uint8_t *lds)
{
    const int tid = threadIdx.x;
    const int ti = sh.ti, half_row = a.D >> 1, nb = a.D >> 4;
    const int code_head = ti * half_row + kLdsPad, code_tensor = a.H * code_head;
    const int sf_head = ti * nb, sf_tensor = a.H * sf_head;
    uint8_t *lc = lds, *ls = lds + 2 * code_tensor;
    const int pieces_head = ti * half_row / 16, pieces = a.H * pieces_head;   // 16-byte code pieces
    const int spieces_head = sf_head / 4, spieces = a.H * spieces_head;       // 4-byte scale pieces
    const int cpt_mask = (1 << sh.s_cpt) - 1, cpr_mask = (1 << sh.s_cpr) - 1;
    const uint32_t page_bytes = (uint32_t)(a.ps * a.H * half_row);
    const uint32_t page_sf_bytes = (uint32_t)(a.ps * a.H * nb);

    for (int item = item0; item < a.num_items; item += step) {
        const int pair = item / a.parts;
        const int part = item - pair * a.parts;
        const int b = pair / a.pages_per_req;
        const int j = pair - b * a.pages_per_req;
        const int len = min(seq_lens[b] - len_sub, a.T);
        const int t_a = part * ti;                        // the item's first token in the page
        const int t_first = j * a.ps + t_a;
        if (t_first >= len)
            continue;                                     // workgroup-uniform
        const int n_tok = min(ti, len - t_first);
        const int64_t page = BT64 ? ((const int64_t *)block_tables)[b * a.bt_row_stride + j]
                                  : (int64_t)((const int32_t *)block_tables)[b * a.bt_row_stride + j];
        const rsrc_t src[2] = {make_rsrc(a.data[0] + page * a.stride[0], page_bytes),
                               make_rsrc(a.data[1] + page * a.stride[1], page_bytes)};
        const rsrc_t sfs[2] = {make_rsrc(a.sf[0] + page * a.sf_stride[0], page_sf_bytes),
                               make_rsrc(a.sf[1] + page * a.sf_stride[1], page_sf_bytes)};
        // head runs into LDS (rows past the valid tokens are read too: they
        // lie in the page, and their outputs are never stored)
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            for (int q = tid; q < pieces; q += kThreads) {
                const int h = q / pieces_head, o = q - h * pieces_head;
                const u32x4 v = buf_load_u32x4(src[kv], (uint32_t)((h * a.ps + t_a) * half_row + o * 16));
                *(u32x4 *)(lc + kv * code_tensor + h * code_head + o * 16) = v;
            }
            for (int q = tid; q < spieces; q += kThreads) {
                const int h = q / spieces_head, o = q - h * spieces_head;
                const uint32_t v = buf_load_u32(sfs[kv], (uint32_t)((h * a.ps + t_a) * nb + o * 4));
                *(uint32_t *)(ls + kv * sf_tensor + h * sf_head + o * 4) = v;
            }
        }
        __syncthreads();
        const int64_t out_off = ((int64_t)b * a.T + t_first) * a.H * a.D;
        const uint32_t n_bytes = (uint32_t)n_tok * a.H * (a.D >> 3) * 16u;
        const rsrc_t dst[2] = {make_rsrc(a.out[0] + out_off, n_bytes), make_rsrc(a.out[1] + out_off, n_bytes)};
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
            for (int u = 0; u < kBatchLds; ++u) {
                const int ci = tid + u * kThreads;            // chunk of the item, output order (t, h, cc)
                const int tl = ci >> sh.s_cpt, rem = ci & cpt_mask;
                const int h = rem >> sh.s_cpr, cc = rem & cpr_mask;
                const uint32_t code = *(const uint32_t *)(lc + kv * code_tensor + h * code_head + tl * half_row + cc * 4);
                const uint32_t sbyte = ls[kv * sf_tensor + h * sf_head + tl * nb + (cc >> 1)];
                const float dec = e4m3_byte_to_f32(sbyte) * g[kv];
                buf_store_u32x4_nt(decode_chunk<BF16>(code, dec), dst[kv], (uint32_t)ci * 16u);
            }
        }
        __syncthreads();                                  // LDS is reused by the next item of this workgroup
    }
}

template <bool BF16, bool BT64>
__global__ __launch_bounds__(kThreads) void dequant_hnd_lds_kernel(DequantArgs a, HndLdsShape sh,
                                                                   const void *__restrict__ block_tables,
                                                                   const int32_t *__restrict__ seq_lens,
                                                                   const float *__restrict__ k_scale,
                                                                   const float *__restrict__ v_scale)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const float g[2] = {*k_scale, *v_scale};
    dequant_lds_items<BF16, BT64>(a, sh, (int)blockIdx.x, (int)gridDim.x, block_tables, seq_lens, g, 0, lds);
}

// ------------------------------------------------ append + dequant, fused ----
// One launch for a decode step (the append page's rows, then the dequantize
// page over the same cache): row r of the append is request
// batch_indices[r]'s newest token, at position seq_lens[b] - 1. The first
// `blocks` workgroups quantize the rows exactly as the append kernel does
// (standard recipe), store their codes and scales in the cache and write the
// rows' dequantized values straight into the outputs (the same fp32 steps as
// the gather, from the codes and scale just computed); the other workgroups
// run the gather over every request with its length cut by one. No workgroup
// reads a byte another one writes in the launch, so there is no ordering to
// keep, and the outputs and cache equal those of the two calls in sequence.
struct AppendPart {
    uint8_t *data[2];
    uint8_t *sf[2];
    const uint8_t *in[2];
    float g[2];          // the append's global scales (host arguments)
    int64_t nnz;
    int32_t batch;
    int32_t blocks;      // leading workgroups that take the rows (a multiple of 8)
};

struct RowScaleTables {
    float dec[2][128];
    float inv[2][128];
};

// block c (16 elements) of head h of row r, K and V: quantized as the append
// kernel does it, stored at the row's (page, slot), and its 16 values
// dequantized into out[b, pos, h, 16c ..]
template <bool HND, bool BF16_IN, bool BF16>
__device__ __forceinline__ void append_row_block(const DequantArgs &a, const AppendPart &p, const RowScaleTables &tab,
                                                 const float g_out[2], int64_t r, int b, int pos, int64_t page,
                                                 int h, int c)
{
    const int nb = a.D >> 4;
    const int slot = pos % a.ps;
    const int64_t row = HND ? ((int64_t)h * a.ps + slot) : ((int64_t)slot * a.H + h);
    // the output row exists for positions inside max_seq_len (later ones are
    // cut, as the gather cuts them) and requests inside the batch
    const bool out_ok = (unsigned)pos < (unsigned)a.T && (unsigned)b < (unsigned)p.batch;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
        float x[16];
        load_block<BF16_IN>(p.in[kv] + (((r * a.H + h) * a.D) + c * 16) * 2, x);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
        uint32_t s;
        const uint2 codes = quantize_block<0>(x, amax, p.g[kv], 448.0f, tab.dec[kv], tab.inv[kv], s);
        const u32x2 cv = {codes.x, codes.y};
        __builtin_nontemporal_store(cv, (u32x2 *)(p.data[kv] + page * a.stride[kv] + row * (a.D >> 1) + c * 8));
        p.sf[kv][page * a.sf_stride[kv] + row * nb + c] = (uint8_t)s;
        if (out_ok) {
            const float dec = e4m3_byte_to_f32(s) * g_out[kv];
            u32x4 *o = (u32x4 *)(a.out[kv] + (((int64_t)b * a.T + pos) * a.H + h) * a.D + c * 16);
            o[0] = decode_chunk<BF16>(codes.x, dec);
            o[1] = decode_chunk<BF16>(codes.y, dec);
        }
    }
}

// the leading workgroups' rows (tab: their scale tables, in LDS)
template <bool HND, bool BF16_IN, bool BF16>
__device__ __forceinline__ void append_rows(const DequantArgs &a, const AppendPart &p, const float g[2],
                                            RowScaleTables *tabp, const int32_t *__restrict__ batch_indices,
                                            const int32_t *__restrict__ positions,
                                            const int32_t *__restrict__ kv_indices,
                                            const int32_t *__restrict__ kv_indptr)
{
    RowScaleTables &tab = *tabp;
    const int bid = (int)blockIdx.x;
    const int tid = threadIdx.x;
    {
        // the append's decode factor and its reciprocal per (tensor, scale byte)
        const int kv = tid >> 7, s = tid & 127;
        const float dec = e4m3_byte_to_f32((uint32_t)s) * p.g[kv];
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
        for (int64_t r = (int64_t)bid * rows_per_iter + row_off; r < p.nnz; r += (int64_t)p.blocks * rows_per_iter) {
            const int b = batch_indices[r];
            const int pos = positions[r];
            const int64_t page = kv_indices[kv_indptr[b] + pos / a.ps];
            append_row_block<HND, BF16_IN, BF16>(a, p, tab, g, r, b, pos, page, h, c);
        }
    } else {
        for (int64_t r = bid; r < p.nnz; r += p.blocks) {
            const int b = batch_indices[r];
            const int pos = positions[r];
            const int64_t page = kv_indices[kv_indptr[b] + pos / a.ps];
            for (int hc = tid; hc < bpr; hc += kThreads) {
                const int h = hc / nb, c = hc - (hc / nb) * nb;
                append_row_block<HND, BF16_IN, BF16>(a, p, tab, g, r, b, pos, page, h, c);
            }
        }
    }
}

// 8 waves per SIMD as the NHD gather alone reaches (the rows' scalar
// addressing would otherwise take the SGPR count past it)
template <bool HND, bool BF16, bool BT64, bool BF16_IN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void append_dequant_kernel(DequantArgs a, AppendPart p,
                                                                  const void *__restrict__ block_tables,
                                                                  const int32_t *__restrict__ seq_lens,
                                                                  const float *__restrict__ k_scale,
                                                                  const float *__restrict__ v_scale,
                                                                  const int32_t *__restrict__ batch_indices,
                                                                  const int32_t *__restrict__ positions,
                                                                  const int32_t *__restrict__ kv_indices,
                                                                  const int32_t *__restrict__ kv_indptr)
{
    __shared__ RowScaleTables tab;
    const float g[2] = {*k_scale, *v_scale};
    const int bid = (int)blockIdx.x;
    if (bid >= p.blocks) {
        // p.blocks is a multiple of 8, so each XCD keeps its runs of items
        dequant_items<HND, BF16, BT64>(a, first_item(bid - p.blocks, a.xcd_chunk), (int)gridDim.x - p.blocks,
                                       block_tables, seq_lens, g, 1);
        return;
    }
    append_rows<HND, BF16_IN, BF16>(a, p, g, &tab, batch_indices, positions, kv_indices, kv_indptr);
}

// the same step for HND pools of the LDS-staged gather's geometry (8 waves
// per SIMD, as that gather alone reaches)
template <bool BF16, bool BT64, bool BF16_IN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void append_dequant_lds_kernel(DequantArgs a, HndLdsShape sh, AppendPart p,
                                                                      const void *__restrict__ block_tables,
                                                                      const int32_t *__restrict__ seq_lens,
                                                                      const float *__restrict__ k_scale,
                                                                      const float *__restrict__ v_scale,
                                                                      const int32_t *__restrict__ batch_indices,
                                                                      const int32_t *__restrict__ positions,
                                                                      const int32_t *__restrict__ kv_indices,
                                                                      const int32_t *__restrict__ kv_indptr)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const float g[2] = {*k_scale, *v_scale};
    const int bid = (int)blockIdx.x;
    if (bid >= p.blocks) {
        dequant_lds_items<BF16, BT64>(a, sh, bid - p.blocks, (int)gridDim.x - p.blocks, block_tables, seq_lens, g, 1,
                                      lds);
        return;
    }
    append_rows<true, BF16_IN, BF16>(a, p, g, (RowScaleTables *)lds, batch_indices, positions, kv_indices, kv_indptr);
}

struct DequantPtrs {
    const void *block_tables;
    const int32_t *seq_lens;
    const float *k_scale, *v_scale;
};

template <bool HND, bool BF16>
hipError_t launch3(bool bt64, const DequantArgs &a, const DequantPtrs &p, int grid, hipStream_t st)
{
    if (bt64)
        hipLaunchKernelGGL((dequant_kernel<HND, BF16, true>), dim3(grid), dim3(kThreads), 0, st, a, p.block_tables,
                           p.seq_lens, p.k_scale, p.v_scale);
    else
        hipLaunchKernelGGL((dequant_kernel<HND, BF16, false>), dim3(grid), dim3(kThreads), 0, st, a, p.block_tables,
                           p.seq_lens, p.k_scale, p.v_scale);
    return hipGetLastError();
}

// the gather's arguments (every field but the items of the LDS path) and
// its grid; returns the item count (0: nothing to do, -1: too many)
int64_t setup_gather(const kvfp4_paged_cache_t &c, int64_t bt_row_stride, int32_t batch, void *out_k, void *out_v,
                     int32_t max_seq_len, DequantArgs &a, int &grid)
{
    a.data[0] = (const uint8_t *)c.k_data;
    a.data[1] = (const uint8_t *)c.v_data;
    a.sf[0] = (const uint8_t *)c.k_sf;
    a.sf[1] = (const uint8_t *)c.v_sf;
    a.stride[0] = c.k_page_stride;
    a.stride[1] = c.v_page_stride;
    a.sf_stride[0] = c.k_sf_page_stride;
    a.sf_stride[1] = c.v_sf_page_stride;
    a.bt_row_stride = bt_row_stride;
    a.out[0] = (uint16_t *)out_k;
    a.out[1] = (uint16_t *)out_v;
    a.ps = c.page_size;
    a.H = c.num_kv_heads;
    a.D = c.head_dim;
    a.T = max_seq_len;
    a.pages_per_req = (max_seq_len + c.page_size - 1) / c.page_size;
    const int64_t page_chunks = (int64_t)c.page_size * c.num_kv_heads * (c.head_dim / 8);
    const int64_t unit = (int64_t)(c.layout == KVFP4_HND ? kBatchHnd : kBatchNhd) * kThreads;
    a.parts = (int32_t)((page_chunks + unit - 1) / unit);
    const int64_t items = (int64_t)batch * a.pages_per_req * a.parts;
    if (items == 0)
        return 0;
    if (items > INT32_MAX)
        return -1;
    a.num_items = (int32_t)items;
    a.xcd_chunk = 0;
    grid = (int)(items < kMaxGrid ? items : kMaxGrid);
    if (kXcdChunk > 0 && items < kMaxGrid) {
        const int64_t run = 8 * (int64_t)kXcdChunk * a.parts;
        a.xcd_chunk = kXcdChunk * a.parts;
        grid = (int)((items + run - 1) / run * run);
    }
    return items;
}

// the LDS path's item shape for HND pages: chunks per token a power of two
// dividing the item, the item's tokens dividing the page, at most 64 heads,
// rows of at least 16 code bytes (16-byte aligned head runs)
bool hnd_lds_shape(const kvfp4_paged_cache_t &c, HndLdsShape &sh)
{
    if (c.layout != KVFP4_HND)
        return false;
    const int64_t cpt = (int64_t)c.num_kv_heads * (c.head_dim / 8);
    const int64_t unit_lds = (int64_t)kBatchLds * kThreads;
    if ((cpt & (cpt - 1)) != 0 || cpt > unit_lds || c.page_size % (unit_lds / cpt) != 0 || c.num_kv_heads > 64 ||
        c.head_dim < 32)
        return false;
    sh.ti = (int32_t)(unit_lds / cpt);
    sh.s_cpt = __builtin_ctzll((unsigned long long)cpt);
    sh.s_cpr = __builtin_ctz((unsigned)(c.head_dim / 8));
    return true;
}

}  // namespace

hipError_t launch_dequantize_paged(const kvfp4_paged_cache_t &c, const void *block_tables, bool bt64,
                                   int64_t bt_row_stride, const int32_t *seq_lens, int32_t batch,
                                   const float *k_scale, const float *v_scale, void *out_k, void *out_v,
                                   bool out_bf16, int32_t max_seq_len, hipStream_t st)
{
    DequantArgs a;
    int grid = 0;
    const int64_t items = setup_gather(c, bt_row_stride, batch, out_k, out_v, max_seq_len, a, grid);
    if (items == 0)
        return hipSuccess;
    if (items < 0)
        return hipErrorInvalidValue;
    const DequantPtrs p = {block_tables, seq_lens, k_scale, v_scale};
    HndLdsShape sh;
    if (hnd_lds_shape(c, sh)) {
        a.parts = (int32_t)(c.page_size / sh.ti);
        const int64_t items_lds = (int64_t)batch * a.pages_per_req * a.parts;
        if (items_lds > INT32_MAX)
            return hipErrorInvalidValue;
        a.num_items = (int32_t)items_lds;
        const int grid_lds = (int)(items_lds < kMaxGrid ? items_lds : kMaxGrid);
        const size_t lds = (size_t)2 * c.num_kv_heads * (sh.ti * (c.head_dim / 2) + kLdsPad) +
                           (size_t)2 * c.num_kv_heads * sh.ti * (c.head_dim / 16);
        if (bt64) {
            if (out_bf16)
                hipLaunchKernelGGL((dequant_hnd_lds_kernel<true, true>), dim3(grid_lds), dim3(kThreads), lds, st, a, sh,
                                   block_tables, seq_lens, k_scale, v_scale);
            else
                hipLaunchKernelGGL((dequant_hnd_lds_kernel<false, true>), dim3(grid_lds), dim3(kThreads), lds, st, a, sh,
                                   block_tables, seq_lens, k_scale, v_scale);
        } else {
            if (out_bf16)
                hipLaunchKernelGGL((dequant_hnd_lds_kernel<true, false>), dim3(grid_lds), dim3(kThreads), lds, st, a, sh,
                                   block_tables, seq_lens, k_scale, v_scale);
            else
                hipLaunchKernelGGL((dequant_hnd_lds_kernel<false, false>), dim3(grid_lds), dim3(kThreads), lds, st, a,
                                   sh, block_tables, seq_lens, k_scale, v_scale);
        }
        return hipGetLastError();
    }
    const bool hnd = c.layout == KVFP4_HND;
    if (hnd)
        return out_bf16 ? launch3<true, true>(bt64, a, p, grid, st) : launch3<true, false>(bt64, a, p, grid, st);
    return out_bf16 ? launch3<false, true>(bt64, a, p, grid, st) : launch3<false, false>(bt64, a, p, grid, st);
}

namespace {

template <bool HND, bool BF16, bool BT64>
hipError_t launch_fused3(bool in_bf16, const DequantArgs &a, const AppendPart &ap, const DequantPtrs &p,
                         const int32_t *batch_indices, const int32_t *positions, const int32_t *kv_indices,
                         const int32_t *kv_indptr, int grid, hipStream_t st)
{
    if (in_bf16)
        hipLaunchKernelGGL((append_dequant_kernel<HND, BF16, BT64, true>), dim3(grid), dim3(kThreads), 0, st, a, ap,
                           p.block_tables, p.seq_lens, p.k_scale, p.v_scale, batch_indices, positions, kv_indices,
                           kv_indptr);
    else
        hipLaunchKernelGGL((append_dequant_kernel<HND, BF16, BT64, false>), dim3(grid), dim3(kThreads), 0, st, a, ap,
                           p.block_tables, p.seq_lens, p.k_scale, p.v_scale, batch_indices, positions, kv_indices,
                           kv_indptr);
    return hipGetLastError();
}

template <bool HND, bool BF16>
hipError_t launch_fused2(bool bt64, bool in_bf16, const DequantArgs &a, const AppendPart &ap, const DequantPtrs &p,
                         const int32_t *batch_indices, const int32_t *positions, const int32_t *kv_indices,
                         const int32_t *kv_indptr, int grid, hipStream_t st)
{
    return bt64 ? launch_fused3<HND, BF16, true>(in_bf16, a, ap, p, batch_indices, positions, kv_indices, kv_indptr,
                                                 grid, st)
                : launch_fused3<HND, BF16, false>(in_bf16, a, ap, p, batch_indices, positions, kv_indices, kv_indptr,
                                                  grid, st);
}

constexpr int kMaxAppendWorkgroups = 1024;

}  // namespace

hipError_t launch_append_dequantize_paged(const kvfp4_paged_cache_t &c, const void *key, const void *value,
                                          bool in_bf16, int64_t nnz, const int32_t *batch_indices,
                                          const int32_t *positions, const int32_t *kv_indices,
                                          const int32_t *kv_indptr, float k_g, float v_g,
                                          const kvfp4_recipe_t *recipe, const void *block_tables, bool bt64,
                                          int64_t bt_row_stride, const int32_t *seq_lens, int32_t batch,
                                          const float *k_scale, const float *v_scale, void *out_k, void *out_v,
                                          bool out_bf16, int32_t max_seq_len, hipStream_t st)
{
    // one launch for the standard recipe; the 4over6 recipes run the two
    // calls in sequence
    HndLdsShape sh;
    DequantArgs a;
    int grid = 0;
    const int64_t items = setup_gather(c, bt_row_stride, batch, out_k, out_v, max_seq_len, a, grid);
    if (recipe != nullptr || nnz == 0 || items <= 0) {
        hipError_t e = launch_quantize_append(c, key, value, in_bf16, nnz, batch_indices, positions, kv_indices,
                                              kv_indptr, k_g, v_g, recipe, st);
        if (e != hipSuccess)
            return e;
        return launch_dequantize_paged(c, block_tables, bt64, bt_row_stride, seq_lens, batch, k_scale, v_scale, out_k,
                                       out_v, out_bf16, max_seq_len, st);
    }
    AppendPart ap;
    ap.data[0] = (uint8_t *)c.k_data;
    ap.data[1] = (uint8_t *)c.v_data;
    ap.sf[0] = (uint8_t *)c.k_sf;
    ap.sf[1] = (uint8_t *)c.v_sf;
    ap.in[0] = (const uint8_t *)key;
    ap.in[1] = (const uint8_t *)value;
    ap.g[0] = k_g;
    ap.g[1] = v_g;
    ap.nnz = nnz;
    ap.batch = batch;
    const int64_t bpr = (int64_t)c.num_kv_heads * (c.head_dim / 16);
    const int64_t rows_per_wg = bpr <= kThreads ? kThreads / bpr : 1;
    int64_t wgs = (nnz + rows_per_wg - 1) / rows_per_wg;
    wgs = wgs < kMaxAppendWorkgroups ? wgs : kMaxAppendWorkgroups;
    ap.blocks = (int32_t)((wgs + 7) / 8 * 8);
    if ((int64_t)grid + ap.blocks > INT32_MAX / kThreads)
        return hipErrorInvalidValue;
    const DequantPtrs p = {block_tables, seq_lens, k_scale, v_scale};
    if (hnd_lds_shape(c, sh)) {
        a.parts = (int32_t)(c.page_size / sh.ti);
        const int64_t items_lds = (int64_t)batch * a.pages_per_req * a.parts;
        if (items_lds > INT32_MAX)
            return hipErrorInvalidValue;
        a.num_items = (int32_t)items_lds;
        const int64_t grid_lds = items_lds < kMaxGrid ? items_lds : kMaxGrid;
        if (grid_lds + ap.blocks > INT32_MAX / kThreads)
            return hipErrorInvalidValue;
        size_t lds = (size_t)2 * c.num_kv_heads * (sh.ti * (c.head_dim / 2) + kLdsPad) +
                     (size_t)2 * c.num_kv_heads * sh.ti * (c.head_dim / 16);
        lds = lds > sizeof(RowScaleTables) ? lds : sizeof(RowScaleTables);   // the rows' workgroups keep their tables there
        const int total_lds = (int)grid_lds + ap.blocks;
#define KVFP4_FUSED_LDS(BF, B64, BIN)                                                                                \
    hipLaunchKernelGGL((append_dequant_lds_kernel<BF, B64, BIN>), dim3(total_lds), dim3(kThreads), lds, st, a, sh, ap, \
                       p.block_tables, p.seq_lens, p.k_scale, p.v_scale, batch_indices, positions, kv_indices,         \
                       kv_indptr)
        if (out_bf16) {
            if (bt64) {
                if (in_bf16) KVFP4_FUSED_LDS(true, true, true); else KVFP4_FUSED_LDS(true, true, false);
            } else {
                if (in_bf16) KVFP4_FUSED_LDS(true, false, true); else KVFP4_FUSED_LDS(true, false, false);
            }
        } else {
            if (bt64) {
                if (in_bf16) KVFP4_FUSED_LDS(false, true, true); else KVFP4_FUSED_LDS(false, true, false);
            } else {
                if (in_bf16) KVFP4_FUSED_LDS(false, false, true); else KVFP4_FUSED_LDS(false, false, false);
            }
        }
#undef KVFP4_FUSED_LDS
        return hipGetLastError();
    }
    const int total = grid + ap.blocks;
    if (c.layout == KVFP4_HND)
        return out_bf16 ? launch_fused2<true, true>(bt64, in_bf16, a, ap, p, batch_indices, positions, kv_indices,
                                                    kv_indptr, total, st)
                        : launch_fused2<true, false>(bt64, in_bf16, a, ap, p, batch_indices, positions, kv_indices,
                                                     kv_indptr, total, st);
    return out_bf16 ? launch_fused2<false, true>(bt64, in_bf16, a, ap, p, batch_indices, positions, kv_indices,
                                                 kv_indptr, total, st)
                    : launch_fused2<false, false>(bt64, in_bf16, a, ap, p, batch_indices, positions, kv_indices,
                                                  kv_indptr, total, st);
}

}  // namespace kvfp4

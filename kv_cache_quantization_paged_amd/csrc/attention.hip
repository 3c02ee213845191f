// attention.hip - decode attention straight from the paged NVFP4 cache, for
// gfx950. The cache is the one that the flashinfer.page append page fills;
// the flashinfer.quantization dequantize page names FlashInfer's NVFP4
// attention kernels as the consumers of its global decode scales. K and V
// are e2m1 * block_scale * global_scale.
//
// out[b, hq, :] = softmax_t(sm_scale * q[b, hq] . K[b, t]) V[b, t] over
// t < seq_lens[b], with kv head h = hq / G (G = Hq / H query heads per kv
// head), head_dim 64, 128 or 256.
//
// Split over the sequence: a work item is (request, kv head, split of
// kSplitTokens tokens), handled by one workgroup of kWaves wavefronts. The
// workgroups are persistent (as many as stay resident); each builds the list
// of live items from seq_lens and takes its share, XCD by XCD (see the split
// kernel). Each wave takes kWaveTiles tiles of 32 tokens of an item with all
// their loads in flight (the page id of a 16-token half tile is one
// wave-uniform scalar load when the page size is a multiple of 16, and every
// lane address is then a scalar base plus a per-lane constant), and keeps an
// online softmax for the G (<= 16) query heads of its kv head. The waves
// merge in LDS and write (max, sum, unnormalised output) to the caller's
// workspace; a second kernel merges the splits of each (request, kv head).
// On NHD pools (a token's heads interleaved, so one head's row is 64 bytes
// every H rows) the waves instead fetch whole row pieces with 16-byte loads in
// lane order and permute them into operand order through a per-wave LDS
// buffer; a tile then holds 18 registers instead of 26, which leaves room to
// issue the next item's first tile before the merge.
//
// Both products run on v_mfma_f32_16x16x32_f16 (A 16x32, B 32x16; lane l
// holds A[l%16][8(l/16)..+8], B[8(l/16)..+8][l%16], D[4(l/16)..+4][l%16]);
// the counts below are head_dim 128's (Shape<D> scales them for 64 and 256):
//  * scores, S^T[token][g] = K[token][d] . Q^T[d][g]: 16 tokens per MFMA
//    row block, the 128 channels in 4 MFMAs of 32. Lane group q = l/16
//    takes channels 32q..32q+31 (one 16-byte code load per lane and token;
//    its two scale bytes come from a 2-byte load, or from the aligned dword
//    that holds them when the pool's scale rows are 4-byte aligned), and Q^T
//    follows the same channel map.
//  * output, O^T[d][g] += V^T[d][token] . P^T[token][g]: the 32 tokens of a
//    tile in one MFMA, 8 MFMAs for the 128 channels, MFMA j covering
//    channels 8m + j. The lane that holds P for tokens {4q + i, 16 + 4q + i}
//    (its own scores) loads V code chunk l%16 of those 8 tokens.
// Decoding runs in packed fp16: an E2M1 code times its E4M3 block scale has
// at most 6 significant bits and lies in [2^-10, 2688], so code (converted
// exactly) times scale (converted exactly) is exact in one v_pk_mul_f16.
// V pairs two tokens per 32-bit word: a nibble interleave of the two
// tokens' code words puts each channel's two codes in one byte, so one
// conversion and one multiply by the two tokens' scales give the transposed
// operand. A bf16 query row is moved into fp16 exactly, after scaling the
// row by a power of two 2^k that puts its largest magnitude in [2^14, 2^15)
// (components more than 2^38 below it round on fp16's subnormal grid); the
// score factor carries 2^-k. The global scales are applied to the scores
// (K) and to the output (V) in fp32; the probabilities are rounded to fp16
// (11 significant bits) for the second MFMA.
#include <mutex>

#include "kvfp4_internal.h"
#include "nvfp4_device.h"

namespace kvfp4 {

namespace {

constexpr int kD = 128;                     // head_dim of the LDS-staged loader
constexpr int kTile = 32;                   // tokens per MFMA tile
constexpr int kWaves = 4;                   // wavefronts per workgroup
constexpr int kWaveTiles = 2;               // tiles per wave
constexpr int kSplitTokens = kTile * kWaveTiles * kWaves;
constexpr int kMaxPagesPerSplit = kSplitTokens + 1;
constexpr float kSlack = 8.0f;              // log2 headroom of the softmax reference
constexpr int kMaxBatchPerLaunch = 2048;    // requests whose split counts one workgroup keeps in LDS
constexpr int kMaxG = 16;                   // query heads per pass: the MFMA's 16 columns

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
    const uint8_t *data[2];
    const uint8_t *sf[2];
    int64_t stride[2];
    int64_t sf_stride[2];
    const uint16_t *q;
    uint16_t *out;
    float *ws;                // [B][H][splits] partials: m[G], l[G], o[G][head_dim]
    int64_t bt_row_stride;
    int32_t ps, H, G, Hq;     // G: query heads of each kv head in this pass (<= 16)
    int32_t Gtot, gq0;        // query heads per kv head; the pass's first one
    int32_t tok_rows;         // rows between consecutive tokens of a page (HND 1, NHD H)
    int32_t head_rows;        // rows between consecutive kv heads of a page (HND ps, NHD 1)
    int32_t splits;           // per (request, kv head)
    int32_t max_len;          // bt_cols * page_size (capped at INT32_MAX): longer lengths are cut to it
    int32_t batch;            // requests of this launch (bt, seq_lens, q and ws start at its first)
    float sm_scale_log2;      // sm_scale * log2(e)
};

// a request's length as the kernels use it: negative lengths count as 0 and
// lengths past the table row are cut to it, so every access stays inside the
// caller's buffers whatever the lengths hold
__device__ __forceinline__ int clamp_len(int len, int max_len) { return max(0, min(len, max_len)); }

// floats per partial result of a split: max and sum per query head, then the
// unnormalised output rows [G][D]
__host__ __device__ constexpr int partial_floats(int G, int D) { return 2 * G + G * D; }

// The lane maps for head_dim D (64, 128 or 256). Scores: lane group qg of a
// 16-token MFMA block takes channels (D / 4) qg .. + D / 4 of its token, D / 32
// code dwords, one MFMA each (dword kappa holds channels (D / 4) qg + 8 kappa
// .. + 8), with D / 64 block-scale bytes. Output: D / 16 MFMAs, MFMA j covering
// channels (D / 16) m + j, so lane n holds channels (D / 16) n .. + D / 16 of
// its 8 tokens: D / 32 code bytes and one scale byte per token.
template <int D>
struct Shape {
    static_assert(D == 64 || D == 128 || D == 256, "head_dim 64, 128 or 256");
    static constexpr int kKDw = D / 32;          // K code dwords per lane and token = score MFMAs per block
    static constexpr int kVBytes = D / 32;       // V code bytes per lane and token
    static constexpr int kVDw = (D / 32 + 3) / 4;  // ... in dwords
    static constexpr int kVMfma = D / 16;        // output MFMAs
};

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 as_f16x8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3)
{
    const u32x4 w = {w0, w1, w2, w3};
    return __builtin_bit_cast(f16x8, w);
}

// two E2M1 codes (byte SEL of w, low nibble first) -> fp16x2, exact
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_f16(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
}

// two E4M3 bytes (bytes 0 and 1 of w) -> fp16x2, exact
__device__ __forceinline__ uint32_t fp8x2_f16(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}

// packed fp16 product (exact for the operands used here)
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b)
{
    const f16x2 r = __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 codes of one dword times the block scale (s, s) -> 8 fp16 values
__device__ __forceinline__ f16x8 decode8(uint32_t codes, uint32_t ss)
{
    return as_f16x8(mul_f16x2(fp4x2_f16<0>(codes), ss), mul_f16x2(fp4x2_f16<1>(codes), ss),
                    mul_f16x2(fp4x2_f16<2>(codes), ss), mul_f16x2(fp4x2_f16<3>(codes), ss));
}

// reductions over the 4 lanes l, l^16, l^32, l^48 (lane swaps, no LDS)
__device__ __forceinline__ float max4(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum4(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ uint32_t max4_u32(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(r[0], r[1]);
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(s[0], s[1]);
}

// raw bytes of one 32-token tile for one lane (D = 128: kc 16 bytes, ks 2,
// vc 4 per token)
template <int D>
struct TileLoads {
    uint32_t kc[2][Shape<D>::kKDw];     // K codes: token 16 eta + n, channels (D / 4) q ..
    uint32_t ks[2];                     // their D / 64 scale bytes, low byte first
    uint32_t vc[8][Shape<D>::kVDw];     // V codes: channels (D / 16) n .. of token 16 (i / 4) + 4 q + i % 4
    uint32_t vs[8];                     // its scale byte (block D n / 256)
};

// K codes of one lane and token (D / 8 bytes at p)
template <int D>
__device__ __forceinline__ void load_kc(const uint8_t *p, uint32_t (&kc)[Shape<D>::kKDw])
{
    if constexpr (D == 64) {
        const u32x2 w = *(const u32x2 *)p;
        kc[0] = w.x;
        kc[1] = w.y;
    } else {
#pragma unroll
        for (int i = 0; i < D / 128; ++i) {
            const u32x4 w = *(const u32x4 *)(p + 16 * i);
            kc[4 * i] = w.x;
            kc[4 * i + 1] = w.y;
            kc[4 * i + 2] = w.z;
            kc[4 * i + 3] = w.w;
        }
    }
}

// K scale bytes of one lane and token (D / 64 bytes at p)
template <int D>
__device__ __forceinline__ uint32_t load_ks(const uint8_t *p)
{
    if constexpr (D == 64)
        return *p;
    else if constexpr (D == 128)
        return *(const uint16_t *)p;
    else
        return *(const uint32_t *)p;
}

// V codes of one lane and token (D / 32 bytes at p)
template <int D>
__device__ __forceinline__ void load_vc(const uint8_t *p, uint32_t (&vc)[Shape<D>::kVDw])
{
    if constexpr (D == 64) {
        vc[0] = *(const uint16_t *)p;
    } else if constexpr (D == 128) {
        vc[0] = *(const uint32_t *)p;
    } else {
        const u32x2 w = *(const u32x2 *)p;
        vc[0] = w.x;
        vc[1] = w.y;
    }
}

// per-lane byte offsets inside a page for the fast loader
struct LaneOffsets {
    uint32_t k, ks, v, vs;
};

// one tile as the staged loader fetches it: K and V in row pieces (token
// 16 eta + l / 4, bytes 16 (l % 4) .. + 16), their scales one dword per lane
// (token l / 2, bytes 4 (l % 2) .. + 4)
struct RawTile {
    u32x4 kw[2];
    uint32_t ksw;
    u32x4 vw[2];
    uint32_t vsw;
};

// a wave's LDS buffer: V rows [32 tokens][80 bytes], V scales [8 blocks][32
// tokens], then K rows [32][80] and K scales [32][8]. The 80-byte pitch puts
// the operand-order reads on 64 distinct banks.
constexpr int kVPitch = 80;
constexpr int kKOff = 32 * kVPitch + 32 * (kD / 16);
constexpr int kVtBytes = 2 * kKOff;

__device__ __forceinline__ void load_tile_staged(const AttnArgs &a, const int64_t page[2], const int row0[2],
                                               const LaneOffsets &o, int l, RawTile &r)
{
    const uint8_t *vs_half[2], *ks_half[2];
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
        const uint8_t *kd = a.data[0] + page[eta] * a.stride[0] + (int64_t)row0[eta] * (kD / 2);
        ks_half[eta] = a.sf[0] + page[eta] * a.sf_stride[0] + (int64_t)row0[eta] * (kD / 16);
        const uint8_t *vd = a.data[1] + page[eta] * a.stride[1] + (int64_t)row0[eta] * (kD / 2);
        vs_half[eta] = a.sf[1] + page[eta] * a.sf_stride[1] + (int64_t)row0[eta] * (kD / 16);
        r.kw[eta] = *(const u32x4 *)(kd + o.v);
        r.vw[eta] = *(const u32x4 *)(vd + o.v);
    }
    r.ksw = *(const uint32_t *)((l < 32 ? ks_half[0] : ks_half[1]) + o.vs);
    r.vsw = *(const uint32_t *)((l < 32 ? vs_half[0] : vs_half[1]) + o.vs);
}

// a staged tile into this wave's LDS buffer, from which K (per lane: token
// 16 eta + n, channels 32 qg ..) and V (chunk n of the tokens
// 16 (i / 4) + 4 qg + i % 4) are read back in MFMA operand order. One wave's
// LDS operations complete in issue order, so only the compiler has to be
// kept from moving them across each other.
__device__ __forceinline__ void stage_tile(const RawTile &r, uint8_t *vt, int l)
{
    asm volatile("" ::: "memory");
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
        *(u32x4 *)(vt + (16 * eta + (l >> 2)) * kVPitch + 16 * (l & 3)) = r.vw[eta];
        *(u32x4 *)(vt + kKOff + (16 * eta + (l >> 2)) * kVPitch + 16 * (l & 3)) = r.kw[eta];
    }
    // V scales block-major ([block][token]), so that two tokens' bytes of a
    // block are one 16-bit read
#pragma unroll
    for (int j = 0; j < 4; ++j)
        vt[32 * kVPitch + (4 * (l & 1) + j) * 32 + (l >> 1)] = (uint8_t)(r.vsw >> (8 * j));
    *(uint32_t *)(vt + kKOff + 32 * kVPitch + 4 * l) = r.ksw;
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void read_v(const uint8_t *vt, int n, int qg, uint32_t (&vc)[8][1], uint32_t vsp[4])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int T = 16 * (i >> 2) + 4 * qg + (i & 3);
        vc[i][0] = *(const uint32_t *)(vt + T * kVPitch + 4 * n);
    }
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2)
        vsp[i2] = *(const uint16_t *)(vt + 32 * kVPitch + (n >> 1) * 32 + 16 * (i2 >> 1) + 4 * qg + 2 * (i2 & 1));
    asm volatile("" ::: "memory");
}


// page size a multiple of 16: each 16-token half of a tile lies in one page,
// so a half is a scalar base (page, first slot) plus per-lane constants.
// With DW (scale rows 4-byte aligned) the scale bytes come in as the
// aligned dwords that hold them and are picked out where they are used: a
// 1- or 2-byte load is zero-extended by the compiler right after it is
// issued, which makes the wave wait for every load in flight, including the
// second tile's (dwords: 3-4% faster on HND pools at head_dim 128).
template <int D, bool DW = false>
__device__ __forceinline__ void load_half_fast(const AttnArgs &a, int64_t page, int row0, const LaneOffsets &o,
                                               int eta, TileLoads<D> &r)
{
    const uint8_t *kd = a.data[0] + page * a.stride[0] + (int64_t)row0 * (D / 2);
    const uint8_t *ksf = a.sf[0] + page * a.sf_stride[0] + (int64_t)row0 * (D / 16);
    const uint8_t *vd = a.data[1] + page * a.stride[1] + (int64_t)row0 * (D / 2);
    const uint8_t *vsf = a.sf[1] + page * a.sf_stride[1] + (int64_t)row0 * (D / 16);
    load_kc<D>(kd + o.k, r.kc[eta]);
    if constexpr (DW)
        r.ks[eta] = *(const uint32_t *)(ksf + (o.ks & ~3u));
    else
        r.ks[eta] = load_ks<D>(ksf + o.ks);
    const int64_t tc = (int64_t)a.tok_rows * (D / 2), ts = (int64_t)a.tok_rows * (D / 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        load_vc<D>(vd + i * tc + o.v, r.vc[4 * eta + i]);
        if constexpr (DW)
            r.vs[4 * eta + i] = *(const uint32_t *)(vsf + i * ts + (o.vs & ~3u));
        else
            r.vs[4 * eta + i] = vsf[i * ts + o.vs];
    }
}

// any page size: per-token page ids from the split's LDS copy; a token past
// the end reads the split's first token (always valid) and is masked later
template <int D>
__device__ __forceinline__ void load_tile_any(const AttnArgs &a, const int *pages, int h, int t0, int t_base,
                                              int len, int n, int qg, TileLoads<D> &r)
{
    auto addr = [&](int t, int &row) -> int64_t {
        t = t < len ? t : t_base;
        const int pi = (t / a.ps) - (t_base / a.ps);
        const int slot = t - (t / a.ps) * a.ps;
        row = slot * a.tok_rows + h * a.head_rows;
        return pages[pi];
    };
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
        int row;
        const int64_t page = addr(t0 + 16 * eta + n, row);
        load_kc<D>(a.data[0] + page * a.stride[0] + (int64_t)row * (D / 2) + (D / 8) * qg, r.kc[eta]);
        r.ks[eta] = load_ks<D>(a.sf[0] + page * a.sf_stride[0] + (int64_t)row * (D / 16) + (D / 64) * qg);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int row;
        const int64_t page = addr(t0 + 16 * (i >> 2) + 4 * qg + (i & 3), row);
        load_vc<D>(a.data[1] + page * a.stride[1] + (int64_t)row * (D / 2) + (D / 32) * n, r.vc[i]);
        r.vs[i] = a.sf[1][page * a.sf_stride[1] + (int64_t)row * (D / 16) + (D * n) / 256];
    }
}

// MFMA J of the value product and those after it: channels (D / 16) m + J
// come from code byte J / 2 of each token (even channel in the low nibble)
template <int D, int J>
__device__ __forceinline__ void pv_mfma(const uint32_t (&ev)[4][Shape<D>::kVDw],
                                        const uint32_t (&od)[4][Shape<D>::kVDw], const uint32_t (&ss)[4], f16x8 pv,
                                        f32x4 *o)
{
    constexpr int byte = J >> 1, dw = byte >> 2, sel = byte & 3;
    const uint32_t(&src)[4][Shape<D>::kVDw] = (J & 1) ? od : ev;
    o[J] = mfma(as_f16x8(mul_f16x2(fp4x2_f16<sel>(src[0][dw]), ss[0]), mul_f16x2(fp4x2_f16<sel>(src[1][dw]), ss[1]),
                         mul_f16x2(fp4x2_f16<sel>(src[2][dw]), ss[2]), mul_f16x2(fp4x2_f16<sel>(src[3][dw]), ss[3])),
                pv, o[J]);
    if constexpr (J + 1 < Shape<D>::kVMfma)
        pv_mfma<D, J + 1>(ev, od, ss, pv, o);
}

// one 32-token tile: scores, online softmax update, value product
template <int D, bool first, class VFetch>
__device__ __forceinline__ void attend_tile(TileLoads<D> cur, VFetch fetch_v, const f16x8 *qv, int t0, int len, int qg,
                                            float c, float &m_run, float &l_run, f32x4 *o, int ks_shift = 0)
{
    const bool partial = t0 + kTile > len;           // wave-uniform

    // ---- scores: S^T[16 eta + 4 qg + i][n]
    float s[8];
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kap = 0; kap < Shape<D>::kKDw; ++kap) {
            // two code dwords per 16-channel block: scale byte kap / 2,
            // doubled into (s, s)
            const int blk = kap >> 1;
            const uint32_t sc = fp8x2_f16((cur.ks[eta] >> ks_shift) >> (16 * (blk >> 1)));
            const uint32_t sp = (blk & 1) ? __builtin_amdgcn_perm(sc, sc, 0x03020302u)
                                          : __builtin_amdgcn_perm(sc, sc, 0x01000100u);
            acc = mfma(decode8(cur.kc[eta][kap], sp), qv[kap], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * eta + i] = acc[i] * c;
    }
    if (partial) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            s[i] = t0 + 16 * (i >> 2) + 4 * qg + (i & 3) < len ? s[i] : -INFINITY;
    }

    // ---- online softmax for head n (the 4 lanes n, n+16, n+32, n+48). The
    // reference m_run moves only when a score exceeds it by more than
    // kSlack, so p <= 2^kSlack (fine for fp16) and (o, l) are rarely
    // rescaled; any reference gives the same o / l.
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = max4(tmax);                                      // finite: the tile holds a valid token
    const float m_new = tmax > m_run + kSlack ? tmax : m_run;   // always taken on the first tile
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 1 if kept, 0 on the first tile
    float p[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
        psum += p[i];
    }
    l_run = l_run * alpha + sum4(psum);
    m_run = m_new;
    if (!first && __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {   // o is still zero on the first tile
#pragma unroll
        for (int j = 0; j < Shape<D>::kVMfma; ++j) o[j] *= alpha;
    }

    // ---- output: O^T[8 m + j][n] += V^T[8 m + j][token] P^T[token][n]
    const f16x8 pv = as_f16x8(pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]), pack_f16x2(p[4], p[5]),
                              pack_f16x2(p[6], p[7]));
    // token pair i2 = (2 i2, 2 i2 + 1): byte b of ev[i2] holds channel 2b of both
    // tokens (low nibble: the first), od[i2] channel 2b + 1; ss[i2] = their scales
    uint32_t vc[8][Shape<D>::kVDw], vsp[4];
    fetch_v(vc, vsp);
    if (partial) {
        // a masked token's V scale becomes 0 so that its (finite) codes add
        // nothing; its score is -inf
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const int T = t0 + 16 * (i2 >> 1) + 4 * qg + 2 * (i2 & 1);
            vsp[i2] = (T < len ? vsp[i2] & 0xFFu : 0u) | (T + 1 < len ? vsp[i2] & 0xFF00u : 0u);
        }
    }
    uint32_t ev[4][Shape<D>::kVDw], od[4][Shape<D>::kVDw], ss[4];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
#pragma unroll
        for (int dw = 0; dw < Shape<D>::kVDw; ++dw) {
            const uint32_t wa = vc[2 * i2][dw], wb = vc[2 * i2 + 1][dw];
            ev[i2][dw] = (wa & 0x0F0F0F0Fu) | ((wb << 4) & 0xF0F0F0F0u);
            od[i2][dw] = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);
        }
        ss[i2] = fp8x2_f16(vsp[i2]);
    }
    // one channel (MFMA) at a time keeps few decoded words live
    pv_mfma<D, 0>(ev, od, ss, pv, o);
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_bits_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_bits_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// one work item: kv head h of request b over tokens [split * kSplitTokens,
// + kSplitTokens) (len > split * kSplitTokens). All waves of the workgroup
// call it together; it ends with the partial result in the workspace.
template <int D, bool BF16, bool FAST16, bool DW = false>
__device__ __forceinline__ void attend_item(const AttnArgs &a, const int32_t *__restrict__ bt,
                                            const float *__restrict__ k_scale, int b, int h, int split, int len,
                                            int *pages, float (*red_m)[16], float (*red_l)[16], float *red_o)
{
    const int tid = threadIdx.x, l = tid & 63, n = l & 15, qg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform by construction

    // the query rows first: their loads need no sequence length
    // Q^T operands: head n of this kv head's group, channels (D / 4) qg + 8 kappa .. +8
    constexpr int kQ = Shape<D>::kKDw;
    u32x4 qraw[kQ];
    {
        const bool live = n < a.G;
        const uint16_t *qrow = a.q + ((int64_t)b * a.Hq + h * a.Gtot + a.gq0 + (live ? n : 0)) * D + (D / 4) * qg;
#pragma unroll
        for (int k = 0; k < kQ; ++k) qraw[k] = *(const u32x4 *)(qrow + 8 * k);
    }

    const int t_split = split * kSplitTokens;
    const int t_w = t_split + w * (kTile * kWaveTiles);   // this wave's first token
    const int32_t *row_bt = bt + b * a.bt_row_stride;

    if (!FAST16) {
        // the split's page ids, once, into LDS (a page may hold tokens of
        // several tiles and halves)
        const int t_end = min(len, t_split + kSplitTokens);
        const int p0 = t_split / a.ps, p1 = (t_end - 1) / a.ps;
        for (int p = p0 + tid; p <= p1; p += 64 * kWaves)
            pages[p - p0] = row_bt[p];
        __syncthreads();
    }

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 o[Shape<D>::kVMfma];
#pragma unroll
    for (int j = 0; j < Shape<D>::kVMfma; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (t_w < len) {
        TileLoads<D> ld[2];
        // fast loader state: the page index and slot of the next half to load
        int pi = 0, slot = 0, pi_w = 0, slot_w = 0;
        LaneOffsets lo;
        if (FAST16) {
            pi_w = t_w / a.ps;
            slot_w = t_w - pi_w * a.ps;
            pi = pi_w;
            slot = slot_w;
            const uint32_t tr = (uint32_t)a.tok_rows;
            lo.k = n * tr * (D / 2) + (D / 8) * qg;
            lo.ks = n * tr * (D / 16) + (D / 64) * qg;
            lo.v = 4 * qg * tr * (D / 2) + (D / 32) * n;
            lo.vs = 4 * qg * tr * (D / 16) + (D * n) / 256;
        }
        // DW: the byte of each V scale dword that is this lane's (into bytes
        // 0 and 1 of the token pair's word) and the half of the K scale
        // dword that holds its two scale bytes
        const uint32_t vb = DW ? lo.vs & 3u : 0u;
        const uint32_t vsel = 0x0C0C0000u | ((vb + 4u) << 8) | vb;
        const int ks_shift = DW ? (int)(8 * (lo.ks & 3u)) : 0;
        // every tile of the wave is issued, also one wholly past the end (its
        // halves then read the wave's first half, and it is not computed):
        // loads issued on one path only make the compiler wait for every
        // load in flight where the paths meet
        auto issue = [&](int k) {
            const int t0 = t_w + kTile * k;
            if (FAST16) {
#pragma unroll
                for (int eta = 0; eta < 2; ++eta) {
                    // a half past the end reads the wave's first half
                    const bool valid = t0 + 16 * eta < len;
                    const int ppi = valid ? pi : pi_w, pslot = valid ? slot : slot_w;
                    load_half_fast<D, DW>(a, row_bt[ppi], pslot * a.tok_rows + h * a.head_rows, lo, eta, ld[k & 1]);
                    slot += 16;
                    if (slot == a.ps) {
                        slot = 0;
                        ++pi;
                    }
                }
            } else {
                load_tile_any<D>(a, pages, h, t0, t_split, len, n, qg, ld[k & 1]);
            }
        };
        issue(0);
        if (kWaveTiles > 1)
            issue(1);

        // the query rows into fp16 while the tiles load
        f16x8 qv[kQ];
        float c = a.sm_scale_log2 * *k_scale;         // scores to log2 units
        if (n >= a.G) {
#pragma unroll
            for (int k = 0; k < kQ; ++k) qraw[k] = u32x4{0u, 0u, 0u, 0u};
        }
        if (BF16) {
            // largest magnitude of the row (bf16 magnitudes order as integers)
            uint32_t mx = 0;
#pragma unroll
            for (int k = 0; k < kQ; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t v = qraw[k][e] & 0x7FFF7FFFu;
                    mx = max(mx, max(v & 0xFFFFu, v >> 16));
                }
            mx = max4_u32(mx);
            const int E = max((int)(mx >> 7), 1);      // biased exponent of the largest |q|
            int ec;
            (void)frexpf(c, &ec);                       // c = f 2^ec, f in [0.5, 1)
            // 2^kk moves the largest |q| into [2^14, 2^15), kept so that
            // c 2^-kk stays a normal fp32 number
            const int kk = min(max(141 - E, ec - 126), ec + 125);
#pragma unroll
            for (int k = 0; k < kQ; ++k) {
                u32x4 o16;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o16[e] = pack_f16x2(ldexpf(bf16_bits_lo(qraw[k][e]), kk), ldexpf(bf16_bits_hi(qraw[k][e]), kk));
                qv[k] = __builtin_bit_cast(f16x8, o16);
            }
            c = ldexpf(c, -kk);
        } else {
#pragma unroll
            for (int k = 0; k < kQ; ++k) qv[k] = __builtin_bit_cast(f16x8, qraw[k]);
        }

#pragma unroll
        for (int k = 0; k < kWaveTiles; ++k) {
            const int t0 = t_w + kTile * k;
            if (t0 < len) {
                const TileLoads<D> &tl = ld[k & 1];
                auto fv = [&](uint32_t (&vc)[8][Shape<D>::kVDw], uint32_t *vsp) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int dw = 0; dw < Shape<D>::kVDw; ++dw) vc[i][dw] = tl.vc[i][dw];
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2)
                        vsp[i2] = DW ? __builtin_amdgcn_perm(tl.vs[2 * i2 + 1], tl.vs[2 * i2], vsel)
                                     : tl.vs[2 * i2] | (tl.vs[2 * i2 + 1] << 8);
                };
                if (k == 0)
                    attend_tile<D, true>(tl, fv, qv, t0, len, qg, c, m_run, l_run, o, ks_shift);
                else
                    attend_tile<D, false>(tl, fv, qv, t0, len, qg, c, m_run, l_run, o, ks_shift);
            }
            if (k + 2 < kWaveTiles)
                issue(k + 2);
        }
    }

    // ---- merge the waves: lane (qg, n) holds O^T[(D / 16) (4 qg + i) + j][n],
    // that is channels (D / 4) qg + (D / 16) i .. + D / 16 of head n
    if (qg == 0) {
        red_m[w][n] = m_run;
        red_l[w][n] = l_run;
    }
    if (n < a.G) {
        float *orow = red_o + (w * a.G + n) * D + (D / 4) * qg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < D / 64; ++jj)
                *(f32x4 *)(orow + (D / 16) * i + 4 * jj) =
                    f32x4{o[4 * jj][i], o[4 * jj + 1][i], o[4 * jj + 2][i], o[4 * jj + 3][i]};
    }
    __syncthreads();
    const int pf = partial_floats(a.G, D);
    float *ws = a.ws + (((int64_t)b * a.H + h) * a.splits + split) * pf;
    for (int idx = tid; idx < a.G * (D / 4); idx += 64 * kWaves) {
        const int g = idx / (D / 4), d0 = (idx - g * (D / 4)) * 4;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) M = fmaxf(M, red_m[v][g]);
        float L = 0.0f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float f = __builtin_amdgcn_exp2f(red_m[v][g] - M);   // 0 for a wave without tokens
            L += red_l[v][g] * f;
            acc += *(const f32x4 *)(red_o + (v * a.G + g) * D + d0) * f;
        }
        if (d0 == 0) {
            ws[g] = M;
            ws[a.G + g] = L;
        }
        *(f32x4 *)(ws + 2 * a.G + g * D + d0) = acc;
    }
    __syncthreads();                                   // LDS is reused by the next item
}

// staged loader, one tile: tile k of wave w in item it = (b, split, h, len)
// into r; false when the wave has no tokens there (and then nothing is
// issued unless `always`). A half past the end reads the wave's first half
// (masked later).
__device__ __forceinline__ bool issue_staged(const AttnArgs &a, const int32_t *__restrict__ bt, int4 it, int w, int k,
                                             const LaneOffsets &lo, int l, RawTile &r, bool always = false)
{
    const int t_w = it.y * kSplitTokens + w * (kTile * kWaveTiles);
    int t0 = t_w + kTile * k;
    const bool has = t0 < it.w;
    if (!has) {
        // with `always` (a wave whose first tile exists), the wave's first
        // tile is read again and not used: loads issued on one path only
        // make the compiler wait for every load in flight where the paths
        // meet
        if (!always)
            return false;
        t0 = t_w;
    }
    const int32_t *row_bt = bt + (int64_t)it.x * a.bt_row_stride;
    int64_t pg[2];
    int rw[2];
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
        const int t = t0 + 16 * eta < it.w ? t0 + 16 * eta : t_w;
        const int pi = t / a.ps;
        pg[eta] = row_bt[pi];
        rw[eta] = (t - pi * a.ps) * a.tok_rows + it.z * a.head_rows;
    }
    load_tile_staged(a, pg, rw, lo, l, r);
    return has;
}

// the query rows of item it into fp16 MFMA operands and the score factor
// the raw query rows of head n of kv head h (zeros for n >= G), issued
// before a wave's second tile so that converting them waits for no tile
__device__ __forceinline__ void query_raw(const AttnArgs &a, int b, int h, int n, int qg, u32x4 qraw[4])
{
    const bool live = n < a.G;
    const uint16_t *qrow = a.q + ((int64_t)b * a.Hq + h * a.Gtot + a.gq0 + (live ? n : 0)) * kD + 32 * qg;
#pragma unroll
    for (int k = 0; k < 4; ++k) qraw[k] = live ? *(const u32x4 *)(qrow + 8 * k) : u32x4{0u, 0u, 0u, 0u};
}

template <bool BF16>
__device__ __forceinline__ float load_query(const AttnArgs &a, const float *__restrict__ k_scale, u32x4 qraw[4],
                                            f16x8 qv[4])
{
    float c = a.sm_scale_log2 * *k_scale;
    if (BF16) {
        uint32_t mx = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t v = qraw[k][e] & 0x7FFF7FFFu;
                mx = max(mx, max(v & 0xFFFFu, v >> 16));
            }
        mx = max4_u32(mx);
        const int E = max((int)(mx >> 7), 1);
        int ec;
        (void)frexpf(c, &ec);
        const int kk = min(max(141 - E, ec - 126), ec + 125);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            u32x4 o16;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o16[e] = pack_f16x2(ldexpf(bf16_bits_lo(qraw[k][e]), kk), ldexpf(bf16_bits_hi(qraw[k][e]), kk));
            qv[k] = __builtin_bit_cast(f16x8, o16);
        }
        c = ldexpf(c, -kk);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) qv[k] = __builtin_bit_cast(f16x8, qraw[k]);
    }
    return c;
}

// one work item on the staged loader. pre holds this wave's first tile of the
// item when have_pre is set; the first tile of the next item (if any) is
// issued into pre before the merge, so that its loads are in flight through
// the merge and the next item's start.
template <bool BF16>
__device__ __forceinline__ void attend_item_staged(const AttnArgs &a, const int32_t *__restrict__ bt,
                                                   const float *__restrict__ k_scale, int4 it, int4 next, bool has_next,
                                                   RawTile &pre, bool &have_pre, float (*red_m)[16],
                                                   float (*red_l)[16], float *red_o, uint8_t *vt_all)
{
    // the thread index through an opaque move, so that the lane-dependent
    // addresses below are recomputed per item rather than held in registers
    // across the item loop
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int l = tid & 63, n = l & 15, qg = l >> 4;
    LaneOffsets lo;
    {
        const uint32_t tr = (uint32_t)a.tok_rows;
        lo.k = 0;
        lo.ks = 0;
        lo.v = (l >> 2) * tr * (kD / 2) + 16 * (l & 3);
        lo.vs = ((l & 31) >> 1) * tr * (kD / 16) + 4 * (l & 1);
    }
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = it.x, split = it.y, h = it.z, len = it.w;
    const int t_w = split * kSplitTokens + w * (kTile * kWaveTiles);
    uint8_t *vt = vt_all + w * kVtBytes;

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    bool have_next = false;
    auto issue_next = [&]() { have_next = has_next && issue_staged(a, bt, next, w, 0, lo, l, pre); };
    auto stage_k = [&](const RawTile &r, TileLoads<kD> &cur) {
        stage_tile(r, vt, l);
#pragma unroll
        for (int eta = 0; eta < 2; ++eta) {
            const u32x4 kw = *(const u32x4 *)(vt + kKOff + (16 * eta + n) * kVPitch + 16 * qg);
            cur.kc[eta][0] = kw.x;
            cur.kc[eta][1] = kw.y;
            cur.kc[eta][2] = kw.z;
            cur.kc[eta][3] = kw.w;
            cur.ks[eta] = *(const uint16_t *)(vt + kKOff + 32 * kVPitch + (16 * eta + n) * (kD / 16) + 2 * qg);
        }
    };
    auto fv = [&](uint32_t (&vc)[8][1], uint32_t *vs) { read_v(vt, n, qg, vc, vs); };

    if (t_w < len) {
        if (!have_pre)
            issue_staged(a, bt, it, w, 0, lo, l, pre);
        u32x4 qraw[4];
        query_raw(a, b, h, n, qg, qraw);
        RawTile r1;
        const bool two = issue_staged(a, bt, it, w, 1, lo, l, r1, true);
        f16x8 qv[4];
        const float c = load_query<BF16>(a, k_scale, qraw, qv);
        {
            TileLoads<kD> cur;
            stage_k(pre, cur);
            if (!two)
                issue_next();
            attend_tile<kD, true>(cur, fv, qv, t_w, len, qg, c, m_run, l_run, o);
        }
        if (two) {
            TileLoads<kD> cur;
            stage_k(r1, cur);
            issue_next();
            attend_tile<kD, false>(cur, fv, qv, t_w + kTile, len, qg, c, m_run, l_run, o);
        }
    } else {
        issue_next();
    }
    have_pre = have_next;

    if (qg == 0) {
        red_m[w][n] = m_run;
        red_l[w][n] = l_run;
    }
    if (n < a.G) {
        float *orow = red_o + (w * a.G + n) * kD + 32 * qg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(f32x4 *)(orow + 8 * i) = f32x4{o[0][i], o[1][i], o[2][i], o[3][i]};
            *(f32x4 *)(orow + 8 * i + 4) = f32x4{o[4][i], o[5][i], o[6][i], o[7][i]};
        }
    }
    __syncthreads();
    const int pf = partial_floats(a.G, kD);
    float *ws = a.ws + (((int64_t)b * a.H + h) * a.splits + split) * pf;
    for (int idx = tid; idx < a.G * (kD / 4); idx += 64 * kWaves) {
        const int g = idx / (kD / 4), d0 = (idx - g * (kD / 4)) * 4;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) M = fmaxf(M, red_m[v][g]);
        float L = 0.0f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float f = __builtin_amdgcn_exp2f(red_m[v][g] - M);
            L += red_l[v][g] * f;
            acc += *(const f32x4 *)(red_o + (v * a.G + g) * kD + d0) * f;
        }
        if (d0 == 0) {
            ws[g] = M;
            ws[a.G + g] = L;
        }
        *(f32x4 *)(ws + 2 * a.G + g * kD + d0) = acc;
    }
    __syncthreads();
}

// block-wide exclusive prefix sum of one int per thread (blockDim 64 * kWaves)
__device__ __forceinline__ int block_exclusive_scan(int v, int *wave_tot, int &total)
{
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (l >= d)
            x += y;
    }
    if (l == 63)
        wave_tot[w] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        before += k < w ? wave_tot[k] : 0;
        total += wave_tot[k];
    }
    __syncthreads();
    return before + x - v;
}

// Persistent workgroups. The live work items are the (request b, split,
// kv head h) with split * kSplitTokens < seq_lens[b]; every workgroup
// builds the same list from seq_lens (whole 256-token splits of all
// requests first, then the shorter tail splits; their counts before each
// request in LDS), so no item is launched dead. Each XCD deals its items in
// rounds of one per workgroup that alternate direction, so the workgroups
// that draw an item in the last, partial round are those that drew tails in
// the round before: 2-3% faster than dealing every round the same way. Item groups (b, split)
// are dealt to the 8 XCDs by index mod 8 (workgroup x runs on XCD x mod 8
// under the round-robin dispatch), and the H heads of a group go to H
// workgroups of that XCD in the same round, so a page's lines shared by
// several heads (NHD rows, scale rows) are fetched into one L2 once.
// Loaders: kAnyPage (per-token page ids from LDS), kDirect (page size a
// multiple of 16, the lanes gather their operands straight from the page)
// and kStaged (the same page sizes, NHD: whole row pieces through LDS, and
// each item's first tile issued before the previous item's merge; measured
// 3.5% faster than kDirect on NHD pools and 8% slower on HND pools, whose
// head runs the direct gathers already read contiguously).
constexpr int kAnyPage = 0, kDirect = 1, kStaged = 2, kDirectDw = 3;
template <int D, bool BF16, int LOADER>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(D == 256 ? 2 : 4))) void attention_split_kernel(AttnArgs a, const int32_t *__restrict__ bt,
                                                                      const int32_t *__restrict__ seq_lens,
                                                                      const float *__restrict__ k_scale)
{
    __shared__ int pages[LOADER == kAnyPage ? kMaxPagesPerSplit : 1];
    __shared__ __attribute__((aligned(16))) uint8_t vt[LOADER == kStaged ? kWaves * kVtBytes : 16];
    __shared__ float red_m[kWaves][16], red_l[kWaves][16];
    __shared__ int wave_tot[kWaves];
    __shared__ int4 items[64 * kWaves];              // (b, split, h, len)
    extern __shared__ float dyn[];                   // red_o [kWaves][G][D], then cum, cut [batch + 1]
    float *red_o = dyn;
    int *cum = (int *)(dyn + kWaves * a.G * D);
    const int tid = threadIdx.x, nthr = 64 * kWaves;

    // ---- cum[b] / cut[b]: whole splits / partial tail splits of the requests before b
    int *cut = cum + a.batch + 1;
    const int per = (a.batch + nthr - 1) / nthr;      // <= kMaxBatchPerLaunch / nthr
    int mf = 0, mt = 0;
    for (int k = 0; k < per; ++k) {
        const int bb = tid * per + k;
        const int len = bb < a.batch ? clamp_len(seq_lens[bb], a.max_len) : 0;
        mf += len / kSplitTokens;
        mt += len % kSplitTokens != 0;
    }
    int tot_f, tot_t;
    int run_f = block_exclusive_scan(mf, wave_tot, tot_f);
    int run_t = block_exclusive_scan(mt, wave_tot, tot_t);
    for (int k = 0; k < per; ++k) {
        const int bb = tid * per + k;
        if (bb < a.batch) {
            const int len = clamp_len(seq_lens[bb], a.max_len);
            cum[bb] = run_f;
            cut[bb] = run_t;
            run_f += len / kSplitTokens;
            run_t += len % kSplitTokens != 0;
        }
    }
    if (tid == 0) {
        cum[a.batch] = tot_f;
        cut[a.batch] = tot_t;
    }
    __syncthreads();
    const int total = tot_f + tot_t;

    // ---- this workgroup's share: groups g = xcd + 8 r (whole splits first,
    // then the tails), items m = r H + h, dealt in rounds of per_xcd that
    // alternate direction: round t gives workgroup j item
    // t per_xcd + (t odd ? per_xcd - 1 - j : j)
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    const int64_t ngx = total > xcd ? (total - xcd + 7) / 8 : 0;
    const int64_t nix = ngx * a.H;
    const int64_t rounds = (nix + per_xcd - 1) / per_xcd;
    for (int64_t base = 0; base < rounds; base += nthr) {
        const int64_t t = base + tid;
        const int64_t m = t * per_xcd + ((t & 1) ? per_xcd - 1 - j : j);
        if (t < rounds && m < nix) {
            const int64_t r = m / a.H;
            const int h = (int)(m - r * a.H);
            const int g = (int)(xcd + 8 * r);
            const int *cc = g < tot_f ? cum : cut;
            const int key = g < tot_f ? g : g - tot_f;
            int lo = 0, hi = a.batch;                 // the request whose splits hold group g
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (cc[mid] <= key)
                    lo = mid;
                else
                    hi = mid;
            }
            const int len = clamp_len(seq_lens[lo], a.max_len);
            items[tid] = int4{lo, g < tot_f ? key - cum[lo] : len / kSplitTokens, h, len};
        }
        __syncthreads();
        // the last round may hold no item of this workgroup
        int count = (int)min((int64_t)nthr, rounds - base);
        if (count > 0) {
            const int64_t tl = base + count - 1;
            if (tl * per_xcd + ((tl & 1) ? per_xcd - 1 - j : j) >= nix)
                --count;
        }
        if constexpr (LOADER == kStaged && D == kD) {
            RawTile pre;                                 // this wave's first tile of the next item
            bool have_pre = false;
            for (int t = 0; t < count; ++t) {
                const int4 nx = items[t + 1 < count ? t + 1 : t];
                attend_item_staged<BF16>(a, bt, k_scale, items[t], nx, t + 1 < count, pre, have_pre, red_m,
                                         red_l, red_o, vt);
            }
        } else {
            for (int t = 0; t < count; ++t) {
                const int4 it = items[t];
                attend_item<D, BF16, LOADER == kDirect || LOADER == kDirectDw, LOADER == kDirectDw>(
                    a, bt, k_scale, it.x, it.z, it.y, it.w, pages, red_m, red_l,
                                                        red_o);
            }
        }
    }
}

// merge the live splits of one (request, kv head); thread -> (head g, 4
// channels). Splits are taken 8 at a time, all their loads in flight, with
// a running (max, sum, output) rescaled per group.
template <int D, bool BF16>
__global__ __launch_bounds__(1024) void attention_merge_kernel(AttnArgs a, const int32_t *__restrict__ seq_lens,
                                                               const float *__restrict__ v_scale)
{
    constexpr int kGroup = 8;
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int g = threadIdx.x / (D / 4), d0 = (threadIdx.x % (D / 4)) * 4;
    const int len = clamp_len(seq_lens[b], a.max_len);
    const int live = (len + kSplitTokens - 1) / kSplitTokens;
    const int pf = partial_floats(a.G, D);
    const float *ws = a.ws + (int64_t)bh * a.splits * pf;
    float M = -INFINITY, L = 0.0f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < live; s0 += kGroup) {
        float ms[kGroup], ls[kGroup];
        f32x4 os[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const float *p = ws + min(s0 + u, live - 1) * pf;   // a repeat of the last split is dropped below
            ms[u] = p[g];
            ls[u] = p[a.G + g];
            os[u] = *(const f32x4 *)(p + 2 * a.G + g * D + d0);
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < kGroup; ++u)
            if (s0 + u < live)
                mx = fmaxf(mx, ms[u]);
        const float f0 = __builtin_amdgcn_exp2f(M - mx);          // 0 on the first group
        L *= f0;
        acc *= f0;
#pragma unroll
        for (int u = 0; u < kGroup; ++u)
            if (s0 + u < live) {
                const float f = __builtin_amdgcn_exp2f(ms[u] - mx);
                L += ls[u] * f;
                acc += os[u] * f;
            }
        M = mx;
    }
    const float scale = L > 0.0f ? *v_scale / L : 0.0f;        // an empty request gives zeros
    const uint32_t w0 = BF16 ? pack_bf16x2(acc[0] * scale, acc[1] * scale) : pack_f16x2(acc[0] * scale, acc[1] * scale);
    const uint32_t w1 = BF16 ? pack_bf16x2(acc[2] * scale, acc[3] * scale) : pack_f16x2(acc[2] * scale, acc[3] * scale);
    *(u32x2 *)(a.out + ((int64_t)b * a.Hq + h * a.Gtot + a.gq0 + g) * D + d0) = u32x2{w0, w1};
}

}  // namespace

// The partial results of kv_decode_attention_noalloc, for callers that cannot
// allocate: a file-scope device array that every GPU the library runs on
// holds until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kMaxScratchDevices];
}  // namespace

hipError_t noalloc_scratch(void **addr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));    // with `dev` current: its own copy
        if (e != hipSuccess)
            return e;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return hipSuccess;
}

int64_t decode_attention_splits(int32_t bt_cols, int32_t page_size)
{
    const int64_t tokens = (int64_t)bt_cols * page_size;
    return tokens > 0 ? (tokens + kSplitTokens - 1) / kSplitTokens : 1;
}

int64_t decode_attention_workspace_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_qo_heads, int32_t bt_cols,
                                         int32_t page_size, int32_t head_dim)
{
    // the query heads of a kv head run in passes of up to 16, one after the
    // other on the stream, each reusing the workspace
    const int G = min(num_qo_heads / num_kv_heads, kMaxG);
    return (int64_t)batch * num_kv_heads * decode_attention_splits(bt_cols, page_size) * partial_floats(G, head_dim) *
           4;
}

namespace {

typedef void (*split_fn)(AttnArgs, const int32_t *, const int32_t *, const float *);
typedef void (*merge_fn)(AttnArgs, const int32_t *, const float *);

// the split kernel for (head_dim, query dtype, loader); the LDS-staged
// loader is built for head_dim 128 only, other sizes read NHD pages directly
template <int D>
split_fn split_kernel_of(bool bf16, int loader)
{
    if (D != kD && loader == kStaged)
        loader = kDirect;
    const split_fn kernels[2][4] = {
        {attention_split_kernel<D, false, kAnyPage>, attention_split_kernel<D, false, kDirect>,
         attention_split_kernel<D, false, D == kD ? kStaged : kDirect>, attention_split_kernel<D, false, kDirectDw>},
        {attention_split_kernel<D, true, kAnyPage>, attention_split_kernel<D, true, kDirect>,
         attention_split_kernel<D, true, D == kD ? kStaged : kDirect>, attention_split_kernel<D, true, kDirectDw>}};
    return kernels[bf16 ? 1 : 0][loader];
}

}  // namespace

hipError_t launch_decode_attention(const kvfp4_paged_cache_t &c, const void *q, bool bf16, int32_t num_qo_heads,
                                   const int32_t *bt, int64_t bt_row_stride, int32_t bt_cols,
                                   const int32_t *seq_lens, int32_t batch, const float *k_scale,
                                   const float *v_scale, float sm_scale, void *out, void *workspace,
                                   hipStream_t st)
{
    AttnArgs a;
    a.data[0] = (const uint8_t *)c.k_data;
    a.data[1] = (const uint8_t *)c.v_data;
    a.sf[0] = (const uint8_t *)c.k_sf;
    a.sf[1] = (const uint8_t *)c.v_sf;
    a.stride[0] = c.k_page_stride;
    a.stride[1] = c.v_page_stride;
    a.sf_stride[0] = c.k_sf_page_stride;
    a.sf_stride[1] = c.v_sf_page_stride;
    a.q = (const uint16_t *)q;
    a.out = (uint16_t *)out;
    a.ws = (float *)workspace;
    a.bt_row_stride = bt_row_stride;
    a.ps = c.page_size;
    a.H = c.num_kv_heads;
    a.Hq = num_qo_heads;
    a.Gtot = num_qo_heads / c.num_kv_heads;
    a.tok_rows = c.layout == KVFP4_HND ? 1 : c.num_kv_heads;
    a.head_rows = c.layout == KVFP4_HND ? c.page_size : 1;
    a.splits = (int32_t)decode_attention_splits(bt_cols, c.page_size);
    // a length past the table row would read other rows' (or no) page ids:
    // such requests are cut to the tokens their row can address
    const int64_t row_tokens = (int64_t)bt_cols * c.page_size;
    a.max_len = (int32_t)(row_tokens < INT32_MAX ? row_tokens : INT32_MAX);
    a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
    const int64_t bh = (int64_t)batch * c.num_kv_heads;
    if (bh == 0)
        return hipSuccess;
    const int D = c.head_dim;
    // pools whose scale rows are 4-byte aligned read their scales as dwords
    const bool sf_dw = ((uintptr_t)c.k_sf | (uintptr_t)c.v_sf | (uint64_t)c.k_sf_page_stride |
                        (uint64_t)c.v_sf_page_stride) % 4 == 0;
    // (NHD pools at head_dim 128 take the LDS-staged loader; at other head
    // dims they read directly, with dword scale loads when aligned)
    const int loader = c.page_size % 16 != 0            ? kAnyPage
                       : c.layout == KVFP4_NHD && D == kD ? kStaged
                       : sf_dw                            ? kDirectDw
                                                          : kDirect;
    const split_fn kernel = D == 64    ? split_kernel_of<64>(bf16, loader)
                            : D == 256 ? split_kernel_of<256>(bf16, loader)
                                       : split_kernel_of<128>(bf16, loader);
    const merge_fn merge = D == 64    ? (bf16 ? attention_merge_kernel<64, true> : attention_merge_kernel<64, false>)
                           : D == 256 ? (bf16 ? attention_merge_kernel<256, true> : attention_merge_kernel<256, false>)
                                      : (bf16 ? attention_merge_kernel<128, true> : attention_merge_kernel<128, false>);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    // query heads beyond the MFMA's 16 columns: passes over blocks of 16
    // query heads (each pass reads K and V again)
    for (int g0 = 0; g0 < a.Gtot; g0 += kMaxG) {
        a.gq0 = g0;
        a.G = a.Gtot - g0 < kMaxG ? a.Gtot - g0 : kMaxG;
        const int64_t pf = partial_floats(a.G, D);
        for (int64_t b0 = 0; b0 < batch; b0 += kMaxBatchPerLaunch) {
            AttnArgs ac = a;
            ac.batch = (int32_t)(batch - b0 < kMaxBatchPerLaunch ? batch - b0 : kMaxBatchPerLaunch);
            ac.q = a.q + b0 * a.Hq * D;
            ac.ws = a.ws + b0 * a.H * a.splits * pf;
            const size_t lds = (size_t)kWaves * a.G * D * sizeof(float) + (size_t)(ac.batch + 1) * 2 * sizeof(int);
            // as many workgroups as stay resident, a multiple of the 8 XCDs,
            // and no more than there can be items
            int occ = 0;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 64 * kWaves, lds);
            if (e != hipSuccess)
                return e;
            const int64_t most = ((int64_t)ac.batch * a.H * a.splits + 7) / 8 * 8;
            int64_t grid = (int64_t)(occ > 0 ? occ : 1) * cus / 8 * 8;
            grid = grid < 8 ? 8 : (grid > most ? most : grid);
            hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64 * kWaves), lds, st, ac, bt + b0 * bt_row_stride,
                               seq_lens + b0, k_scale);
        }
        const dim3 merge_threads((unsigned)(D / 4 * a.G));    // one thread per (query head, 4 channels)
        hipLaunchKernelGGL(merge, dim3((unsigned)bh), merge_threads, 0, st, a, seq_lens, v_scale);
    }
    return hipGetLastError();
}

}  // namespace kvfp4

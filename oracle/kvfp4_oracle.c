/*
 * kvfp4_oracle.c - plain, slow, by-definition CPU oracle for the paged NVFP4
 * KV-cache path.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or helper with the GPU library, and neither side calls the other.
 *
 * What it follows (FlashInfer 0.7.4 documentation pages):
 *   [AP] flashinfer.page.nvfp4_quantize_append_paged_kv_cache - the append
 *        call: shapes [nnz, H, D] in, packed E2M1 (D/2 bytes) and E4M3 block
 *        scales (D/16 bytes) out, CSR page table, global decode scales.
 *   [DQ] flashinfer.quantization.nvfp4_kv_dequantize_paged - the gather:
 *        block_tables / seq_lens, e2m1 * block_scale * global_scale into
 *        [batch, max_seq_len, H, D], tail positions untouched.
 *   [MF] flashinfer.quantization.kernels.nvfp4_kv_materialize.
 *        nvfp4_kv_materialize_fp8 and the NVFP4KVMaterializer.run() entry of
 *        the flashinfer.quantization module page ("NVFP4 KV Cache
 *        Materialization") - E2M1 x E4M3 products as float8_e4m3fn pages.
 *   [R46] flashinfer.quantization module page, "NVFP4 4over6 Recipes" - the
 *        amax/6 block scale, the amax/4 candidate, MSE/MAE scoring in fp32,
 *        e4m3_max = 256.
 *
 * The pages name E2M1 and E4M3 but print no bit layout; the codecs below use
 * the standard OCP FP4 (E2M1) and FP8 (E4M3, "fn": no infinities, one NaN
 * mantissa) encodings, and every encoder is a scan for the nearest
 * representable value with ties going to the even code.
 *
 * Precision: the quantizer decides integer codes from fp32 values and the
 * 4over6 page fixes the error evaluation at exact fp32, so every step of
 * the method is an fp32 operation here; the file is built with
 * -ffp-contract=off so that no multiply-add is fused, and on x86-64 each
 * float operation rounds to fp32. Only the format definitions themselves
 * (code -> value, nearest-value scans) use double, where they are exact.
 *
 * Readings of steps the pages leave open (each stated again where it is used):
 *   R1  block scale: sf = amax / fp32(C * g), one IEEE fp32 division.
 *   R2  element encode: v = x * fp32(1 / fp32(E4M3(s) * g)); 0 when that
 *       decode factor is 0.
 *   R3  E2M1 rounding: nearest, ties to even, saturating at +-6; the sign of
 *       v is kept, so negative values that round to zero give code 0x8.
 *   R4  4over6 clamps: the amax/6 candidate is clamped at the recipe's
 *       e4m3_max, the amax/4 candidate at 448 (the page notes that its 1.5x
 *       larger value 384 stays inside the E4M3 range).
 *   R5  4over6 error: reconstruction versus the input, in fp32, per element
 *       d = x - fp32(dec * e2m1); term d*d (MSE) or |d| (MAE); summed by a
 *       balanced pairwise tree in index order; amax/4 kept only when its
 *       error is strictly smaller.
 *   R6  global scale: g = amax / fp32(6 * e4m3_max); 1 for an all-zero tensor.
 *   R7  dequant value: RNE_half(fp32(fp32(E4M3(s) * g) * e2m1)).
 *   R8  materialize value: RNE of the exact product E2M1 * E4M3 to E4M3,
 *       saturating to +-448 with the sign kept; whole pages are written.
 *   R9  V block scales for materialize, when interleaved: inside a
 *       (page, head) tile, the scale of token t, block column c sits at byte
 *       ((t / 4) * (D / 16) + c) * 4 + t % 4.
 *   R10 contiguous codec [KV]: the linear-layout quantize / dequantize of
 *       the "FP4 KV Cache Quantization" section take the same global decode
 *       scale g and the same block arithmetic (R1-R7) as the paged calls;
 *       blocks of 16 run along the last dimension, scales are linear.
 *   R12 4over6 "err_use_fast_math" [R46]: the page says the error is then
 *       evaluated in fp16 instead of exactly in fp32. Read as: x and the fp32
 *       reconstruction rounded to fp16, then the difference, the square
 *       (MSE) and each pairwise sum rounded to fp16 (RNE, overflow to inf);
 *       the candidates compare as in R5.
 *   R11 whole-pool quantizer [KV] (nvfp4_quantize_paged_kv_cache, which the
 *       page ties to the trtllm-gen MHA kernel): quantizes every slot of every page with
 *       R1-R5, K scales linear, V scales in the R9 interleave, which is the
 *       layout [MF] says this function produces.
 *
 *   R13 decode attention over the NVFP4 cache [DQ: the page names the NVFP4
 *       attention kernels as users of its global decode scales; values
 *       e2m1 * block_scale * global_scale]:
 *       scaled dot-product attention of one query token per request over
 *       the exact dequantized K and V (no 16-bit rounding, as a fused
 *       consumer has none), grouped-query heads hq -> hq / (Hq / H); an
 *       empty request gives zeros.
 *
 * [KV] flashinfer.quantization module page, "FP4 KV Cache Quantization"
 *      (nvfp4_kv_quantize, nvfp4_kv_dequantize, nvfp4_quantize_paged_kv_cache).
 */
#include "kvfp4_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* E2M1 (OCP FP4): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa. */
/* Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity, no NaN.              */
/* ======================================================================== */
static double e2m1_magnitude(int k)
{
    int e = (k >> 1) & 3, m = k & 1;
    if (e == 0)
        return 0.5 * m;                          /* subnormal: m * 2^(1-1) / 2 */
    return (1.0 + 0.5 * m) * ldexp(1.0, e - 1);  /* normal: (1 + m/2) * 2^(e-1) */
}

double orc_e2m1_value(int code)
{
    double v = e2m1_magnitude(code & 7);
    return (code & 8) ? -v : v;
}

/* R3: nearest magnitude, ties to the even code (even mantissa bit), values
 * above 6 go to 6 because 6 is the nearest grid point; sign bit from v.     */
int orc_e2m1_encode(float v)
{
    double a = fabs((double)v);
    if (a >= 6.0)                                /* saturate (also keeps huge |v| exact) */
        return (signbit(v) ? 8 : 0) | 7;
    int best = 0;
    double best_d = a;
    for (int k = 1; k < 8; k++) {
        double d = fabs(a - e2m1_magnitude(k));
        if (d < best_d || (d == best_d && (k & 1) == 0)) {
            best = k;
            best_d = d;
        }
    }
    return (signbit(v) ? 8 : 0) | best;
}

/* ======================================================================== */
/* E4M3 (OCP FP8 e4m3fn): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 */
/* mantissa; subnormals m * 2^-9; 0x7F / 0xFF are NaN; largest finite 448.  */
/* ======================================================================== */
double orc_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = m * ldexp(1.0, -9);
    else
        v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -v : v;
}

static double g_e4m3_table[127];   /* values of codes 0x00..0x7E */
static pthread_once_t g_e4m3_once = PTHREAD_ONCE_INIT;

static void e4m3_table_init(void)
{
    for (int c = 0; c <= 0x7E; c++)
        g_e4m3_table[c] = orc_e4m3_value(c);
}

/* Nearest non-negative finite E4M3 code to a >= 0, ties to the even code. */
static int e4m3_nearest_magnitude(double a)
{
    pthread_once(&g_e4m3_once, e4m3_table_init);
    if (a >= 448.0)
        return 0x7E;
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= 0x7E; c++) {
        double d = fabs(a - g_e4m3_table[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* Block-scale encode: clamp at the recipe maximum (itself an E4M3 value),
 * then round to nearest even. For sf >= 0.                                  */
int orc_e4m3_encode_scale(float sf, float e4m3_max)
{
    float x = sf < e4m3_max ? sf : e4m3_max;
    return e4m3_nearest_magnitude((double)x);
}

/* R8: round to nearest even with saturation to the largest finite value;
 * the sign is kept (so -0 gives 0x80); NaN stays NaN.                      */
int orc_e4m3_encode_satfinite(float p)
{
    int sign = signbit(p) ? 0x80 : 0;
    if (isnan(p))
        return sign | 0x7F;
    return sign | e4m3_nearest_magnitude(fabs((double)p));
}

/* ======================================================================== */
/* IEEE binary16 and bfloat16                                               */
/* ======================================================================== */
struct half_fmt { int p, ebits, bias, emin, emax; };
static const struct half_fmt FMT_F16 = {10, 5, 15, -14, 15};
static const struct half_fmt FMT_BF16 = {7, 8, 127, -126, 127};

double orc_half_value(uint16_t bits, int is_bf16)
{
    const struct half_fmt *f = is_bf16 ? &FMT_BF16 : &FMT_F16;
    int s = bits >> 15;
    int ef = (bits >> f->p) & ((1 << f->ebits) - 1);
    int m = bits & ((1 << f->p) - 1);
    double v;
    if (ef == (1 << f->ebits) - 1)
        v = m ? NAN : INFINITY;
    else if (ef == 0)
        v = ldexp((double)m, f->emin - f->p);
    else
        v = ldexp(1.0 + ldexp((double)m, -f->p), ef - f->bias);
    return s ? -v : v;
}

/* real number (held exactly in a double) -> 16-bit float, round to nearest,
 * ties to even, by the definition: find the representable neighbours below
 * and above |x| at the spacing of its binade (or the subnormal spacing), take
 * the nearer, on a tie the one with an even last mantissa bit; past the
 * largest finite value -> inf.                                              */
static uint16_t round_half_exact(double x, int is_bf16)
{
    const struct half_fmt *f = is_bf16 ? &FMT_BF16 : &FMT_F16;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    uint16_t exp_ones = (uint16_t)(((1u << f->ebits) - 1u) << f->p);
    if (isnan(x))
        return (uint16_t)(sign | exp_ones | (1u << (f->p - 1)));
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | exp_ones);
    int e;
    if (a < ldexp(1.0, f->emin)) {
        e = f->emin;
    } else {
        frexp(a, &e);
        e -= 1;                                   /* a in [2^e, 2^(e+1)) */
    }
    double ulp = ldexp(1.0, e - f->p);
    double q = a / ulp;                           /* exact: power-of-two divisor */
    double n = floor(q), r = q - n;
    if (r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;
    double val = n * ulp;
    double max_finite = (2.0 - ldexp(1.0, -f->p)) * ldexp(1.0, f->emax);
    if (val > max_finite)
        return (uint16_t)(sign | exp_ones);
    if (val < ldexp(1.0, f->emin))                /* subnormal or zero */
        return (uint16_t)(sign | (uint16_t)n);
    int ev;
    frexp(val, &ev);
    ev -= 1;
    uint16_t mant = (uint16_t)(val / ldexp(1.0, ev - f->p) - ldexp(1.0, f->p));
    uint16_t ef = (uint16_t)(ev + f->bias);
    return (uint16_t)(sign | (uint16_t)(ef << f->p) | mant);
}

/* fp32 -> 16-bit float (RNE) */
uint16_t orc_round_half(float x, int is_bf16)
{
    return round_half_exact((double)x, is_bf16);
}

/* the IEEE binary16 value nearest to v (ties to even), as a double */
static double f16_round(double v)
{
    return orc_half_value(round_half_exact(v, 0), 0);
}

void orc_e2m1_encode_array(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (uint8_t)orc_e2m1_encode(v[i]);
}

void orc_e4m3_encode_scale_array(const float *sf, int64_t n, float e4m3_max, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (uint8_t)orc_e4m3_encode_scale(sf[i], e4m3_max);
}

void orc_e4m3_encode_satfinite_array(const float *p, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (uint8_t)orc_e4m3_encode_satfinite(p[i]);
}

void orc_round_half_array(const float *x, int64_t n, int is_bf16, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_round_half(x[i], is_bf16);
}

/* ======================================================================== */
/* Block quantization ([AP] description of k_scale; [R46])                  */
/* ======================================================================== */

/* One candidate: block scale from amax / C (R1), elements encoded against
 * the decoded factor E4M3(s) * g (R2, R3). Returns the scale byte and the
 * fp32 decode factor.                                                       */
static int quantize_candidate(const float *x, float amax, float g, float C, float clamp,
                              uint8_t *codes, float *dec_out)
{
    float t = C * g;
    float sf = amax / t;
    int s = orc_e4m3_encode_scale(sf, clamp);
    float dec = (float)orc_e4m3_value(s) * g;
    float inv = (dec == 0.0f) ? 0.0f : 1.0f / dec;
    for (int i = 0; i < 16; i++) {
        float v = x[i] * inv;
        codes[i] = (uint8_t)orc_e2m1_encode(v);
    }
    *dec_out = dec;
    return s;
}

/* R5: dequantize with the candidate, score in fp32, pairwise tree sum. */
static float candidate_error(const float *x, const uint8_t *codes, float dec, int err_mode)
{
    float t[16];
    for (int i = 0; i < 16; i++) {
        float deq = dec * (float)orc_e2m1_value(codes[i]);
        float d = x[i] - deq;
        t[i] = (err_mode == 0) ? d * d : fabsf(d);
    }
    for (int w = 16; w > 1; w /= 2)
        for (int j = 0; j < w / 2; j++)
            t[j] = t[2 * j] + t[2 * j + 1];
    return t[0];
}

/* R12: the same error in IEEE binary16 arithmetic ("fast math"): the input
 * and the fp32 reconstruction are each rounded to fp16, then the difference,
 * the square (MSE) and every sum of the pairwise tree are rounded to fp16.
 * Each operation is done exactly in double (the operands are fp16 values, so
 * differences, squares and sums are exact there) and rounded once.          */
static float candidate_error_fp16(const float *x, const uint8_t *codes, float dec, int err_mode)
{
    double t[16];
    for (int i = 0; i < 16; i++) {
        float deq = dec * (float)orc_e2m1_value(codes[i]);
        double d = f16_round(f16_round((double)x[i]) - f16_round((double)deq));
        t[i] = (err_mode == 0) ? f16_round(d * d) : fabs(d);
    }
    for (int w = 16; w > 1; w /= 2)
        for (int j = 0; j < w / 2; j++)
            t[j] = f16_round(t[2 * j] + t[2 * j + 1]);
    return (float)t[0];
}

static int recipe_ok(const orc_recipe_t *r)
{
    if (!r)
        return 1;
    if (!(r->e4m3_max > 0.0f && r->e4m3_max <= 448.0f))
        return 0;
    /* the clamp must itself be an E4M3 value */
    if ((float)orc_e4m3_value(e4m3_nearest_magnitude(r->e4m3_max)) != r->e4m3_max)
        return 0;
    if (r->four_over_six && r->err_mode != 0 && r->err_mode != 1)
        return 0;
    return 1;
}

static void quantize_block_unchecked(const float *x, float g, const orc_recipe_t *r,
                                     uint8_t *codes, uint8_t *scale,
                                     float *err6, float *err4, int *chose4)
{
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float e4m3_max = r ? r->e4m3_max : 448.0f;
    if (!r || !r->four_over_six) {
        float dec;
        *scale = (uint8_t)quantize_candidate(x, amax, g, 6.0f, e4m3_max, codes, &dec);
        if (err6) *err6 = 0.0f;
        if (err4) *err4 = 0.0f;
        if (chose4) *chose4 = 0;
        return;
    }
    uint8_t c6[16], c4[16];
    float d6, d4;
    int s6 = quantize_candidate(x, amax, g, 6.0f, e4m3_max, c6, &d6);   /* R4 */
    int s4 = quantize_candidate(x, amax, g, 4.0f, 448.0f, c4, &d4);     /* R4 */
    float e6 = r->err_fp16 ? candidate_error_fp16(x, c6, d6, r->err_mode) : candidate_error(x, c6, d6, r->err_mode);
    float e4 = r->err_fp16 ? candidate_error_fp16(x, c4, d4, r->err_mode) : candidate_error(x, c4, d4, r->err_mode);
    int take4 = e4 < e6;                          /* R5; an inf or NaN error never wins */
    memcpy(codes, take4 ? c4 : c6, 16);
    *scale = (uint8_t)(take4 ? s4 : s6);
    if (err6) *err6 = e6;
    if (err4) *err4 = e4;
    if (chose4) *chose4 = take4;
}

int orc_quantize_block(const float *x16, float g, const orc_recipe_t *recipe,
                       uint8_t *codes16, uint8_t *scale_byte,
                       float *err6, float *err4, int *chose4)
{
    if (!x16 || !codes16 || !scale_byte || !recipe_ok(recipe))
        return -1;
    if (!(g > 0.0f) || !isfinite(g))
        return -2;
    for (int i = 0; i < 16; i++)
        if (!isfinite(x16[i]))
            return -3;
    quantize_block_unchecked(x16, g, recipe, codes16, scale_byte, err6, err4, chose4);
    return 0;
}

/* R6 */
float orc_global_scale(const uint16_t *x, int64_t n, int is_bf16, float e4m3_max)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf((float)orc_half_value(x[i], is_bf16));
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f)
        return 1.0f;
    float denom = 6.0f * e4m3_max;
    return amax / denom;
}

/* ======================================================================== */
/* a plain parallel-for over independent index ranges                      */
/* ======================================================================== */
typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);
struct range_job { range_fn fn; void *ctx; int64_t lo, hi; };

static void *range_job_run(void *p)
{
    struct range_job *j = (struct range_job *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static void parallel_for(int64_t n, int threads, range_fn fn, void *ctx)
{
    enum { MAXT = 256 };
    if (threads > MAXT)
        threads = MAXT;
    if (threads > n)
        threads = (int)n;
    if (threads <= 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t tid[MAXT];
    struct range_job jobs[MAXT];
    int started = 0;
    for (int t = 0; t < threads; t++) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = n * t / threads;
        jobs[t].hi = n * (t + 1) / threads;
        if (pthread_create(&tid[t], NULL, range_job_run, &jobs[t]) == 0)
            started = t + 1;
        else
            break;
    }
    /* any range whose thread could not start runs here */
    for (int t = started; t < threads; t++)
        range_job_run(&jobs[t]);
    for (int t = 0; t < started; t++)
        pthread_join(tid[t], NULL);
}

/* ======================================================================== */
/* shared cache-geometry checks                                             */
/* ======================================================================== */
static int cache_ok(const orc_cache_t *c)
{
    if (!c || !c->k_data || !c->v_data || !c->k_sf || !c->v_sf)
        return 0;
    if (c->page_size <= 0 || c->num_heads <= 0 || c->head_dim <= 0 || c->num_pages <= 0)
        return 0;
    if (c->head_dim % 16 != 0)
        return 0;
    if (c->layout != 0 && c->layout != 1)
        return 0;
    int64_t data_page = (int64_t)c->page_size * c->num_heads * (c->head_dim / 2);
    int64_t sf_page = (int64_t)c->page_size * c->num_heads * (c->head_dim / 16);
    if (c->k_page_stride < data_page || c->v_page_stride < data_page)
        return 0;
    if (c->k_sf_page_stride < sf_page || c->v_sf_page_stride < sf_page)
        return 0;
    return 1;
}

/* row index of (slot, head) inside a page: NHD [ps, H, *], HND [H, ps, *] */
static int64_t page_row(const orc_cache_t *c, int64_t slot, int64_t h)
{
    return c->layout == 0 ? slot * c->num_heads + h : h * c->page_size + slot;
}

/* ======================================================================== */
/* quantize-append [AP]                                                      */
/* ======================================================================== */
struct append_ctx {
    const orc_cache_t *c;
    const uint16_t *key, *value;
    int bf16;
    const int32_t *bi, *pos, *indices, *indptr;
    float ks, vs;
    const orc_recipe_t *recipe;
};

static void append_rows(void *vctx, int64_t lo, int64_t hi)
{
    const struct append_ctx *a = (const struct append_ctx *)vctx;
    const orc_cache_t *c = a->c;
    const int64_t H = c->num_heads, D = c->head_dim, ps = c->page_size;
    for (int64_t r = lo; r < hi; r++) {
        int64_t b = a->bi[r], p = a->pos[r];
        /* the row's page is entry p / ps of request b's page list; slot p % ps */
        int64_t page = a->indices[a->indptr[b] + p / ps];
        int64_t slot = p % ps;
        for (int kv = 0; kv < 2; kv++) {
            const uint16_t *src = kv ? a->value : a->key;
            float g = kv ? a->vs : a->ks;
            uint8_t *data = (kv ? c->v_data : c->k_data) + page * (kv ? c->v_page_stride : c->k_page_stride);
            uint8_t *sf = (kv ? c->v_sf : c->k_sf) + page * (kv ? c->v_sf_page_stride : c->k_sf_page_stride);
            for (int64_t h = 0; h < H; h++) {
                int64_t row = page_row(c, slot, h);
                uint8_t *drow = data + row * (D / 2);
                uint8_t *srow = sf + row * (D / 16);
                for (int64_t blk = 0; blk < D / 16; blk++) {
                    float x[16];
                    uint8_t codes[16], s;
                    for (int i = 0; i < 16; i++)
                        x[i] = (float)orc_half_value(src[(r * H + h) * D + blk * 16 + i], a->bf16);
                    quantize_block_unchecked(x, g, a->recipe, codes, &s, NULL, NULL, NULL);
                    srow[blk] = s;
                    /* low nibble = even element, high nibble = odd element */
                    for (int j = 0; j < 8; j++)
                        drow[blk * 8 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
                }
            }
        }
    }
}

int orc_quantize_append(const orc_cache_t *cache,
                        const uint16_t *key, const uint16_t *value, int in_is_bf16, int64_t nnz,
                        const int32_t *batch_indices, const int32_t *positions,
                        const int32_t *kv_indices, const int32_t *kv_indptr,
                        const int32_t *kv_last_page_len, int32_t batch_size,
                        float k_scale, float v_scale, const orc_recipe_t *recipe, int threads)
{
    if (!cache_ok(cache) || !recipe_ok(recipe) || nnz < 0 || batch_size < 0)
        return -1;
    if (nnz == 0)
        return 0;
    if (!key || !value || !batch_indices || !positions || !kv_indices || !kv_indptr || !kv_last_page_len)
        return -1;
    if (!(k_scale > 0.0f) || !isfinite(k_scale) || !(v_scale > 0.0f) || !isfinite(v_scale))
        return -2;
    const int64_t H = cache->num_heads, D = cache->head_dim, ps = cache->page_size;
    for (int64_t i = 0; i < nnz * H * D; i++)
        if (!isfinite(orc_half_value(key[i], in_is_bf16)) || !isfinite(orc_half_value(value[i], in_is_bf16)))
            return -3;
    /* values: each row must fall inside the space its request has reserved */
    for (int64_t r = 0; r < nnz; r++) {
        int64_t b = batch_indices[r], p = positions[r];
        if (b < 0 || b >= batch_size || p < 0)
            return -4;
        int64_t n_pages = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        int64_t last = kv_last_page_len[b];
        if (n_pages < 1 || last < 1 || last > ps)
            return -4;
        if (p >= (n_pages - 1) * ps + last)
            return -4;
        int64_t page = kv_indices[kv_indptr[b] + p / ps];
        if (page < 0 || page >= cache->num_pages)
            return -4;
    }
    struct append_ctx ctx = {cache, key, value, in_is_bf16, batch_indices, positions,
                             kv_indices, kv_indptr, k_scale, v_scale, recipe};
    parallel_for(nnz, threads, append_rows, &ctx);
    return 0;
}

/* ======================================================================== */
/* gather-dequantize [DQ]                                                    */
/* ======================================================================== */
struct dequant_ctx {
    const orc_cache_t *c;
    const void *bt;
    int bt64;
    int64_t bt_row_stride;
    const int32_t *seq_lens;
    float ks, vs;
    uint16_t *out_k, *out_v;
    int bf16;
    int64_t max_seq_len;
};

static int64_t table_entry(const void *bt, int is64, int64_t idx)
{
    return is64 ? ((const int64_t *)bt)[idx] : (int64_t)((const int32_t *)bt)[idx];
}

static void dequant_requests(void *vctx, int64_t lo, int64_t hi)
{
    const struct dequant_ctx *a = (const struct dequant_ctx *)vctx;
    const orc_cache_t *c = a->c;
    const int64_t H = c->num_heads, D = c->head_dim, ps = c->page_size, T = a->max_seq_len;
    for (int64_t b = lo; b < hi; b++) {
        int64_t len = a->seq_lens[b] < T ? a->seq_lens[b] : T;
        for (int64_t t = 0; t < len; t++) {
            int64_t page = table_entry(a->bt, a->bt64, b * a->bt_row_stride + t / ps);
            int64_t slot = t % ps;
            for (int kv = 0; kv < 2; kv++) {
                const uint8_t *data = (kv ? c->v_data : c->k_data) + page * (kv ? c->v_page_stride : c->k_page_stride);
                const uint8_t *sf = (kv ? c->v_sf : c->k_sf) + page * (kv ? c->v_sf_page_stride : c->k_sf_page_stride);
                float g = kv ? a->vs : a->ks;
                uint16_t *out = kv ? a->out_v : a->out_k;
                for (int64_t h = 0; h < H; h++) {
                    int64_t row = page_row(c, slot, h);
                    for (int64_t e = 0; e < D; e++) {
                        uint8_t byte = data[row * (D / 2) + e / 2];
                        int code = (e & 1) ? (byte >> 4) : (byte & 15);
                        uint8_t s = sf[row * (D / 16) + e / 16];
                        float dec = (float)orc_e4m3_value(s) * g;          /* R7 */
                        float y = dec * (float)orc_e2m1_value(code);
                        out[((b * T + t) * H + h) * D + e] = orc_round_half(y, a->bf16);
                    }
                }
            }
        }
    }
}

int orc_dequantize_paged(const orc_cache_t *cache,
                         const void *block_tables, int bt_is_int64, int64_t bt_row_stride, int32_t bt_cols,
                         const int32_t *seq_lens, int32_t batch_size,
                         float k_scale, float v_scale,
                         uint16_t *out_k, uint16_t *out_v, int out_is_bf16, int32_t max_seq_len,
                         int threads)
{
    if (!cache_ok(cache) || batch_size < 0 || max_seq_len < 0 || bt_cols < 0)
        return -1;
    if (batch_size == 0 || max_seq_len == 0)
        return 0;
    if (!block_tables || !seq_lens || !out_k || !out_v || bt_row_stride < bt_cols)
        return -1;
    if (!isfinite(k_scale) || !isfinite(v_scale))
        return -2;
    const int64_t ps = cache->page_size;
    for (int64_t b = 0; b < batch_size; b++) {
        if (seq_lens[b] < 0)
            return -4;
        int64_t len = seq_lens[b] < max_seq_len ? seq_lens[b] : max_seq_len;
        int64_t pages = (len + ps - 1) / ps;
        if (pages > bt_cols)
            return -4;
        for (int64_t j = 0; j < pages; j++) {
            int64_t page = table_entry(block_tables, bt_is_int64, b * bt_row_stride + j);
            if (page < 0 || page >= cache->num_pages)
                return -4;
        }
    }
    struct dequant_ctx ctx = {cache, block_tables, bt_is_int64, bt_row_stride, seq_lens,
                              k_scale, v_scale, out_k, out_v, out_is_bf16, max_seq_len};
    parallel_for(batch_size, threads, dequant_requests, &ctx);
    return 0;
}

/* ======================================================================== */
/* materialize-FP8 [MF]                                                      */
/* ======================================================================== */
struct materialize_ctx {
    const orc_cache_t *c;
    int v_interleaved;
    const int32_t *bt;
    int shared;
    int64_t bt_row_stride, bt_kv_stride;
    const int32_t *seq_lens, *indptr;
    uint8_t *out;
    int32_t *table;
    int64_t maxp;
    int64_t batch;
};

/* the threads split the reserved output pages p < indptr[batch]: page p
 * belongs to the request b with indptr[b] <= p < indptr[b + 1] and is its
 * page j = p - indptr[b], converted when j < ceil(seq_lens[b] / ps) */
static void materialize_pages(void *vctx, int64_t lo, int64_t hi)
{
    const struct materialize_ctx *a = (const struct materialize_ctx *)vctx;
    const orc_cache_t *c = a->c;
    const int64_t H = c->num_heads, D = c->head_dim, ps = c->page_size, nb = D / 16;
    const int64_t half_page = H * ps * D;        /* bytes of the K (or V) half of an FP8 page */
    for (int64_t p = lo; p < hi; p++) {
        int64_t b = 0, top = a->batch;           /* the last b with indptr[b] <= p */
        while (top - b > 1) {
            int64_t mid = (b + top) / 2;
            if (a->indptr[mid] <= p)
                b = mid;
            else
                top = mid;
        }
        int64_t n = (a->seq_lens[b] + ps - 1) / ps;
        int64_t j = p - a->indptr[b];
        if (j < n) {
            int64_t dst = (int64_t)a->indptr[b] + j + 1;
            int64_t kpage = a->bt[b * a->bt_row_stride + j];
            int64_t vpage = a->shared ? kpage : a->bt[b * a->bt_row_stride + a->bt_kv_stride + j];
            for (int kv = 0; kv < 2; kv++) {
                int64_t page = kv ? vpage : kpage;
                const uint8_t *data = (kv ? c->v_data : c->k_data) + page * (kv ? c->v_page_stride : c->k_page_stride);
                const uint8_t *sf = (kv ? c->v_sf : c->k_sf) + page * (kv ? c->v_sf_page_stride : c->k_sf_page_stride);
                uint8_t *o = a->out + (dst * 2 + kv) * half_page;
                for (int64_t h = 0; h < H; h++)
                    for (int64_t t = 0; t < ps; t++)            /* R8: the whole page */
                        for (int64_t e = 0; e < D; e++) {
                            uint8_t byte = data[(h * ps + t) * (D / 2) + e / 2];
                            int code = (e & 1) ? (byte >> 4) : (byte & 15);
                            int64_t sidx;
                            if (kv == 1 && a->v_interleaved)     /* R9 */
                                sidx = h * ps * nb + ((t / 4) * nb + e / 16) * 4 + t % 4;
                            else
                                sidx = (h * ps + t) * nb + e / 16;
                            float prod = (float)orc_e2m1_value(code) * (float)orc_e4m3_value(sf[sidx]);
                            o[(h * ps + t) * D + e] = (uint8_t)orc_e4m3_encode_satfinite(prod);
                        }
            }
            a->table[b * a->maxp + j] = (int32_t)dst;
        }
    }
}

int orc_materialize_fp8(const orc_cache_t *cache, int v_sf_interleaved,
                        const int32_t *block_tables, int shared, int64_t bt_row_stride,
                        int64_t bt_kv_stride, int32_t bt_cols,
                        const int32_t *seq_lens, const int32_t *kv_page_indptr, int32_t batch_size,
                        uint8_t *out, int64_t num_out_pages,
                        int32_t *fp8_block_tables, int32_t max_pages_per_seq, int threads)
{
    if (!cache_ok(cache) || cache->layout != 1 || batch_size < 0 || !out || num_out_pages < 1)
        return -1;
    if (v_sf_interleaved && cache->page_size % 4 != 0)
        return -1;
    const int64_t H = cache->num_heads, D = cache->head_dim, ps = cache->page_size;
    /* page 0 of the FP8 copy is zero, K and V halves */
    memset(out, 0, (size_t)(2 * H * ps * D));
    if (batch_size == 0)
        return 0;
    if (!block_tables || !seq_lens || !kv_page_indptr || !fp8_block_tables)
        return -1;
    if (max_pages_per_seq < 0 || bt_cols < max_pages_per_seq)
        return -1;
    /* values the launcher does not check; the oracle rejects them */
    if (kv_page_indptr[0] != 0)
        return -4;
    for (int64_t b = 0; b < batch_size; b++) {
        int64_t len = seq_lens[b];
        int64_t n = (len + ps - 1) / ps;
        if (len < 0 || len > (int64_t)max_pages_per_seq * ps)
            return -4;
        if ((int64_t)kv_page_indptr[b + 1] - kv_page_indptr[b] < n)
            return -4;
        for (int64_t j = 0; j < n; j++) {
            int64_t kp = block_tables[b * bt_row_stride + j];
            int64_t vp = shared ? kp : block_tables[b * bt_row_stride + bt_kv_stride + j];
            if (kp < 0 || kp >= cache->num_pages || vp < 0 || vp >= cache->num_pages)
                return -4;
        }
    }
    if ((int64_t)kv_page_indptr[batch_size] + 1 > num_out_pages)
        return -4;
    struct materialize_ctx ctx = {cache, v_sf_interleaved, block_tables, shared, bt_row_stride,
                                  bt_kv_stride, seq_lens, kv_page_indptr, out, fp8_block_tables,
                                  max_pages_per_seq, batch_size};
    parallel_for(kv_page_indptr[batch_size], threads, materialize_pages, &ctx);
    return 0;
}

/* ======================================================================== */
/* contiguous codec [KV], R10                                                */
/* ======================================================================== */
struct contig_q_ctx {
    const uint16_t *x;
    int bf16;
    int64_t cols;
    float g;
    const orc_recipe_t *recipe;
    uint8_t *codes, *scales;
};

static void quantize_rows(void *vctx, int64_t lo, int64_t hi)
{
    const struct contig_q_ctx *a = (const struct contig_q_ctx *)vctx;
    const int64_t nb = a->cols / 16;
    for (int64_t r = lo; r < hi; r++)
        for (int64_t blk = 0; blk < nb; blk++) {
            float x[16];
            uint8_t codes[16], s;
            for (int i = 0; i < 16; i++)
                x[i] = (float)orc_half_value(a->x[r * a->cols + blk * 16 + i], a->bf16);
            quantize_block_unchecked(x, a->g, a->recipe, codes, &s, NULL, NULL, NULL);
            a->scales[r * nb + blk] = s;
            for (int j = 0; j < 8; j++)
                a->codes[r * (a->cols / 2) + blk * 8 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
}

int orc_quantize_contiguous(const uint16_t *x, int in_is_bf16, int64_t rows, int64_t cols, float g,
                            const orc_recipe_t *recipe, uint8_t *codes, uint8_t *scales, int threads)
{
    if (!recipe_ok(recipe) || rows < 0 || cols < 0 || cols % 16 != 0)
        return -1;
    if (rows == 0 || cols == 0)
        return 0;
    if (!x || !codes || !scales)
        return -1;
    if (!(g > 0.0f) || !isfinite(g))
        return -2;
    for (int64_t i = 0; i < rows * cols; i++)
        if (!isfinite(orc_half_value(x[i], in_is_bf16)))
            return -3;
    struct contig_q_ctx ctx = {x, in_is_bf16, cols, g, recipe, codes, scales};
    parallel_for(rows, threads, quantize_rows, &ctx);
    return 0;
}

struct contig_dq_ctx {
    const uint8_t *codes, *scales;
    int64_t cols;
    float g;
    uint16_t *out;
    int bf16;
};

static void dequantize_rows(void *vctx, int64_t lo, int64_t hi)
{
    const struct contig_dq_ctx *a = (const struct contig_dq_ctx *)vctx;
    for (int64_t r = lo; r < hi; r++)
        for (int64_t e = 0; e < a->cols; e++) {
            uint8_t byte = a->codes[r * (a->cols / 2) + e / 2];
            int code = (e & 1) ? (byte >> 4) : (byte & 15);
            float dec = (float)orc_e4m3_value(a->scales[r * (a->cols / 16) + e / 16]) * a->g;   /* R7 */
            a->out[r * a->cols + e] = orc_round_half(dec * (float)orc_e2m1_value(code), a->bf16);
        }
}

int orc_dequantize_contiguous(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                              float g, uint16_t *out, int out_is_bf16, int threads)
{
    if (rows < 0 || cols < 0 || cols % 16 != 0)
        return -1;
    if (rows == 0 || cols == 0)
        return 0;
    if (!codes || !scales || !out)
        return -1;
    if (!isfinite(g))
        return -2;
    struct contig_dq_ctx ctx = {codes, scales, cols, g, out, out_is_bf16};
    parallel_for(rows, threads, dequantize_rows, &ctx);
    return 0;
}

/* ======================================================================== */
/* whole-pool quantizer [KV], R11                                            */
/* ======================================================================== */
struct pool_ctx {
    const orc_cache_t *c;
    const uint16_t *k_in, *v_in;
    int bf16;
    float ks, vs;
    const orc_recipe_t *recipe;
    int v_interleaved;
};

static void quantize_pages(void *vctx, int64_t lo, int64_t hi)
{
    const struct pool_ctx *a = (const struct pool_ctx *)vctx;
    const orc_cache_t *c = a->c;
    const int64_t H = c->num_heads, D = c->head_dim, ps = c->page_size, nb = D / 16;
    for (int64_t page = lo; page < hi; page++)
        for (int kv = 0; kv < 2; kv++) {
            const uint16_t *src = (kv ? a->v_in : a->k_in) + page * ps * H * D;
            float g = kv ? a->vs : a->ks;
            uint8_t *data = (kv ? c->v_data : c->k_data) + page * (kv ? c->v_page_stride : c->k_page_stride);
            uint8_t *sf = (kv ? c->v_sf : c->k_sf) + page * (kv ? c->v_sf_page_stride : c->k_sf_page_stride);
            for (int64_t t = 0; t < ps; t++)
                for (int64_t h = 0; h < H; h++) {
                    int64_t row = page_row(c, t, h);       /* the input page has the same row order */
                    for (int64_t blk = 0; blk < nb; blk++) {
                        float x[16];
                        uint8_t codes[16], s;
                        for (int i = 0; i < 16; i++)
                            x[i] = (float)orc_half_value(src[row * D + blk * 16 + i], a->bf16);
                        quantize_block_unchecked(x, g, a->recipe, codes, &s, NULL, NULL, NULL);
                        for (int j = 0; j < 8; j++)
                            data[row * (D / 2) + blk * 8 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
                        int64_t sidx;
                        if (kv == 1 && a->v_interleaved)         /* R9 / R11 */
                            sidx = h * ps * nb + ((t / 4) * nb + blk) * 4 + t % 4;
                        else
                            sidx = row * nb + blk;
                        sf[sidx] = s;
                    }
                }
        }
}

int orc_quantize_paged_cache(const orc_cache_t *cache, const uint16_t *k_in, const uint16_t *v_in,
                             int in_is_bf16, float k_scale, float v_scale, const orc_recipe_t *recipe,
                             int v_sf_interleaved, int threads)
{
    if (!cache_ok(cache) || !recipe_ok(recipe) || !k_in || !v_in)
        return -1;
    if (v_sf_interleaved && (cache->layout != 1 || cache->page_size % 4 != 0))
        return -1;
    if (!(k_scale > 0.0f) || !isfinite(k_scale) || !(v_scale > 0.0f) || !isfinite(v_scale))
        return -2;
    const int64_t n = (int64_t)cache->num_pages * cache->page_size * cache->num_heads * cache->head_dim;
    for (int64_t i = 0; i < n; i++)
        if (!isfinite(orc_half_value(k_in[i], in_is_bf16)) || !isfinite(orc_half_value(v_in[i], in_is_bf16)))
            return -3;
    struct pool_ctx ctx = {cache, k_in, v_in, in_is_bf16, k_scale, v_scale, recipe, v_sf_interleaved};
    parallel_for(cache->num_pages, threads, quantize_pages, &ctx);
    return 0;
}

/* ======================================================================== */
/* decode attention over the paged cache, R13                               */
/* ======================================================================== */
struct attn_ctx {
    const orc_cache_t *c;
    const uint16_t *q;
    int bf16;
    int64_t hq;
    const int32_t *bt;
    int64_t bt_row_stride;
    const int32_t *seq_lens;
    double gk, gv, sm;
    double *out;
};

/* exact dequantized value of element e of (page, slot, h) */
static double cache_value(const orc_cache_t *c, int kv, int64_t page, int64_t slot, int64_t h, int64_t e, double g)
{
    const int64_t D = c->head_dim;
    const uint8_t *data = (kv ? c->v_data : c->k_data) + page * (kv ? c->v_page_stride : c->k_page_stride);
    const uint8_t *sf = (kv ? c->v_sf : c->k_sf) + page * (kv ? c->v_sf_page_stride : c->k_sf_page_stride);
    int64_t row = page_row(c, slot, h);
    uint8_t byte = data[row * (D / 2) + e / 2];
    int code = (e & 1) ? (byte >> 4) : (byte & 15);
    return orc_e2m1_value(code) * orc_e4m3_value(sf[row * (D / 16) + e / 16]) * g;
}

static void attention_requests(void *vctx, int64_t lo, int64_t hi)
{
    const struct attn_ctx *a = (const struct attn_ctx *)vctx;
    const orc_cache_t *c = a->c;
    const int64_t H = c->num_heads, D = c->head_dim, ps = c->page_size, group = a->hq / H;
    for (int64_t b = lo; b < hi; b++) {
        int64_t len = a->seq_lens[b];
        double *s = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
        for (int64_t qh = 0; qh < a->hq; qh++) {
            int64_t h = qh / group;
            const uint16_t *qv = a->q + (b * a->hq + qh) * D;
            double *o = a->out + (b * a->hq + qh) * D;
            for (int64_t e = 0; e < D; e++)
                o[e] = 0.0;
            if (len <= 0)
                continue;
            double m = -INFINITY;
            for (int64_t t = 0; t < len; t++) {
                int64_t page = a->bt[b * a->bt_row_stride + t / ps];
                double dot = 0.0;
                for (int64_t e = 0; e < D; e++)
                    dot += orc_half_value(qv[e], a->bf16) * cache_value(c, 0, page, t % ps, h, e, a->gk);
                s[t] = a->sm * dot;
                if (s[t] > m)
                    m = s[t];
            }
            double denom = 0.0;
            for (int64_t t = 0; t < len; t++) {
                s[t] = exp(s[t] - m);
                denom += s[t];
            }
            for (int64_t t = 0; t < len; t++) {
                int64_t page = a->bt[b * a->bt_row_stride + t / ps];
                double p = s[t] / denom;
                for (int64_t e = 0; e < D; e++)
                    o[e] += p * cache_value(c, 1, page, t % ps, h, e, a->gv);
            }
        }
        free(s);
    }
}

int orc_decode_attention(const orc_cache_t *cache, const uint16_t *q, int q_is_bf16, int32_t num_qo_heads,
                         const int32_t *block_tables, int64_t bt_row_stride, int32_t bt_cols,
                         const int32_t *seq_lens, int32_t batch_size, float k_scale, float v_scale,
                         float sm_scale, double *out, int threads)
{
    if (!cache_ok(cache) || batch_size < 0 || num_qo_heads <= 0 || num_qo_heads % cache->num_heads != 0)
        return -1;
    if (batch_size == 0)
        return 0;
    if (!q || !block_tables || !seq_lens || !out || bt_row_stride < bt_cols)
        return -1;
    if (!isfinite(k_scale) || !isfinite(v_scale) || !isfinite(sm_scale))
        return -2;
    const int64_t ps = cache->page_size;
    for (int64_t b = 0; b < batch_size; b++) {
        if (seq_lens[b] < 0)
            return -4;
        int64_t pages = (seq_lens[b] + ps - 1) / ps;
        if (pages > bt_cols)
            return -4;
        for (int64_t j = 0; j < pages; j++) {
            int64_t page = block_tables[b * bt_row_stride + j];
            if (page < 0 || page >= cache->num_pages)
                return -4;
        }
    }
    struct attn_ctx ctx = {cache, q, q_is_bf16, num_qo_heads, block_tables, bt_row_stride, seq_lens,
                           (double)k_scale, (double)v_scale, (double)sm_scale, out};
    parallel_for(batch_size, threads, attention_requests, &ctx);
    return 0;
}

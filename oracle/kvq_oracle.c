/*
 * kvq_oracle.c -- plain, slow CPU oracle for the quantized-KV-cache hot path of
 * WUSH-KV (key transform after RoPE, clipped per-token-group quantization, paged
 * packed cache, decode attention over the dequantized cache).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no source, header,
 * table or helper with the HIP library and it includes nothing from it.
 *
 * Sources (page title, section):
 *   [W]  "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" (summary page)
 *        §4.1  GQA cache: several query heads read one KV head; cached keys are
 *              post-normalisation, post-RoPE.
 *        §4.2  one key transform per KV head, applied online after RoPE; the query is
 *              compensated; the value transform is folded into W_V/W_O offline.
 *        §4.3  QuEST quantizer: each token's d channels are one group, RMS-based clip.
 *        §5.3  OSCAR-style percentile-clipped affine quantizer.
 *        App. C.5  values do not enter the softmax.
 *   [N]  "Spend Bits Where Queries Look" (NOVA-KV project page), "Three requirements"
 *        (fixed number of bits per token in a paged cache) and the online-inference
 *        figure (encode once on the write path, decode on every read).
 *
 * The pages give prose only.  Every step below is the plain definition; where the
 * pages leave a choice open this file takes one reading and states it next to the
 * code.  Floating point: built with -O2 -ffp-contract=off and no fast-math, so each
 * fp32 expression rounds exactly as written (IEEE-754, round to nearest even).
 *
 * Inputs must be finite.  Values are fp32 (bf16 and fp16 inputs are passed as the
 * fp32 numbers they represent).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HEAD_DIM 128
#define PAGE_TOKENS 64

int oracle_abi_version(void) { return 1; }

/* ------------------------------------------------------------------------- */
/* binary16 conversions, from the IEEE-754 format definition: 1 sign bit,     */
/* 5 exponent bits with bias 15, 10 fraction bits, subnormal spacing 2^-24.   */
/* ------------------------------------------------------------------------- */

/* Round to nearest, ties to even.  Magnitudes at or above 65520 become infinity. */
uint16_t oracle_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    int e2;
    (void)frexp(a, &e2);      /* a = m * 2^e2 with m in [0.5, 1) */
    int e = e2 - 1;           /* a lies in [2^e, 2^(e+1)) */
    if (e < -14) e = -14;     /* subnormals share the spacing of the lowest binade */
    double m = nearbyint(a / ldexp(1.0, e - 10)); /* exact scaling, then RNE */
    if (m >= 2048.0) { m = 1024.0; e += 1; }      /* rounding carried into next binade */
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    if (m < 1024.0) return (uint16_t)(sign | (uint16_t)m);       /* subnormal */
    return (uint16_t)(sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024)));
}

float oracle_f16_to_f32(uint16_t h)
{
    int ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v;
    if (ex == 0x1F) v = fr ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)fr, -24);
    else v = ldexp((double)(fr + 1024), ex - 25);
    return (float)((h & 0x8000u) ? -v : v);
}

void oracle_f32_to_f16_array(const float* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(x[i]);
}

void oracle_f16_to_f32_array(const uint16_t* h, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------- */
/* O1  key transform after RoPE ([W] §4.2): k' = k . T_K, per KV head.         */
/* Accumulated in fp64 over the given values, then rounded once to fp32.      */
/* The transformed keys are kept in fp32 (they are only an intermediate).     */
/* ------------------------------------------------------------------------- */

/* k: [n][heads][128]; t: [heads][128 (c)][128 (j)] or NULL (identity);
   out: [n][heads][128], out[j] = sum_c k[c] * T[c][j]. */
void oracle_transform_keys(const float* k, const float* t, int64_t n, int heads, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        for (int h = 0; h < heads; ++h) {
            const float* kr = k + (i * heads + h) * HEAD_DIM;
            float* o = out + (i * heads + h) * HEAD_DIM;
            if (!t) { memcpy(o, kr, HEAD_DIM * sizeof(float)); continue; }
            const float* th = t + (int64_t)h * HEAD_DIM * HEAD_DIM;
            for (int j = 0; j < HEAD_DIM; ++j) {
                double acc = 0.0;
                for (int c = 0; c < HEAD_DIM; ++c)
                    acc += (double)kr[c] * (double)th[c * HEAD_DIM + j];
                o[j] = (float)acc;
            }
        }
}

/* ------------------------------------------------------------------------- */
/* O2  clip bounds of one group.                                              */
/* ------------------------------------------------------------------------- */

static int cmp_float(const void* a, const void* b)
{
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

/* Percentile position for probability p over n sorted values: linear interpolation
   between order statistics at rank p*(n-1) (the common "linear" definition).
   p is an fp32 value (the type the cache descriptor carries); rank is formed in fp64
   from it and the fractional weight is rounded once to fp32. */
void oracle_percentile_position(float p, int n, int* i_out, float* f_out)
{
    double rank = (double)p * (double)(n - 1);
    int i = (int)floor(rank);
    if (i < 0) i = 0;
    float f = (float)(rank - (double)i);
    if (i >= n - 1) { i = n - 1; f = 0.0f; }
    *i_out = i;
    *f_out = f;
}

/* Interpolated order statistic: s[i] + f*(s[i+1]-s[i]) as one fused multiply-add
   in fp32, plus +0.0f so that a zero result is +0. */
static float interpolate_sorted(const float* s, int n, float p)
{
    int i; float f;
    oracle_percentile_position(p, n, &i, &f);
    float next = s[i + 1 < n ? i + 1 : n - 1];
    return fmaf(f, next - s[i], s[i]) + 0.0f;
}

/* OSCAR-style percentile clip ([W] §5.3): lo/hi are the p_lo/p_hi percentiles of the
   group's values. */
void oracle_clip_percentile(const float* x, int n, float p_lo, float p_hi, float* lo, float* hi)
{
    float* s = (float*)malloc((size_t)n * sizeof(float));
    memcpy(s, x, (size_t)n * sizeof(float));
    qsort(s, (size_t)n, sizeof(float), cmp_float);
    *lo = interpolate_sorted(s, n, p_lo);
    *hi = interpolate_sorted(s, n, p_hi);
    free(s);
}

/* QuEST-style RMS clip ([W] §4.3): symmetric range [-alpha*rms, +alpha*rms] where
   rms = sqrt(mean(x^2)) over the group's n = 128 channels.  The fp32 sum of squares
   is taken in a fixed order (the pages fix none): one pairwise tree over the channel
   index -- at stride n/2, n/4, ..., 1 (64 .. 1 for a group of 128), element i < stride
   adds element i + stride -- so sq[0] ends as the sum. */
void oracle_clip_rms(const float* x, int n, float alpha, float* lo, float* hi)
{
    float sq[HEAD_DIM];
    for (int i = 0; i < n; ++i) sq[i] = x[i] * x[i];
    for (int stride = n / 2; stride >= 1; stride /= 2)
        for (int i = 0; i < stride; ++i) sq[i] = sq[i] + sq[i + stride];
    float rms = sqrtf(sq[0] / (float)n);
    float cl = alpha * rms;
    *lo = -cl;
    *hi = cl;
}

/* ------------------------------------------------------------------------- */
/* O3/O4  affine codes of one group with fp16 scale and zero.                 */
/* ------------------------------------------------------------------------- */

static float saturate_f16_range(float v)
{
    if (v > 65504.0f) return 65504.0f;
    if (v < -65504.0f) return -65504.0f;
    return v;
}

/* 2^bits levels z + c*s, c = 0..L, L = 2^bits - 1, spanning [lo, hi].  Scale and zero
   are stored as fp16; the codes are computed from the stored (rounded) values so
   that encoder and decoder agree.  A zero scale gives all-zero codes. */
void oracle_quantize_group(const float* x, int n, int bits, float lo, float hi,
                           uint8_t* codes, uint16_t* scale_h, uint16_t* zero_h)
{
    int L = (1 << bits) - 1;
    float s = (hi - lo) / (float)L;
    uint16_t s16 = oracle_f32_to_f16(saturate_f16_range(s));
    uint16_t z16 = oracle_f32_to_f16(saturate_f16_range(lo));
    float sf = oracle_f16_to_f32(s16), zf = oracle_f16_to_f32(z16);
    float r = (sf == 0.0f) ? 0.0f : 1.0f / sf;
    for (int i = 0; i < n; ++i) {
        float t = (x[i] - zf) * r;
        float c = rintf(t);
        if (c < 0.0f) c = 0.0f;
        if (c > (float)L) c = (float)L;
        codes[i] = (uint8_t)c;
    }
    *scale_h = s16;
    *zero_h = z16;
}

enum { ORACLE_PERCENTILE = 0, ORACLE_RMS = 1 };

/* Clip + quantize each row of x [rows][128]. */
void oracle_quantize_rows(const float* x, int64_t rows, int bits, int quantizer,
                          float p_lo, float p_hi, float alpha,
                          uint8_t* codes, uint16_t* scale_h, uint16_t* zero_h,
                          float* lo_out, float* hi_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * HEAD_DIM;
        float lo, hi;
        if (quantizer == ORACLE_RMS) oracle_clip_rms(xr, HEAD_DIM, alpha, &lo, &hi);
        else oracle_clip_percentile(xr, HEAD_DIM, p_lo, p_hi, &lo, &hi);
        oracle_quantize_group(xr, HEAD_DIM, bits, lo, hi, codes + r * HEAD_DIM,
                              scale_h + r, zero_h + r);
        if (lo_out) lo_out[r] = lo;
        if (hi_out) hi_out[r] = hi;
    }
}

/* ------------------------------------------------------------------------- */
/* O5  fixed-width paged layout ([N] "Three requirements").                   */
/*                                                                           */
/* A pool is [num_pages][kv_heads] blocks.  One block holds 64 tokens of one  */
/* KV head:                                                                  */
/*   codes   64*128*bits/8 bytes, read as little-endian 32-bit words (2 or 4 */
/*           bits as below; 3 bits as two planes, see high_plane_position)    */
/*     keys:   word (o * 128*bits/32 + c/(32/bits)), bit (c % (32/bits))*bits  */
/*             (token-major rows)                                             */
/*     values: word ((o/(32/bits)) * 128 + c),      bit (o % (32/bits))*bits   */
/*             (each word holds 32/bits consecutive tokens of one channel)    */
/*   scales  64 x fp16 (token o at byte 2*o after the codes)                  */
/*   zeros   64 x fp16 (token o at byte 128 + 2*o after the scales)           */
/* o = slot % 64 is the token's offset in its page, page = slot / 64.         */
/* ------------------------------------------------------------------------- */

int64_t oracle_block_bytes(int bits)
{
    return (int64_t)PAGE_TOKENS * HEAD_DIM * bits / 8 + 2 * 2 * PAGE_TOKENS;
}

static uint32_t load_word(const uint8_t* p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static void store_word(uint8_t* p, uint32_t w)
{
    p[0] = (uint8_t)(w & 0xFF); p[1] = (uint8_t)((w >> 8) & 0xFF);
    p[2] = (uint8_t)((w >> 16) & 0xFF); p[3] = (uint8_t)((w >> 24) & 0xFF);
}

static void code_position(int which, int bits, int o, int c, int64_t* word, int* bit)
{
    int per_word = 32 / bits;
    if (which == 0) { *word = (int64_t)o * (HEAD_DIM * bits / 32) + c / per_word; *bit = (c % per_word) * bits; }
    else            { *word = (int64_t)(o / per_word) * HEAD_DIM + c;             *bit = (o % per_word) * bits; }
}

/* 3-bit codes are kept as two bit planes, so that each plane packs whole words:     */
/*   low plane  (bits 0-1 of every code): the 2-bit code section, word for word;     */
/*   high plane (bit 2 of every code): 1024 bytes after the low plane (word 512 on):  */
/*     keys    token o's 128 bits are words o*4 + c/32; channel offset u = c % 32 is */
/*             at bit 4*((u % 16)/2) + 2*(u/16) + u % 2                               */
/*     values  word (o/32)*128 + c holds tokens 32*(o/32) .. +31 of channel c; token */
/*             offset t = o % 32 is at bit t % 8 + 16*((t/8) % 2) + 8*(t/16)          */
/* (the in-word orders are a layout choice of this cache; any bijection would do)    */
static void high_plane_position(int which, int o, int c, int64_t* word, int* bit)
{
    const int64_t base = (int64_t)PAGE_TOKENS * HEAD_DIM * 2 / 32;   /* words of the low plane */
    if (which == 0) {
        int u = c % 32;
        *word = base + (int64_t)o * 4 + c / 32;
        *bit = 4 * ((u % 16) / 2) + 2 * (u / 16) + u % 2;
    } else {
        int t = o % 32;
        *word = base + (int64_t)(o / 32) * HEAD_DIM + c;
        *bit = t % 8 + 16 * ((t / 8) % 2) + 8 * (t / 16);
    }
}

static void put_bits(uint8_t* block, int64_t w, int b, uint32_t mask, uint32_t v)
{
    uint32_t word = load_word(block + 4 * w);
    store_word(block + 4 * w, (word & ~(mask << b)) | ((v & mask) << b));
}

static uint8_t* block_at(uint8_t* pool, int64_t page, int h, int kv_heads, int bits)
{
    return pool + (page * kv_heads + h) * oracle_block_bytes(bits);
}

/* Writes one token's group (128 codes + scale + zero) into its block; other bits
   of the block are left as they were. */
void oracle_pack_token(uint8_t* block, int which, int bits, int o, const uint8_t* codes,
                       uint16_t scale_h, uint16_t zero_h)
{
    for (int c = 0; c < HEAD_DIM; ++c) {
        int64_t w; int b;
        if (bits == 3) {
            code_position(which, 2, o, c, &w, &b);
            put_bits(block, w, b, 3u, codes[c]);
            high_plane_position(which, o, c, &w, &b);
            put_bits(block, w, b, 1u, (uint32_t)codes[c] >> 2);
        } else {
            code_position(which, bits, o, c, &w, &b);
            put_bits(block, w, b, (1u << bits) - 1u, codes[c]);
        }
    }
    uint8_t* meta = block + (int64_t)PAGE_TOKENS * HEAD_DIM * bits / 8;
    meta[2 * o] = (uint8_t)(scale_h & 0xFF); meta[2 * o + 1] = (uint8_t)(scale_h >> 8);
    meta[2 * PAGE_TOKENS + 2 * o] = (uint8_t)(zero_h & 0xFF);
    meta[2 * PAGE_TOKENS + 2 * o + 1] = (uint8_t)(zero_h >> 8);
}

void oracle_unpack_token(const uint8_t* block, int which, int bits, int o, uint8_t* codes,
                         uint16_t* scale_h, uint16_t* zero_h)
{
    for (int c = 0; c < HEAD_DIM; ++c) {
        int64_t w; int b;
        if (bits == 3) {
            code_position(which, 2, o, c, &w, &b);
            uint32_t lo = (load_word(block + 4 * w) >> b) & 3u;
            high_plane_position(which, o, c, &w, &b);
            codes[c] = (uint8_t)(lo | (((load_word(block + 4 * w) >> b) & 1u) << 2));
        } else {
            code_position(which, bits, o, c, &w, &b);
            codes[c] = (uint8_t)((load_word(block + 4 * w) >> b) & ((1u << bits) - 1u));
        }
    }
    const uint8_t* meta = block + (int64_t)PAGE_TOKENS * HEAD_DIM * bits / 8;
    *scale_h = (uint16_t)(meta[2 * o] | (meta[2 * o + 1] << 8));
    *zero_h = (uint16_t)(meta[2 * PAGE_TOKENS + 2 * o] | (meta[2 * PAGE_TOKENS + 2 * o + 1] << 8));
}

/* ------------------------------------------------------------------------- */
/* Write path: transform (keys only), clip, quantize, pack.                   */
/* k, v: [n][kv_heads][128]; t_k: [kv_heads][128][128] or NULL; slots: [n],   */
/* a negative slot skips the token.  Returns 0, or -1 on an out-of-range slot  */
/* (nothing after that token is written).                                    */
/* ------------------------------------------------------------------------- */
int oracle_append(uint8_t* k_pool, uint8_t* v_pool, int64_t num_pages, int kv_heads,
                  int bits_k, int bits_v, int quant_k, int quant_v,
                  float p_lo, float p_hi, float alpha_k, float alpha_v,
                  const float* k, const float* v, const float* t_k,
                  int64_t n, const int64_t* slots)
{
    float kt[HEAD_DIM];
    uint8_t codes[HEAD_DIM];
    for (int64_t i = 0; i < n; ++i) {
        int64_t slot = slots[i];
        if (slot < 0) continue;
        int64_t page = slot / PAGE_TOKENS;
        int o = (int)(slot % PAGE_TOKENS);
        if (page >= num_pages) return -1;
        for (int h = 0; h < kv_heads; ++h) {
            const float* kr = k + (i * kv_heads + h) * HEAD_DIM;
            const float* vr = v + (i * kv_heads + h) * HEAD_DIM;
            float lo, hi; uint16_t s16, z16;

            /* keys: k' = k . T_K after RoPE, then quantize k' */
            if (t_k) {
                for (int j = 0; j < HEAD_DIM; ++j) {
                    double acc = 0.0;
                    for (int c = 0; c < HEAD_DIM; ++c)
                        acc += (double)kr[c] * (double)t_k[((int64_t)h * HEAD_DIM + c) * HEAD_DIM + j];
                    kt[j] = (float)acc;
                }
            } else {
                memcpy(kt, kr, sizeof kt);
            }
            if (quant_k == ORACLE_RMS) oracle_clip_rms(kt, HEAD_DIM, alpha_k, &lo, &hi);
            else oracle_clip_percentile(kt, HEAD_DIM, p_lo, p_hi, &lo, &hi);
            oracle_quantize_group(kt, HEAD_DIM, bits_k, lo, hi, codes, &s16, &z16);
            oracle_pack_token(block_at(k_pool, page, h, kv_heads, bits_k), 0, bits_k, o, codes, s16, z16);

            /* values arrive already in the folded (transformed) basis: no transform here */
            if (quant_v == ORACLE_RMS) oracle_clip_rms(vr, HEAD_DIM, alpha_v, &lo, &hi);
            else oracle_clip_percentile(vr, HEAD_DIM, p_lo, p_hi, &lo, &hi);
            oracle_quantize_group(vr, HEAD_DIM, bits_v, lo, hi, codes, &s16, &z16);
            oracle_pack_token(block_at(v_pool, page, h, kv_heads, bits_v), 1, bits_v, o, codes, s16, z16);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O6  dequantize: x^ = fma(code, scale, zero) in fp32.                       */
/* out: [n][kv_heads][128]; a negative slot leaves its rows untouched.        */
/* ------------------------------------------------------------------------- */
void oracle_dequant(const uint8_t* pool, int which, int kv_heads, int bits,
                    const int64_t* slots, int64_t n, float* out)
{
    uint8_t codes[HEAD_DIM];
    for (int64_t i = 0; i < n; ++i) {
        if (slots[i] < 0) continue;
        int64_t page = slots[i] / PAGE_TOKENS;
        int o = (int)(slots[i] % PAGE_TOKENS);
        for (int h = 0; h < kv_heads; ++h) {
            uint16_t s16, z16;
            oracle_unpack_token(block_at((uint8_t*)pool, page, h, kv_heads, bits), which, bits, o,
                                codes, &s16, &z16);
            float sf = oracle_f16_to_f32(s16), zf = oracle_f16_to_f32(z16);
            float* orow = out + (i * kv_heads + h) * HEAD_DIM;
            for (int c = 0; c < HEAD_DIM; ++c) orow[c] = fmaf((float)codes[c], sf, zf);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* O7  decode attention over the quantized cache, all in fp64.                */
/*   q' = q . T_K^{-T}                     ([W] §4.2 query-side compensation) */
/*   s_t = sm_scale * q' . k^_t            (k^ dequantized, transformed basis) */
/*   p = softmax(s) (two passes: max, then normalised exponentials)           */
/*   o = sum_t p_t v^_t                    (transformed value basis, App. C.5) */
/* Query head hq reads KV head hq / (heads_q / kv_heads) ([W] §4.1).           */
/* Token t of sequence b is slot block_table[b][t/64]*64 + t%64.              */
/* An empty sequence gives o = 0 and lse = -inf.                             */
/* q: [batch][heads_q][128]; t_inv_t: [kv_heads][128][128] or NULL;          */
/* out: [batch][heads_q][128]; lse (optional): [batch][heads_q], natural log  */
/* of sum_t exp(s_t).                                                        */
/* ------------------------------------------------------------------------- */
void oracle_decode_attention(const uint8_t* k_pool, const uint8_t* v_pool, int kv_heads,
                             int bits_k, int bits_v, const float* q, int batch, int heads_q,
                             const float* t_inv_t, const int32_t* block_table, int max_pages,
                             const int32_t* seq_lens, double sm_scale, double* out, double* lse)
{
    int group = heads_q / kv_heads;
    uint8_t codes[HEAD_DIM];
    for (int b = 0; b < batch; ++b) {
        int n = seq_lens[b];
        double* kd = (double*)malloc(((size_t)n + 1) * HEAD_DIM * sizeof(double));
        double* vd = (double*)malloc(((size_t)n + 1) * HEAD_DIM * sizeof(double));
        double* s = (double*)malloc(((size_t)n + 1) * sizeof(double));
        for (int h = 0; h < kv_heads; ++h) {
            for (int t = 0; t < n; ++t) {
                int64_t page = block_table[(int64_t)b * max_pages + t / PAGE_TOKENS];
                int o = t % PAGE_TOKENS;
                uint16_t s16, z16;
                oracle_unpack_token(block_at((uint8_t*)k_pool, page, h, kv_heads, bits_k), 0, bits_k, o,
                                    codes, &s16, &z16);
                float sf = oracle_f16_to_f32(s16), zf = oracle_f16_to_f32(z16);
                for (int c = 0; c < HEAD_DIM; ++c) kd[(int64_t)t * HEAD_DIM + c] = fmaf((float)codes[c], sf, zf);
                oracle_unpack_token(block_at((uint8_t*)v_pool, page, h, kv_heads, bits_v), 1, bits_v, o,
                                    codes, &s16, &z16);
                sf = oracle_f16_to_f32(s16); zf = oracle_f16_to_f32(z16);
                for (int c = 0; c < HEAD_DIM; ++c) vd[(int64_t)t * HEAD_DIM + c] = fmaf((float)codes[c], sf, zf);
            }
            for (int g = 0; g < group; ++g) {
                int hq = h * group + g;
                const float* qr = q + ((int64_t)b * heads_q + hq) * HEAD_DIM;
                double qp[HEAD_DIM];
                for (int j = 0; j < HEAD_DIM; ++j) {
                    if (!t_inv_t) { qp[j] = qr[j]; continue; }
                    double acc = 0.0;
                    for (int c = 0; c < HEAD_DIM; ++c)
                        acc += (double)qr[c] * (double)t_inv_t[((int64_t)h * HEAD_DIM + c) * HEAD_DIM + j];
                    qp[j] = acc;
                }
                double* o = out + ((int64_t)b * heads_q + hq) * HEAD_DIM;
                for (int j = 0; j < HEAD_DIM; ++j) o[j] = 0.0;
                if (n == 0) { if (lse) lse[(int64_t)b * heads_q + hq] = -INFINITY; continue; }
                double m = -INFINITY;
                for (int t = 0; t < n; ++t) {
                    double acc = 0.0;
                    for (int c = 0; c < HEAD_DIM; ++c) acc += qp[c] * kd[(int64_t)t * HEAD_DIM + c];
                    s[t] = sm_scale * acc;
                    if (s[t] > m) m = s[t];
                }
                double l = 0.0;
                for (int t = 0; t < n; ++t) { s[t] = exp(s[t] - m); l += s[t]; }
                for (int t = 0; t < n; ++t) {
                    double p = s[t] / l;
                    for (int j = 0; j < HEAD_DIM; ++j) o[j] += p * vd[(int64_t)t * HEAD_DIM + j];
                }
                if (lse) lse[(int64_t)b * heads_q + hq] = m + log(l);
            }
        }
        free(kd); free(vd); free(s);
    }
}

/* ------------------------------------------------------------------------- */
/* Full-precision cache windows ([W] §4.4).                                  */
/* The first `sink` positions and the newest `keep` positions of a sequence  */
/* stay in full precision.  A position from `sink` on that has at least      */
/* `keep` newer positions is eligible; eligible positions are quantized, the */
/* oldest first, in batches of `flush` whenever at least `flush` of them are */
/* waiting.  New positions are appended (and read by that step's attention)  */
/* in full precision before the batches that became eligible are quantized.  */
/*                                                                           */
/* Reading taken: the quantized positions of a sequence are stored in the    */
/* paged cache at index j = position - sink (page block_table[b][j/64]).     */
/* ------------------------------------------------------------------------- */

/* Number of quantized positions after a sequence has grown, one position at  */
/* a time, to `length` positions and every waiting batch has been quantized.  */
int64_t oracle_window_quantized(int64_t length, int sink, int keep, int flush)
{
    int64_t quantized_end = sink;             /* positions [sink, quantized_end) are quantized */
    for (int64_t x = 1; x <= length; ++x) {  /* position x-1 arrives */
        /* eligible and not yet quantized: [quantized_end, x - keep) */
        while (x - keep - quantized_end >= flush) quantized_end += flush;
    }
    return quantized_end - sink;
}

/* Decode attention over a windowed cache: one exact two-pass softmax over    */
/* all seq_lens[b] positions of sequence b, where                             */
/*   quantized positions p (sink <= p < sink + Q) read key k'_j and value v_j */
/*     dequantized from the paged cache at j = p - sink and use the          */
/*     compensated query q' = q T^-T (as oracle_decode_attention);            */
/*   every other position reads its full-precision key and value from       */
/*     k_fp / v_fp ([batch][fp_len][kv_heads][128], position-major) with the  */
/*     plain query q (no transform on either side).                           */
/* Q = oracle_window_quantized(seq_lens[b] - pending): `pending` positions    */
/* were appended since the last quantization (1 for a decode step, whose     */
/* attention runs before its flush; 0 for a read after the flush).           */
/* out: [batch][heads_q][128] fp64; lse (optional) natural log of sum exp(s). */
/* ------------------------------------------------------------------------- */
void oracle_window_attention(const uint8_t* k_pool, const uint8_t* v_pool, int kv_heads,
                             int bits_k, int bits_v, const float* q, int batch, int heads_q,
                             const float* t_inv_t, const int32_t* block_table, int max_pages,
                             const int32_t* seq_lens, int pending, int sink, int keep, int flush,
                             const float* k_fp, const float* v_fp, int64_t fp_len,
                             double sm_scale, double* out, double* lse)
{
    int group = heads_q / kv_heads;
    uint8_t codes[HEAD_DIM];
    for (int b = 0; b < batch; ++b) {
        int64_t n = seq_lens[b];
        int64_t x = n - pending > 0 ? n - pending : 0;
        int64_t nq = oracle_window_quantized(x, sink, keep, flush);
        double* kd = (double*)malloc(((size_t)n + 1) * HEAD_DIM * sizeof(double));
        double* vd = (double*)malloc(((size_t)n + 1) * HEAD_DIM * sizeof(double));
        int* quantized = (int*)malloc(((size_t)n + 1) * sizeof(int));
        double* s = (double*)malloc(((size_t)n + 1) * sizeof(double));
        for (int h = 0; h < kv_heads; ++h) {
            for (int64_t t = 0; t < n; ++t) {
                quantized[t] = t >= sink && t < sink + nq;
                if (quantized[t]) {
                    int64_t j = t - sink;
                    int64_t page = block_table[(int64_t)b * max_pages + j / PAGE_TOKENS];
                    int o = (int)(j % PAGE_TOKENS);
                    uint16_t s16, z16;
                    oracle_unpack_token(block_at((uint8_t*)k_pool, page, h, kv_heads, bits_k), 0, bits_k, o,
                                        codes, &s16, &z16);
                    float sf = oracle_f16_to_f32(s16), zf = oracle_f16_to_f32(z16);
                    for (int c = 0; c < HEAD_DIM; ++c) kd[t * HEAD_DIM + c] = fmaf((float)codes[c], sf, zf);
                    oracle_unpack_token(block_at((uint8_t*)v_pool, page, h, kv_heads, bits_v), 1, bits_v, o,
                                        codes, &s16, &z16);
                    sf = oracle_f16_to_f32(s16); zf = oracle_f16_to_f32(z16);
                    for (int c = 0; c < HEAD_DIM; ++c) vd[t * HEAD_DIM + c] = fmaf((float)codes[c], sf, zf);
                } else {
                    const float* kr = k_fp + (((int64_t)b * fp_len + t) * kv_heads + h) * HEAD_DIM;
                    const float* vr = v_fp + (((int64_t)b * fp_len + t) * kv_heads + h) * HEAD_DIM;
                    for (int c = 0; c < HEAD_DIM; ++c) { kd[t * HEAD_DIM + c] = kr[c]; vd[t * HEAD_DIM + c] = vr[c]; }
                }
            }
            for (int g = 0; g < group; ++g) {
                int hq = h * group + g;
                const float* qr = q + ((int64_t)b * heads_q + hq) * HEAD_DIM;
                double qp[HEAD_DIM];
                for (int j = 0; j < HEAD_DIM; ++j) {
                    if (!t_inv_t) { qp[j] = qr[j]; continue; }
                    double acc = 0.0;
                    for (int c = 0; c < HEAD_DIM; ++c)
                        acc += (double)qr[c] * (double)t_inv_t[((int64_t)h * HEAD_DIM + c) * HEAD_DIM + j];
                    qp[j] = acc;
                }
                double* o = out + ((int64_t)b * heads_q + hq) * HEAD_DIM;
                for (int j = 0; j < HEAD_DIM; ++j) o[j] = 0.0;
                if (n == 0) { if (lse) lse[(int64_t)b * heads_q + hq] = -INFINITY; continue; }
                double m = -INFINITY;
                for (int64_t t = 0; t < n; ++t) {
                    double acc = 0.0;
                    for (int c = 0; c < HEAD_DIM; ++c)
                        acc += (quantized[t] ? qp[c] : (double)qr[c]) * kd[t * HEAD_DIM + c];
                    s[t] = sm_scale * acc;
                    if (s[t] > m) m = s[t];
                }
                double l = 0.0;
                for (int64_t t = 0; t < n; ++t) { s[t] = exp(s[t] - m); l += s[t]; }
                for (int64_t t = 0; t < n; ++t) {
                    double p = s[t] / l;
                    for (int j = 0; j < HEAD_DIM; ++j) o[j] += p * vd[t * HEAD_DIM + j];
                }
                if (lse) lse[(int64_t)b * heads_q + hq] = m + log(l);
            }
        }
        free(kd); free(vd); free(quantized); free(s);
    }
}

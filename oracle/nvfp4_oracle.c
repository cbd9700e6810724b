/*
 * CPU oracle for the NVFP4 quantized-linear hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, deliberately
 * unoptimised restatement of what the method computes.  It exists so that the
 * HIP library can be checked against it.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product
 * path never does.  It shares no code, header, table or constant generator
 * with the HIP sources.
 *
 * Sources (the pages this follows):
 *  [VZ]  "4bit.vizuara.ai" tutorial: section 3-4 (E2M1 / E4M3 formats),
 *        section 5-6 (block scales, the single rounding function, nvfp4()),
 *        section 9 (stochastic rounding), section 13 (quantize kernel: the
 *        block-scale code is never below 1).
 *  [NV]  "Pretraining Large Language Models with NVFP4" summary, section
 *        "NVFP4 Format and Quantization Procedure" (steps 1-5: tensor scale,
 *        block decode scale, E4M3 RNE, encode scale, element quantization,
 *        block-scaled dot product), "Random Hadamard Transforms",
 *        "Two-Dimensional Weight Scaling", "Stochastic Rounding".
 *  [TML] "End-to-End 4-Bit Training" (translation): E4M3 widget, value =
 *        FP4 x FP8 x FP32 reconstruction.
 *  [AIC] "FP4 Training on Blackwell": E2M1 encoding table, power-of-two
 *        scale 2^ceil(log2(amax/elem_max)), stochastic rounding.
 *  Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *        Easy as 1, 2, 3", SC'11 (the generator is not on the pages; it is
 *        the counter-based generator both sides implement independently).
 *  [E2E] "End-to-End 4-Bit Training", quantized communication: 32-point
 *        RHT, then block-scaled S2F6 (int8 / 64, one E8M0 scale per 32);
 *        [VZ] section 11 (the combine wire format, dequantize + sum on
 *        receipt, then the inverse rotation).
 *  [FTB] "FP4 Training on Blackwell", "The scaling math, worked": MXFP4.
 *  GELU: Hendrycks and Gimpel, "Gaussian Error Linear Units", tanh form; exp
 *        by Cody-Waite range reduction and a Taylor polynomial (neither is on
 *        the pages; both sides implement the same FP32 steps independently so
 *        that the fused GELU + quantize of [VZ] section 13 is reproducible).
 *
 * Readings where the pages are silent or disagree are listed in the
 * design notes; the ones that change arithmetic are repeated inline below.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 *        -fopenmp (OpenMP only splits independent rows across threads).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <float.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats ([VZ] sec 3-4, sec 6; [AIC] "The E2M1 format")             */
/* ------------------------------------------------------------------------ */

/* A format for the single rounding function of [VZ] sec 6: mantissa bits,
 * smallest and largest binade exponent, largest magnitude. */
typedef struct { int mbits, emin, emax; float vmax; } orc_fmt;

static const orc_fmt FMT_E2M1 = {1, 0, 2, 6.0f};
static const orc_fmt FMT_E4M3 = {3, -6, 8, 448.0f};

enum { ORC_E2M1 = 0, ORC_E4M3 = 1 };
enum { ORC_RTN = 0, ORC_SR = 1 };

/* E2M1 nibble s|ee|m: exponent field 0 is subnormal (0.5*m), otherwise
 * 2^(e-1) * (1 + m/2).  Bit 3 is the sign.  ([AIC] E2M1 table, [VZ] sec 3.) */
double orc_e2m1_value(uint32_t code)
{
    uint32_t e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

/* E4M3 byte s|eeee|mmm, bias 7: exponent field 0 is subnormal m*2^-9,
 * otherwise 2^(e-7) * (1 + m/8).  0x7F / 0xFF are NaN (never produced here;
 * returned as NaN).  ([VZ] sec 4: max 448, min 2^-9; [TML] E4M3 widget.) */
double orc_e4m3_value(uint32_t byte)
{
    uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
    if (e == 15u && m == 7u) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return (byte & 0x80u) ? -mag : mag;
}

/* E8M0 byte b -> 2^(b-127) ([AIC] "MXFP4 ... 2^(s-127)"). */
double orc_e8m0_value(uint32_t byte) { return ldexp(1.0, (int)byte - 127); }

/* The single rounding function of [VZ] sec 6, in FP32:
 *   a = |v|; frexp gives a = m*2^ex with m in [0.5,1); the binade is
 *   e = clamp(ex-1, emin, emax); step = 2^(e-mbits); t = a/step;
 *   RTN: q = round-half-even(t)   (torch.round is half-to-even)
 *   SR : q = floor(t + u)         (u uniform in (0,1); the sum is exact:
 *                                  t and u are summed in FP64, where both
 *                                  are exact and so is their sum)
 *   result = copysign(min(q*step, vmax), v).
 * t = a/step is a power-of-two scaling, done with ldexpf (exact). */
float orc_round(float v, int fmt_id, int mode, float u)
{
    const orc_fmt f = (fmt_id == ORC_E2M1) ? FMT_E2M1 : FMT_E4M3;
    float a = fabsf(v);
    int ex = 0;
    (void)frexpf(a, &ex);              /* a == 0 gives ex == 0 */
    int e = ex - 1;
    if (e < f.emin) e = f.emin;
    if (e > f.emax) e = f.emax;
    float t = ldexpf(a, f.mbits - e);
    float q;
    if (mode == ORC_RTN) {
        q = rintf(t);                  /* default rounding mode: half to even */
    } else {
        /* t has 24 significant bits and u 17 fractional bits, so the FP64
         * sum is exact: the decision is floor of the true t + u. */
        q = (float)floor((double)t + (double)u);
    }
    float r = ldexpf(q, e - f.mbits);
    if (r > f.vmax) r = f.vmax;
    return copysignf(r, v);
}

/* Grid value -> E2M1 nibble, by looking the magnitude up in the decode table. */
uint32_t orc_e2m1_code(float g)
{
    uint32_t sign = signbit(g) ? 8u : 0u;
    double a = fabs((double)g);
    for (uint32_t c = 0; c < 8; ++c)
        if (orc_e2m1_value(c) == a) return sign | c;
    return 0xFFu;                      /* not on the grid: caller bug */
}

/* Grid value -> E4M3 byte: inverse of orc_e4m3_value. */
uint32_t orc_e4m3_code(float g)
{
    uint32_t sign = signbit(g) ? 0x80u : 0u;
    double a = fabs((double)g);
    if (a < ldexp(1.0, -6)) {          /* subnormal: a = m * 2^-9 */
        double m = ldexp(a, 9);
        return sign | (uint32_t)m;
    }
    int ex = 0;
    double mant = frexp(a, &ex);       /* a = mant * 2^ex, mant in [0.5,1) */
    int E = ex - 1 + 7;
    uint32_t M = (uint32_t)((mant * 2.0 - 1.0) * 8.0);
    return sign | ((uint32_t)E << 3) | M;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11)                                      */
/* ------------------------------------------------------------------------ */

/* One Philox-4x32 round: two 32x32->64 multiplies by the round constants,
 * the high halves XORed with the other two words and the key. */
static void philox_round(uint32_t c[4], const uint32_t k[2])
{
    uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

/* Ten rounds; the key is bumped by the Weyl constants between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k[0] += 0x9E3779B9u; k[1] += 0xBB67AE85u; }
        philox_round(c, k);
    }
    memcpy(out, c, sizeof c);
}

/* The uniform used by stochastic rounding for element `idx` of one output
 * copy.  Keying (a reading, since the pages only say "random"): key = the
 * 64-bit seed, counter = (n_lo, n_hi, stream, 0) with n = idx/8; the 128
 * output bits are eight 16-bit lanes, lane (idx % 8) low half first.
 * u = (h + 1/2) / 2^16 lies strictly inside (0, 1). */
float orc_sr_uniform(uint64_t seed, uint32_t stream, uint64_t idx)
{
    uint64_t n = idx >> 3;
    uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), stream, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    uint32_t w = out[(idx & 7u) >> 1];
    uint32_t h = (idx & 1u) ? (w >> 16) : (w & 0xFFFFu);
    return ((float)h + 0.5f) * (1.0f / 65536.0f);
}

/* ------------------------------------------------------------------------ */
/* 16-point random Hadamard transform ([NV] "Random Hadamard Transforms")    */
/* ------------------------------------------------------------------------ */

/* y <- (y * S) * H16: flip the sign of y[i] where bit i of `signs` is set,
 * then multiply by the natural-order Sylvester Hadamard matrix with entries
 * +-1/4.  The product is formed as four sum/difference stages (pair distance
 * 1, 2, 4, 8) followed by one multiply by 1/4, every step in FP32. */
void orc_rht16(float y[16], uint32_t signs)
{
    for (int i = 0; i < 16; ++i)
        if ((signs >> i) & 1u) y[i] = -y[i];
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                float p = y[i], q = y[i + h];
                y[i] = p + q;
                y[i + h] = p - q;
            }
    for (int i = 0; i < 16; ++i) y[i] = y[i] * 0.25f;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 two-level quantization ([NV] steps 1-4; [VZ] sec 6)                 */
/* ------------------------------------------------------------------------ */

/* Step 1: s_enc = (6 * 448) / amax in FP32.  Readings: amax == 0 gives
 * s_enc = 1; an overflowing quotient is clamped to FLT_MAX. */
float orc_tensor_s_enc(float amax)
{
    if (amax == 0.0f) return 1.0f;
    float s = 2688.0f / amax;
    if (isinf(s)) s = FLT_MAX;
    return s;
}

float orc_amax(const float *x, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > m) m = a;
    }
    return m;
}

/* Steps 2-3: block decode scale amax_b/6, times s_enc, rounded to E4M3
 * (round half to even, saturating at 448).  Reading from [VZ] sec 13: a
 * code of 0 is replaced by 1 (2^-9), so the encode scale stays finite. */
uint32_t orc_block_scale_code(float amax_b, float s_enc)
{
    float t = (amax_b / 6.0f) * s_enc;
    float g = orc_round(t, ORC_E4M3, ORC_RTN, 0.0f);
    uint32_t code = orc_e4m3_code(g);
    if (code == 0u) code = 1u;
    return code;
}

/* Quantize a row-major FP32 matrix x[R][C] to NVFP4 with blocks of 16 along
 * C (1x16), or 16x16 tiles when tile2d != 0.
 *   codes : R * C/2 bytes, element 2j of a row in the low nibble of byte j
 *   scales: R * C/16 (1x16) or R/16 * C/16 (16x16) E4M3 bytes, row-major
 * s_enc is the tensor encode scale.  For SR, element (i, j) draws its
 * uniform at index i*C + j of this copy. */
void orc_nvfp4_encode(const float *x, int64_t R, int64_t C, int tile2d, float s_enc,
                      int mode, uint64_t seed, uint32_t stream,
                      uint8_t *codes, uint8_t *scales)
{
    const float s_dec = 1.0f / s_enc;
    const int64_t nb = C / 16;
    const int64_t br = tile2d ? 16 : 1;          /* rows per scale block */
#pragma omp parallel for schedule(static)
    for (int64_t rb = 0; rb < R / br; ++rb) {
        for (int64_t kb = 0; kb < nb; ++kb) {
            /* Step 2: block amax over the 16 (or 256) values. */
            float amax_b = 0.0f;
            for (int64_t i = rb * br; i < (rb + 1) * br; ++i)
                for (int64_t j = kb * 16; j < kb * 16 + 16; ++j) {
                    float a = fabsf(x[i * C + j]);
                    if (a > amax_b) amax_b = a;
                }
            /* Step 3: E4M3 block scale. */
            uint32_t sc = orc_block_scale_code(amax_b, s_enc);
            scales[rb * nb + kb] = (uint8_t)sc;
            /* Step 3b: s_enc_b = 1 / (fp32(e4m3) * s_dec). */
            float sdec_b = (float)orc_e4m3_value(sc);
            float prod = sdec_b * s_dec;
            float s_enc_b = 1.0f / prod;
            /* Step 4: element quantization x * s_enc_b onto E2M1. */
            for (int64_t i = rb * br; i < (rb + 1) * br; ++i)
                for (int64_t j = kb * 16; j < kb * 16 + 16; ++j) {
                    float v = x[i * C + j] * s_enc_b;
                    float u = (mode == ORC_SR)
                                  ? orc_sr_uniform(seed, stream, (uint64_t)(i * C + j))
                                  : 0.0f;
                    float g = orc_round(v, ORC_E2M1, mode, u);
                    uint32_t c = orc_e2m1_code(g);
                    uint8_t *byte = &codes[i * (C / 2) + j / 2];
                    if ((j & 1) == 0) *byte = (uint8_t)((*byte & 0xF0u) | c);
                    else              *byte = (uint8_t)((*byte & 0x0Fu) | (c << 4));
                }
        }
    }
}

/* BF16 bit patterns -> FP32 (exact widening). */
void orc_bf16_to_f32(const uint16_t *src, int64_t R, int64_t C, int64_t ld, float *dst)
{
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            uint32_t b = (uint32_t)src[i * ld + j] << 16;
            float f;
            memcpy(&f, &b, 4);
            dst[i * C + j] = f;
        }
}

void orc_transpose_f32(const float *src, int64_t R, int64_t C, float *dst)
{
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) dst[j * R + i] = src[i * C + j];
}

/* RHT over consecutive 16-chunks of every row of x[R][C] (in place). */
void orc_rht_rows(float *x, int64_t R, int64_t C, uint32_t signs)
{
    for (int64_t i = 0; i < R; ++i)
        for (int64_t g = 0; g < C / 16; ++g) orc_rht16(&x[i * C + g * 16], signs);
}

/* One complete NVFP4 copy of a BF16 matrix src[R][C] (leading dim ld).
 * transpose != 0 produces the copy of src^T (shape C x R, blocks along R),
 * rht != 0 applies the 16-point RHT to the 16-chunks of that copy's rows
 * before the amax.  Returns s_dec (= 1/s_enc) and writes codes/scales. */
float orc_nvfp4_quantize(const uint16_t *src, int64_t R, int64_t C, int64_t ld,
                         int transpose, int tile2d, int rht, uint32_t signs,
                         int mode, uint64_t seed, uint32_t stream,
                         uint8_t *codes, uint8_t *scales)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_bf16_to_f32(src, R, C, ld, x);
    int64_t r = R, c = C;
    if (transpose) {
        float *t = (float *)malloc(sizeof(float) * (size_t)(R * C));
        orc_transpose_f32(x, R, C, t);
        free(x);
        x = t; r = C; c = R;
    }
    if (rht) orc_rht_rows(x, r, c, signs);
    float s_enc = orc_tensor_s_enc(orc_amax(x, r * c));
    orc_nvfp4_encode(x, r, c, tile2d, s_enc, mode, seed, stream, codes, scales);
    free(x);
    return 1.0f / s_enc;
}

/* Dequantize an NVFP4 matrix in FP32 as ([TML]) code x E4M3 x FP32, left to
 * right: the first product is exact, the second is one FP32 multiply. */
void orc_nvfp4_dequant_f32(const uint8_t *codes, const uint8_t *scales, float s_dec,
                           int64_t R, int64_t C, int tile2d, float *out)
{
    const int64_t nb = C / 16;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            uint32_t byte = codes[i * (C / 2) + j / 2];
            uint32_t c = (j & 1) ? (byte >> 4) : (byte & 0xFu);
            uint32_t sc = scales[(tile2d ? i / 16 : i) * nb + j / 16];
            float v = (float)orc_e2m1_value(c) * (float)orc_e4m3_value(sc);
            out[i * C + j] = v * s_dec;
        }
}

/* The same values in FP64 (code x scale x s_dec is exact in FP64). */
/* ------------------------------------------------------------------------ */
/* Activation copy with a per-token outer scale and Four Over Six            */
/* ([VZ] sec 11, the article's smaller choices; [TML] recipe details)        */
/* ------------------------------------------------------------------------ */

/* Block scale that puts the block's largest magnitude on `top` (6 is the
 * standard choice, 4 the alternative of Four Over Six): E4M3 of
 * (amax_b / top) * s_enc, round half to even, saturating at 448, never
 * below code 1 (as orc_block_scale_code). */
static uint32_t orc_block_scale_code_top(float amax_b, float s_enc, float top)
{
    float t = (amax_b / top) * s_enc;
    float g = orc_round(t, ORC_E4M3, ORC_RTN, 0.0f);
    uint32_t code = orc_e4m3_code(g);
    if (code == 0u) code = 1u;
    return code;
}

/* Encode one block of 16 with block scale code sc (round to nearest):
 * nibbles to q[16]; returns the block's squared error against x, in FP32,
 * with d = x - (g * S) * s_dec, e = d * d, summed in order over elements
 * 0..7 and over 8..15, then low + high (the order is part of the reading:
 * the decision between two encodings is taken on this FP32 value). */
static float orc_encode_block_err(const float *x, float s_dec, uint32_t sc, uint32_t q[16])
{
    const float S = (float)orc_e4m3_value(sc);
    const float s_enc_b = 1.0f / (S * s_dec);
    float half[2] = {0.0f, 0.0f};
    for (int i = 0; i < 16; ++i) {
        float g = orc_round(x[i] * s_enc_b, ORC_E2M1, ORC_RTN, 0.0f);
        q[i] = orc_e2m1_code(g);
        volatile float deq = (g * S) * s_dec;     /* g * S is exact */
        volatile float d = x[i] - deq;
        volatile float e = d * d;
        half[i / 8] = half[i / 8] + e;
    }
    return half[0] + half[1];
}

/* exp in FP32 by Cody-Waite range reduction and a Taylor polynomial
 * (W. J. Cody and W. Waite, Software Manual for the Elementary Functions,
 * 1980): k = rint(v * log2 e); r = (v - k * ln2_hi) - k * ln2_lo, with ln2
 * split so that k * ln2_hi is exact; exp(v) = 2^k * P(r), P the degree-7
 * Taylor polynomial of exp evaluated by Horner's rule.  Every step is one
 * FP32 operation in this order; v >= 88.5 gives +inf and v <= -87 gives 0
 * (so no result is subnormal). */
float orc_exp_f32(float v)
{
    if (v >= 88.5f) return INFINITY;
    if (v <= -87.0f) return 0.0f;
    const float log2e = 1.44269502162933349609375f;
    const float ln2_hi = 0.693145751953125f;           /* 0x3F317200 */
    const float ln2_lo = 1.428606765330187045e-06f;    /* 0x35BFBE8E */
    volatile float t = v * log2e;
    const float k = rintf(t);
    volatile float a = k * ln2_hi;
    volatile float r = v - a;
    volatile float b = k * ln2_lo;
    r = r - b;
    const float c[8] = {1.0f, 1.0f, 0.5f, 1.0f / 6.0f, 1.0f / 24.0f, 1.0f / 120.0f,
                        1.0f / 720.0f, 1.0f / 5040.0f};
    volatile float p = c[7];
    for (int i = 6; i >= 0; --i) {
        volatile float q = p * r;
        p = q + c[i];
    }
    return ldexpf(p, (int)k);
}

/* GELU in its tanh form (Hendrycks and Gimpel, "Gaussian Error Linear Units",
 * 2016): 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), with
 * tanh(u) = 1 - 2 / (exp(2u) + 1) and exp as orc_exp_f32; FP32 steps in the
 * order written, no fused operations.  The fused GELU + quantize of the
 * pages' kernel (4bit.vizuara.ai, section 13) leaves the GELU output in FP32
 * and quantizes it directly. */
float orc_gelu_f32(float x)
{
    const float c0 = 0.797884583473205566f;            /* sqrt(2/pi) in FP32 */
    const float c1 = 0.044715f;
    volatile float x2 = x * x;
    volatile float x3 = x2 * x;
    volatile float w = c1 * x3;
    volatile float z = x + w;
    volatile float u = c0 * z;
    volatile float e = orc_exp_f32(2.0f * u);
    volatile float den = e + 1.0f;
    volatile float q = 2.0f / den;
    volatile float th = 1.0f - q;
    volatile float h = 0.5f * x;
    volatile float g = 1.0f + th;
    return h * g;
}

void orc_gelu_n(const float *x, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_gelu_f32(x[i]);
}

void orc_exp_n(const float *x, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_f32(x[i]);
}

/* One row-wise NVFP4 copy of src[R][C] (1x16 blocks, round to nearest) with
 *   per_token != 0: outer scale per row, s_enc_i = 2688 / amax(row i)
 *                   (1 for an all-zero row), s_dec[i] = 1 / s_enc_i;
 *   per_token == 0: one tensor scale, s_dec[0];
 *   four_six != 0 : each block keeps whichever of its top-6 and top-4
 *                   encodings has the smaller squared error (top-6 on ties);
 *                   the chosen scale is the block's stored E4M3 scale;
 *   gelu != 0     : the quantized values are orc_gelu_f32 of the inputs.
 * s_dec receives R values (per_token) or 1. */
void orc_nvfp4_quantize_act(const uint16_t *src, int64_t R, int64_t C, int64_t ld,
                            int per_token, int four_six, int gelu, uint8_t *codes,
                            uint8_t *scales, float *s_dec)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_bf16_to_f32(src, R, C, ld, x);
    if (gelu)
        for (int64_t i = 0; i < R * C; ++i) x[i] = orc_gelu_f32(x[i]);
    float s_enc_t = orc_tensor_s_enc(orc_amax(x, R * C));
    if (!per_token) s_dec[0] = 1.0f / s_enc_t;
    const int64_t nb = C / 16;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i) {
        const float *xr = &x[i * C];
        const float s_enc = per_token ? orc_tensor_s_enc(orc_amax(xr, C)) : s_enc_t;
        const float sd = 1.0f / s_enc;
        if (per_token) s_dec[i] = sd;
        for (int64_t kb = 0; kb < nb; ++kb) {
            const float *xb = &xr[kb * 16];
            const float amax_b = orc_amax(xb, 16);
            uint32_t q6[16], q4[16];
            const uint32_t sc6 = orc_block_scale_code_top(amax_b, s_enc, 6.0f);
            const float e6 = orc_encode_block_err(xb, sd, sc6, q6);
            uint32_t sc = sc6, *q = q6;
            if (four_six) {
                const uint32_t sc4 = orc_block_scale_code_top(amax_b, s_enc, 4.0f);
                const float e4 = orc_encode_block_err(xb, sd, sc4, q4);
                if (e4 < e6) {
                    sc = sc4;
                    q = q4;
                }
            }
            scales[i * nb + kb] = (uint8_t)sc;
            for (int j = 0; j < 16; j += 2)
                codes[i * (C / 2) + kb * 8 + j / 2] = (uint8_t)(q[j] | (q[j + 1] << 4));
        }
    }
    free(x);
}

/* Exact dequantization of a 1x16 NVFP4 copy whose rows carry their own
 * decode scale s_dec[i]: (code * scale) * s_dec[i] in FP64. */
void orc_nvfp4_dequant_rows_f64(const uint8_t *codes, const uint8_t *scales, const float *s_dec,
                                int64_t R, int64_t C, double *out)
{
    const int64_t nb = C / 16;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            uint32_t byte = codes[i * (C / 2) + j / 2];
            uint32_t c = (j & 1) ? (byte >> 4) : (byte & 0xFu);
            out[i * C + j] = orc_e2m1_value(c) * orc_e4m3_value(scales[i * nb + j / 16]) *
                             (double)s_dec[i];
        }
}

void orc_nvfp4_dequant_f64(const uint8_t *codes, const uint8_t *scales, float s_dec,
                           int64_t R, int64_t C, int tile2d, double *out)
{
    const int64_t nb = C / 16;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            uint32_t byte = codes[i * (C / 2) + j / 2];
            uint32_t c = (j & 1) ? (byte >> 4) : (byte & 0xFu);
            uint32_t sc = scales[(tile2d ? i / 16 : i) * nb + j / 16];
            out[i * C + j] = orc_e2m1_value(c) * orc_e4m3_value(sc) * (double)s_dec;
        }
}

/* ------------------------------------------------------------------------ */
/* MXFP8: E4M3 elements, one E8M0 scale per 32 ([VZ] sec 5; [AIC] scale rule) */
/* ------------------------------------------------------------------------ */

/* The power-of-two scale 2^k of a block ([AIC] "scale = 2^ceil(log2(amax /
 * elem_max))"): the smallest integer k with amax <= elem_max * 2^k, decided
 * exactly.  Clamped to [-127, 127]; an all-zero block gives -127 (byte 0).
 * MXFP8 uses elem_max = 448, the E4M3 maximum. */
int orc_e8m0_k_for(float amax, double elem_max)
{
    int k = -127;
    while (k < 127 && (double)amax > ldexp(elem_max, k)) ++k;
    return k;
}

int orc_e8m0_k(float amax) { return orc_e8m0_k_for(amax, 448.0); }

/* Quantize a row-major FP32 matrix x[R][C] to MXFP8 with blocks of 32 along
 * C.  codes: R*C E4M3 bytes; scales: R*C/32 E8M0 bytes (k + 127).  Elements
 * are x * 2^-k rounded to E4M3 (RTN or SR; SR index i*C + j). */
void orc_mxfp8_encode(const float *x, int64_t R, int64_t C, int mode, uint64_t seed,
                      uint32_t stream, uint8_t *codes, uint8_t *scales)
{
    const int64_t nb = C / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t b = 0; b < nb; ++b) {
            float amax_b = 0.0f;
            for (int64_t j = b * 32; j < b * 32 + 32; ++j) {
                float a = fabsf(x[i * C + j]);
                if (a > amax_b) amax_b = a;
            }
            int k = orc_e8m0_k(amax_b);
            scales[i * nb + b] = (uint8_t)(k + 127);
            for (int64_t j = b * 32; j < b * 32 + 32; ++j) {
                float v = ldexpf(x[i * C + j], -k);
                float u = (mode == ORC_SR)
                              ? orc_sr_uniform(seed, stream, (uint64_t)(i * C + j))
                              : 0.0f;
                float g = orc_round(v, ORC_E4M3, mode, u);
                codes[i * C + j] = (uint8_t)orc_e4m3_code(g);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Combine wire format: 32-point RHT + block-scaled S2F6 ([E2E] quantized   */
/* communication; [VZ] section 11)                                          */
/* ------------------------------------------------------------------------ */

/* y <- (y * S) * H32 / sqrt(32): flip the sign of y[i] where bit i of
 * `signs` is set, then the natural-order Sylvester Hadamard matrix as five
 * sum/difference stages (pair distance 1, 2, 4, 8, 16), then one multiply
 * by 1/sqrt(32) rounded to FP32; every step in FP32. */
static const float ORC_INV_SQRT32 = 0.17677669529663688f;

void orc_rht32(float y[32], uint32_t signs)
{
    for (int i = 0; i < 32; ++i)
        if ((signs >> i) & 1u) y[i] = -y[i];
    for (int h = 1; h < 32; h <<= 1)
        for (int i = 0; i < 32; ++i)
            if ((i & h) == 0) {
                float p = y[i], q = y[i + h];
                y[i] = p + q;
                y[i + h] = p - q;
            }
    for (int i = 0; i < 32; ++i) y[i] = y[i] * ORC_INV_SQRT32;
}

/* The inverse: H32 / sqrt(32) is its own inverse, so the same stages and
 * multiply come first and the sign flips last. */
void orc_rht32_inv(float y[32], uint32_t signs)
{
    for (int h = 1; h < 32; h <<= 1)
        for (int i = 0; i < 32; ++i)
            if ((i & h) == 0) {
                float p = y[i], q = y[i + h];
                y[i] = p + q;
                y[i + h] = p - q;
            }
    for (int i = 0; i < 32; ++i) y[i] = y[i] * ORC_INV_SQRT32;
    for (int i = 0; i < 32; ++i)
        if ((signs >> i) & 1u) y[i] = -y[i];
}

/* S2F6 copy of x[R][C] (C % 32 == 0), blocks of 32 along the rows: with
 * rht, each block is rotated first; k = the smallest integer (clamped to
 * [-127, 127]) with amax <= (127/64) 2^k, so no value saturates; codes
 * q = rint(y 2^-k 64) (nearest, ties to even) as int8, scale byte k + 127.
 * The value of a code is q / 64 * 2^k. */
void orc_s2f6_encode(const float *x, int64_t R, int64_t C, int rht, uint32_t signs,
                     int8_t *codes, uint8_t *scales)
{
    const int64_t nb = C / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t b = 0; b < nb; ++b) {
            float y[32];
            for (int j = 0; j < 32; ++j) y[j] = x[i * C + b * 32 + j];
            if (rht) orc_rht32(y, signs);
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j)
                if (fabsf(y[j]) > amax) amax = fabsf(y[j]);
            const int k = orc_e8m0_k_for(amax, 127.0 / 64.0);
            scales[i * nb + b] = (uint8_t)(k + 127);
            for (int j = 0; j < 32; ++j) {
                float q = rintf(ldexpf(y[j], 6 - k));
                if (q > 127.0f) q = 127.0f;
                if (q < -128.0f) q = -128.0f;
                codes[i * C + b * 32 + j] = (int8_t)q;
            }
        }
}

void orc_s2f6_quantize(const uint16_t *src, int64_t R, int64_t C, int64_t ld, int rht,
                       uint32_t signs, int8_t *codes, uint8_t *scales)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_bf16_to_f32(src, R, C, ld, x);
    orc_s2f6_encode(x, R, C, rht, signs, codes, scales);
    free(x);
}

/* Receiver side: out[t] = inverse RHT (if rht) of sum_j w[t][j] * deq(row
 * src[t][j]) per block of 32, j = 0 .. K-1 in order (rows with a negative
 * index are skipped; w == NULL means weight 1 and no multiply); every step
 * in FP32: the decoded value q 2^(k-6) is exact, then the product with the
 * weight and each addition round. */
void orc_s2f6_combine(const int8_t *codes, const uint8_t *scales, int64_t C,
                      const int32_t *src, const float *w, int64_t T, int K, int rht,
                      uint32_t signs, float *out)
{
    const int64_t nb = C / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t b = 0; b < nb; ++b) {
            float acc[32];
            for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
            for (int j = 0; j < K; ++j) {
                const int32_t r = src[t * K + j];
                if (r < 0) continue;
                const int k = (int)scales[(int64_t)r * nb + b] - 127;
                for (int i = 0; i < 32; ++i) {
                    float d = ldexpf((float)codes[(int64_t)r * C + b * 32 + i], k - 6);
                    if (w) d = w[t * K + j] * d;
                    acc[i] = acc[i] + d;
                }
            }
            if (rht) orc_rht32_inv(acc, signs);
            for (int i = 0; i < 32; ++i) out[t * C + b * 32 + i] = acc[i];
        }
}

void orc_s2f6_dequant_f64(const int8_t *codes, const uint8_t *scales, int64_t R, int64_t C,
                          double *out)
{
    const int64_t nb = C / 32;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j)
            out[i * C + j] = ldexp((double)codes[i * C + j],
                                   (int)scales[i * nb + j / 32] - 127 - 6);
}

/* ------------------------------------------------------------------------ */
/* MXFP4 ([FTB] "The scaling math, worked")                                  */
/* ------------------------------------------------------------------------ */

/* MXFP4 copy of x[R][C] (C % 32 == 0), blocks of 32 along the rows: scale
 * 2^k with k = ceil(log2(amax / 6)), i.e. the smallest k with amax <= 6 2^k
 * (clamped to [-127, 127]); elements x 2^-k rounded onto the E2M1 grid
 * (nearest even, or stochastic with the element's draw), packed two per
 * byte (even column in the low nibble); scale byte k + 127. */
void orc_mxfp4_encode(const float *x, int64_t R, int64_t C, int mode, uint64_t seed,
                      uint32_t stream, uint8_t *codes, uint8_t *scales)
{
    const int64_t nb = C / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t b = 0; b < nb; ++b) {
            float amax_b = 0.0f;
            for (int64_t j = b * 32; j < b * 32 + 32; ++j)
                if (fabsf(x[i * C + j]) > amax_b) amax_b = fabsf(x[i * C + j]);
            const int k = orc_e8m0_k_for(amax_b, 6.0);
            scales[i * nb + b] = (uint8_t)(k + 127);
            for (int64_t j = b * 32; j < b * 32 + 32; j += 2) {
                uint32_t nib[2];
                for (int e = 0; e < 2; ++e) {
                    const float v = ldexpf(x[i * C + j + e], -k);
                    const float u = (mode == ORC_SR)
                                        ? orc_sr_uniform(seed, stream, (uint64_t)(i * C + j + e))
                                        : 0.0f;
                    nib[e] = orc_e2m1_code(orc_round(v, ORC_E2M1, mode, u));
                }
                codes[(i * C + j) / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
            }
        }
}

void orc_mxfp4_quantize(const uint16_t *src, int64_t R, int64_t C, int64_t ld, int mode,
                        uint64_t seed, uint32_t stream, uint8_t *codes, uint8_t *scales)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_bf16_to_f32(src, R, C, ld, x);
    orc_mxfp4_encode(x, R, C, mode, seed, stream, codes, scales);
    free(x);
}

void orc_mxfp4_dequant_f64(const uint8_t *codes, const uint8_t *scales, int64_t R, int64_t C,
                           double *out)
{
    const int64_t nb = C / 32;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            const uint32_t byte = codes[(i * C + j) / 2];
            const uint32_t nib = (j & 1) ? (byte >> 4) : (byte & 15u);
            out[i * C + j] = orc_e2m1_value(nib) *
                             ldexp(1.0, (int)scales[i * nb + j / 32] - 127);
        }
}

/* Dequantize -> transpose -> requantize to MXFP8 ([VZ] sec 9-10; [TML]
 * "requantization with stochastic rounding"): the NVFP4 matrix src[R][C]
 * becomes the MXFP8 matrix of src^T, shape C x R, blocks of 32 along R. */
void orc_mxfp8_requantize_t(const uint8_t *codes, const uint8_t *scales, float s_dec,
                            int64_t R, int64_t C, int tile2d, int mode, uint64_t seed,
                            uint32_t stream, uint8_t *out_codes, uint8_t *out_scales)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)(R * C));
    float *t = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_nvfp4_dequant_f32(codes, scales, s_dec, R, C, tile2d, x);
    orc_transpose_f32(x, R, C, t);
    orc_mxfp8_encode(t, C, R, mode, seed, stream, out_codes, out_scales);
    free(x);
    free(t);
}

/* MXFP8 copy of a BF16 matrix (blocks of 32 along its rows). */
void orc_mxfp8_quantize(const uint16_t *src, int64_t R, int64_t C, int64_t ld, int mode,
                        uint64_t seed, uint32_t stream, uint8_t *codes, uint8_t *scales)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)(R * C));
    orc_bf16_to_f32(src, R, C, ld, x);
    orc_mxfp8_encode(x, R, C, mode, seed, stream, codes, scales);
    free(x);
}

void orc_mxfp8_dequant_f64(const uint8_t *codes, const uint8_t *scales, int64_t R,
                           int64_t C, double *out)
{
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j)
            out[i * C + j] = orc_e4m3_value(codes[i * C + j]) *
                             orc_e8m0_value(scales[i * (C / 32) + j / 32]);
}

/* ------------------------------------------------------------------------ */
/* GEMM reference ([NV] step 5; [VZ] sec 7): Y = A * B^T over dequantized    */
/* operands, accumulated in FP64 in k order.                                 */
/* ------------------------------------------------------------------------ */

void orc_gemm_f64(const double *A, const double *B, int64_t M, int64_t N, int64_t K,
                  double *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += A[m * K + k] * B[n * K + k];
            Y[m * N + n] = s;
        }
}

/* Selected outputs only: Y[i] = sum_k A[rows[i]][k] * B[cols[i]][k]. */
void orc_gemm_f64_sampled(const double *A, const double *B, int64_t K, const int64_t *rows,
                          const int64_t *cols, int64_t count, double *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += A[rows[i] * K + k] * B[cols[i] * K + k];
        Y[i] = s;
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Element-wise array forms of the helpers above, for the Python wrapper.    */
/* ------------------------------------------------------------------------ */

void orc_round_n(const float *v, const float *u, int64_t n, int fmt_id, int mode, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_round(v[i], fmt_id, mode, u ? u[i] : 0.0f);
}

void orc_e2m1_code_n(const float *g, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_code(g[i]);
}

void orc_e4m3_code_n(const float *g, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_code(g[i]);
}

void orc_sr_uniform_n(uint64_t seed, uint32_t stream, const uint64_t *idx, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_uniform(seed, stream, idx[i]);
}

void orc_rht32_n(float *y, int64_t nchunks, uint32_t signs, int inverse)
{
    for (int64_t i = 0; i < nchunks; ++i) {
        if (inverse) orc_rht32_inv(y + 32 * i, signs);
        else orc_rht32(y + 32 * i, signs);
    }
}

void orc_rht16_n(float *y, int64_t nchunks, uint32_t signs)
{
    for (int64_t i = 0; i < nchunks; ++i) orc_rht16(&y[i * 16], signs);
}

void orc_e8m0_k_n(const float *amax, int64_t n, int32_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e8m0_k(amax[i]);
}

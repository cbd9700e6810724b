// Device-side building blocks of the NVFP4 / MXFP8 kernels (gfx950).
//
// Formats follow 4bit.vizuara.ai (sections 3-6) and "Pretraining LLMs with
// NVFP4" ("NVFP4 Format and Quantization Procedure"):
//   E2M1  s|ee|m, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//   E4M3  s|eeee|mmm, bias 7, max 448, min 2^-9, 0x7F is NaN (never written)
//   E8M0  2^(byte - 127)
// Every FP32 step before a rounding decision is a single IEEE operation
// rounded to nearest even (the library is built with FP contraction off);
// the decisions themselves are made by the gfx950 conversion instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bbs {

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// Two FP32 values -> two BF16 (nearest even, as f32_to_bf16 for finite
// values; one v_cvt_pk_bf16_f32), low half first.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2_t h = __builtin_convertvector(f32x2_v{a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Unbiased binade exponent floor(log2 a) read from the FP32 bits (a >= 0);
// zero and FP32 subnormals give -127, below every clamp used here.
__device__ __forceinline__ int binade(float a) {
    return (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
}

// 2^e as an FP32 constant, for |e| < 127.
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// ---------------------------------------------------------------------------
// Decoders
// ---------------------------------------------------------------------------

// Positive E4M3 code -> value.
__device__ __forceinline__ float e4m3_pos_value(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// E2M1 nibble -> FP32 value.
__device__ __forceinline__ float e2m1_value(uint32_t n) {
    uint32_t e = (n >> 1) & 3u, m = n & 1u;
    uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
    return __uint_as_float(bits | ((n & 8u) << 28));
}

// ---------------------------------------------------------------------------
// Rounding onto the E2M1 / E4M3 grids with the gfx950 conversion
// instructions, always at conversion scale 1.0 (the value is scaled before).
// Measured behaviour these helpers rely on (checked on the device by the
// instruction tests):
//  * round to nearest: ties to the even code, -0 kept, E2M1 saturates at 6;
//    E4M3 is exact up to 448 (inputs above 448 are clamped first here);
//  * stochastic: with r the 32-bit random operand, the first (or only)
//    element rounds as floor(t + (r >> (32 - d)) / 2^d) on the exact t (the
//    magnitude in units of the grid step), d = 22 for E2M1 and 20 for E4M3.
//    With r = (h << 16) | 0x8000 that is floor(t + (h + 1/2) / 2^16): the
//    16-bit uniform h of the stochastic-rounding rule.  The pair form's second
//    element draws from bits overlapping the first one's, so one element is
//    converted per instruction (the other slot gets +0, code 0).
// ---------------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));

// Bytes 0 of four words -> one word (b0 in bits 7:0).
__device__ __forceinline__ uint32_t pack_bytes4(uint32_t b0, uint32_t b1, uint32_t b2,
                                                uint32_t b3) {
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// The conversions below only write part of their destination word; the
// rest comes from their first operand.  The first write into a word passes a
// dead input there (no register needs clearing first), later ones the word
// built so far, until the writes cover it.

// Eight values times s, rounded to nearest, packed little-endian: pair k is
// written into byte k of one word (the four byte writes cover it).
__device__ __forceinline__ uint32_t e2m1_rne8(const float *f, float s) {
    uint32_t w = __float_as_uint(f[0]);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0] * s, f[1] * s, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2] * s, f[3] * s, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4] * s, f[5] * s, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6] * s, f[7] * s, 1.0f, 3);
    return w;
}

// Random operand for a 16-bit uniform held in the low / high half of w.
__device__ __forceinline__ uint32_t sr_word_lo(uint32_t w) { return (w << 16) | 0x8000u; }
__device__ __forceinline__ uint32_t sr_word_hi(uint32_t w) {
    return __builtin_amdgcn_bitop3_b32(w, 0xFFFF0000u, 0x8000u, 0xEA);   // (w & b) | c
}

// Stochastic E2M1 code of one value (nibble in bits 3:0, bits 7:4 zero from
// the +0 in the second slot, upper bytes unspecified: the compiler does not
// carry the first operand of this conversion into its destination).
__device__ __forceinline__ uint32_t e2m1_sr1(float v, uint32_t r) {
    f32x2_t p = {v, 0.0f};
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(__float_as_uint(v), p, r, 1.0f, 0);
}

// Eight values times s, stochastically rounded with the eight 16-bit
// uniforms of one Philox block (value j uses half j & 1 of word j >> 1).
// Byte 0 of (hi << 4) | lo is the code pair, as bits 7:4 of lo are zero.
__device__ __forceinline__ uint32_t e2m1_sr8(const float *f, float s, const uint32_t w[4]) {
    uint32_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = e2m1_sr1(f[2 * i] * s, sr_word_lo(w[i]));
        const uint32_t hi = e2m1_sr1(f[2 * i + 1] * s, sr_word_hi(w[i]));
        b[i] = (hi << 4) | lo;
    }
    return pack_bytes4(b[0], b[1], b[2], b[3]);
}

__device__ __forceinline__ i16x2_t as_i16x2(float f) { return __builtin_bit_cast(i16x2_t, f); }

// E4M3 round-to-nearest-even code of t >= 0 (saturating at 448).
__device__ __forceinline__ uint32_t e4m3_rne_code(float t) {
    t = fminf(t, 448.0f);
    i16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(as_i16x2(t), t, t, 1.0f, false);
    return (uint32_t)r[0] & 0xFFu;
}

// Four values (|y| <= 448) rounded to nearest E4M3, bytes little-endian.
__device__ __forceinline__ uint32_t e4m3_rne4(float y0, float y1, float y2, float y3) {
    i16x2_t w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(as_i16x2(y0), y0, y1, 1.0f, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, y2, y3, 1.0f, true);
    return __builtin_bit_cast(uint32_t, w);
}

// Four values (|y| <= 448) stochastically rounded to E4M3 with random
// operands r0..r3, bytes little-endian (the four byte writes cover the word).
__device__ __forceinline__ uint32_t e4m3_sr4(float y0, float y1, float y2, float y3,
                                             uint32_t r0, uint32_t r1, uint32_t r2,
                                             uint32_t r3) {
    int w = __float_as_int(y0);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y0, r0, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y1, r1, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y2, r2, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y3, r3, 1.0f, 3);
    return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// NVFP4 scales (steps 1-3 of the NVFP4 procedure)
// ---------------------------------------------------------------------------

// s_enc = 2688 / amax (1 when amax == 0, FLT_MAX on overflow).
__device__ __forceinline__ float tensor_s_enc(float amax) {
    if (amax == 0.0f) return 1.0f;
    float s = 2688.0f / amax;
    return (s > 3.40282347e38f) ? 3.40282347e38f : s;
}

// a / 6 rounded to nearest even (a >= 0 finite), as IEEE division gives it:
// q = a * RN(1/6) and one FMA correction, q + RN(1/6) * (a - 6q), whose
// remainder a - 6q is exact.  Over every non-negative finite FP32 a this
// equals the correctly rounded quotient whenever the quotient is normal
// (exhaustive host check); below a = 2^-124 the division itself is taken.
__device__ __forceinline__ float div6(float a) {
    constexpr float kInv6 = 0x1.555556p-3f;             // RN(1/6)
    float q = a * kInv6;
    q = __builtin_fmaf(__builtin_fmaf(-q, 6.0f, a), kInv6, q);
    if (__builtin_amdgcn_ballot_w64(a < 0x1p-124f)) {     // rare: wave-uniform branch
        // (an empty volatile statement keeps the compiler from hoisting the
        // division out of the branch into every call)
        asm volatile("");
        if (a < 0x1p-124f) q = a / 6.0f;
    }
    return q;
}

// Block scale code: E4M3(rne((amax_b / top) * s_enc)), never below code 1.
// top = 6 puts the block's largest magnitude on the top of the E2M1 grid;
// Four Over Six also tries top = 4 (a division by 4 is the multiply by 1/4,
// rounded the same way).
__device__ __forceinline__ uint32_t block_scale_code(float amax_b, float s_enc,
                                                     float top = 6.0f) {
    const float q = top == 4.0f ? amax_b * 0.25f : (top == 6.0f ? div6(amax_b) : amax_b / top);
    const uint32_t c = e4m3_rne_code(q * s_enc);
    return c ? c : 1u;
}

// s_enc_b = 1 / (E4M3(code) * s_dec).
__device__ __forceinline__ float block_enc_scale(uint32_t code, float s_dec) {
    return 1.0f / (__builtin_amdgcn_cvt_scalef32_f32_fp8((int)code, 1.0f, 0) * s_dec);
}

// The encode scales of every positive E4M3 code for one decode scale, into
// an LDS table of 128 floats (entry c = block_enc_scale(c, s_dec), entry 0
// unused).  Threads 0..127 of the workgroup each write one entry; the
// caller synchronises before the first lookup.
__device__ __forceinline__ void enc_scale_table(float *tab, float s_dec) {
    if (threadIdx.x < 128) tab[threadIdx.x] = block_enc_scale(threadIdx.x, s_dec);
}

// MXFP8 block exponent: the smallest k with amax <= 448 * 2^k.  With
// amax = m * 2^E, m in [0.5, 1): k = E - 9 if m <= 0.875 else E - 8; clamped
// to [-127, 127]; amax == 0 gives -127.
__device__ __forceinline__ int e8m0_k(float amax) {
    if (amax == 0.0f) return -127;
    int E;
    float m = frexpf(amax, &E);
    int k = (m <= 0.875f) ? E - 9 : E - 8;
    return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// The same exponent as its E8M0 byte k + 127, from the FP32 bits of amax
// (>= 0, finite): with amax = (1 + f / 2^23) 2^(e - 127), 448 = 1.75 * 2^8,
// k + 127 = e - 8 when f <= 0x600000 and e - 7 above, i.e.
// ((bits + 0x1FFFFF) >> 23) - 8; zero and subnormal amax give a negative
// value, clamped to byte 0 (k = -127).
__device__ __forceinline__ uint32_t e8m0_byte(float amax) {
    const int b = (int)((__float_as_uint(amax) + 0x1FFFFFu) >> 23) - 8;
    return (uint32_t)(b < 0 ? 0 : b);
}

// Conversion scale 2^k of an E8M0 byte (byte >= 1): the FP8 conversions
// divide their input by it exactly before rounding (checked on the device
// against ldexp at scale 1.0).  Byte 0 (2^-127) is not an FP32 normal; its
// blocks are converted at 2^-126 after doubling their values (exact).
__device__ __forceinline__ float e8m0_cvt_scale(uint32_t byte) {
    return __uint_as_float((byte < 1u ? 1u : byte) << 23);
}

// Four values rounded to nearest E4M3 after division by the scale,
// bytes little-endian.
__device__ __forceinline__ uint32_t e4m3_rne4_scaled(float y0, float y1, float y2, float y3,
                                                     float scale) {
    i16x2_t w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(as_i16x2(y0), y0, y1, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, y2, y3, scale, true);
    return __builtin_bit_cast(uint32_t, w);
}

// Four values stochastically rounded to E4M3 after division by the scale.
__device__ __forceinline__ uint32_t e4m3_sr4_scaled(float y0, float y1, float y2, float y3,
                                                    uint32_t r0, uint32_t r1, uint32_t r2,
                                                    uint32_t r3, float scale) {
    int w = __float_as_int(y0);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y0, r0, scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y1, r1, scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y2, r2, scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, y3, r3, scale, 3);
    return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): one 128-bit block per
// counter; a block feeds eight elements with 16 bits each.
// ---------------------------------------------------------------------------

struct u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // full 64-bit products (one v_mad_u64_u32 each); each three-way XOR
        // is one v_bitop3_b32 (truth table 0x96)
        const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// The Philox block of elements 8n .. 8n+7 of one output copy: counter
// (n lo, n hi, stream, 0), key = seed.
__device__ __forceinline__ void sr_block(uint64_t seed, uint32_t stream, uint64_t n,
                                         uint32_t w[4]) {
    const u32x4 o = philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), stream, 0u, (uint32_t)seed,
                                  (uint32_t)(seed >> 32));
    w[0] = o.x;
    w[1] = o.y;
    w[2] = o.z;
    w[3] = o.w;
}

// ---------------------------------------------------------------------------
// 16-point random Hadamard transform: sign flips (bit i of `signs` negates
// y[i], as an exact flip of the sign bit), four sum/difference stages with
// pair distance 1, 2, 4, 8, then one multiply by 1/4 (all FP32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rht16_butterflies(float y[16], uint32_t signs) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        y[i] = __uint_as_float(__float_as_uint(y[i]) ^ (((signs >> i) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                float p = y[i], q = y[i + h];
                y[i] = p + q;
                y[i + h] = p - q;
            }
        }
    }
}

__device__ __forceinline__ void rht16(float y[16], uint32_t signs) {
    rht16_butterflies(y, signs);
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = y[i] * 0.25f;
}

// ---------------------------------------------------------------------------
// GELU in its tanh form (Hendrycks and Gimpel, "Gaussian Error Linear
// Units"): 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), with
// tanh(u) = 1 - 2 / (exp(2u) + 1).  exp by Cody-Waite range reduction:
// k = rint(v log2 e), r = (v - k ln2_hi) - k ln2_lo, where ln2_hi has 15
// significant bits so that k ln2_hi is exact, then the degree-7 Taylor
// polynomial of exp(r) by Horner's rule, times 2^k; v >= 88.5 gives +inf and
// v <= -87 gives 0.  Every step is one FP32 operation rounded to nearest
// even, in the order written, so the result is reproducible bit for bit
// (finite inputs).  Over every finite BF16 input, GELU is non-decreasing for
// x >= 0 and |GELU(x)| < kGeluNegBound for x < 0 (exhaustive tests).
// ---------------------------------------------------------------------------
constexpr float kGeluNegBound = 0.171875f;

__device__ __forceinline__ float exp_cw(float v) {
    const float w = fminf(fmaxf(v, -87.0f), 88.5f);      // keeps k in range
    const float k = __builtin_rintf(w * 1.4426950408889634f);
    float r = w - k * 0.693145751953125f;
    r = r - k * 1.4286068202862268e-06f;
    float p = 1.0f / 5040.0f;
    p = p * r + 1.0f / 720.0f;
    p = p * r + 1.0f / 120.0f;
    p = p * r + 1.0f / 24.0f;
    p = p * r + 1.0f / 6.0f;
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    const float e = __builtin_amdgcn_ldexpf(p, (int)k);
    return v >= 88.5f ? __builtin_inff() : (v <= -87.0f ? 0.0f : e);
}

__device__ __forceinline__ float gelu_tanh(float x) {
    const float z = x + 0.044715f * ((x * x) * x);
    const float u = 0.7978845608028654f * z;
    const float th = 1.0f - 2.0f / (exp_cw(2.0f * u) + 1.0f);
    return (0.5f * x) * (1.0f + th);
}

// GELU of a BF16 input by table.  Over the finite BF16 values, gelu_tanh(x)
// is exactly 0.5 x below 2^-25 in magnitude (BF16 exponent field < 102),
// exactly x for x >= 8 and -0 for x <= -8 (exponent field >= 130); the
// 2 x 28 binades between are tabulated (entry = gelu_tanh of the value, so
// the lookup equals gelu_tanh bit for bit; exhaustive tests).  The amax pass
// writes the table to the workspace; each encode workgroup copies it to LDS.
constexpr int kGeluTabE0 = 102, kGeluTabE1 = 130;
constexpr int kGeluTabHalf = (kGeluTabE1 - kGeluTabE0) * 128;    // one sign
constexpr int kGeluTabSize = 2 * kGeluTabHalf;

// Entry i of the table (positive values first, then negative ones).
__device__ __forceinline__ float gelu_table_entry(int i) {
    const uint32_t h = (uint32_t)(i % kGeluTabHalf + (kGeluTabE0 << 7)) |
                       (i >= kGeluTabHalf ? 0x8000u : 0u);
    return gelu_tanh(__uint_as_float(h << 16));
}

// Workspace table -> LDS (every thread of the workgroup takes part; the
// caller synchronises before the first lookup).
__device__ __forceinline__ void gelu_table_load(float *lds, const float *tab) {
    for (int i = threadIdx.x; i < kGeluTabSize / 4; i += blockDim.x)
        reinterpret_cast<float4 *>(lds)[i] = reinterpret_cast<const float4 *>(tab)[i];
}

// The same without a branch (for code where a wave-uniform branch per
// element would split the control flow too finely).
__device__ __forceinline__ float gelu_bf16_select(uint32_t h, const float *tab) {
    const uint32_t a = h & 0x7FFFu;
    const uint32_t d = a - (uint32_t)(kGeluTabE0 << 7);
    const uint32_t i = min(d, (uint32_t)kGeluTabHalf - 1u) + (h >> 15) * (uint32_t)kGeluTabHalf;
    const float t = tab[i];                  // always in the table: loaded unconditionally
    const float x = __uint_as_float(h << 16);
    const float big = (h & 0x8000u) ? -0.0f : x;
    const float out = a < (uint32_t)(kGeluTabE0 << 7) ? 0.5f * x : big;
    return d >= (uint32_t)kGeluTabHalf ? out : t;
}

__device__ __forceinline__ float gelu_bf16(uint32_t h, const float *tab) {
    const uint32_t a = h & 0x7FFFu;
    const uint32_t d = a - (uint32_t)(kGeluTabE0 << 7);     // wraps below the table
    const uint32_t i = min(d, (uint32_t)kGeluTabHalf - 1u) + (h >> 15) * (uint32_t)kGeluTabHalf;
    float r = tab[i];
    // outside the table (rare): skipped unless some lane of the wave needs it
    if (__builtin_amdgcn_ballot_w64(d >= (uint32_t)kGeluTabHalf)) {
        const float x = __uint_as_float(h << 16);
        const float big = (h & 0x8000u) ? -0.0f : x;
        if (d >= (uint32_t)kGeluTabHalf) r = a < (uint32_t)(kGeluTabE0 << 7) ? 0.5f * x : big;
    }
    return r;
}

// ---------------------------------------------------------------------------
// Slab copies (global -> LDS, asynchronous) are issued through inline
// assembly.  Issued through the compiler builtin, a copy counts as an LDS
// store to an unknown address, and the compiler then waits for every copy in
// flight before any later LDS read, which serialises the ring.  The loop
// orders copies and reads itself (s_waitcnt vmcnt, then a workgroup barrier).
// M0 holds the wave's LDS destination; a wait state separates its write from
// the copy that reads it.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void copy_lds16(const void *g, const void *lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_addr(lds))
                 : "memory");
}
__device__ __forceinline__ void copy_lds4(const void *g, const void *lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_addr(lds))
                 : "memory");
}

// ---------------------------------------------------------------------------
// Cross-lane maxima inside aligned groups of 2 and 4 lanes (DPP quad_perm).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max_lane_pair(float v) {
    // quad_perm [1,0,3,2]
    float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    return fmaxf(v, o);
}

__device__ __forceinline__ float max_lane_quad(float v) {
    v = max_lane_pair(v);
    // quad_perm [2,3,0,1]
    float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    return fmaxf(v, o);
}

// ---- combine wire format: 32-point RHT and S2F6 (4bit.vizuara.ai, section
// 11; End-to-End 4-Bit Training, "quantized communication") ----

constexpr float kInvSqrt32 = 0.17677669529663688f;   // 1/sqrt(32), rounded to FP32

// Five sum / difference stages (pair distance 1, 2, 4, 8, 16) and the
// multiply by 1/sqrt(32); every step one FP32 operation.
__device__ __forceinline__ void hadamard32(float y[32]) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if ((i & h) == 0) {
                const float p = y[i], q = y[i + h];
                y[i] = p + q;
                y[i + h] = p - q;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = y[i] * kInvSqrt32;
}

__device__ __forceinline__ void flip_signs32(float y[32], uint32_t signs) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
        y[i] = __uint_as_float(__float_as_uint(y[i]) ^ (((signs >> i) & 1u) << 31));
}

// The smallest k with amax <= (127/64) 2^k, clamped to [-127, 127]: with
// amax = m 2^E, m in [0.5, 1), 127/64 = 0.9921875 * 2: k = E - 1 if
// m <= 0.9921875, else E.
__device__ __forceinline__ int s2f6_k(float amax) {
    if (amax == 0.0f) return -127;
    int E;
    const float m = frexpf(amax, &E);
    const int k = (m <= 0.9921875f) ? E - 1 : E;
    return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// S2F6 code byte of y * 2^(6-k): nearest integer, ties to even, within
// [-128, 127].  Adding 1.5 * 2^23 rounds to an integer (nearest even) and
// leaves it, two's complement, in the low bits of the sum.
__device__ __forceinline__ uint32_t s2f6_byte(float y, int k) {
    const float t = fminf(fmaxf(ldexpf(y, 6 - k), -128.0f), 127.0f);
    return __float_as_uint(t + 12582912.0f) & 0xFFu;
}

}  // namespace bbs

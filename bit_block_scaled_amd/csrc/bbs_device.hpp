// Device-side building blocks of the NVFP4 / MXFP8 kernels (gfx950).
//
// Formats follow 4bit.vizuara.ai (sections 3-6) and "Pretraining LLMs with
// NVFP4" ("NVFP4 Format and Quantization Procedure"):
//   E2M1  s|ee|m, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//   E4M3  s|eeee|mmm, bias 7, max 448, min 2^-9, 0x7F is NaN (never written)
//   E8M0  2^(byte - 127)
// Every FP32 step that decides a code is a single IEEE operation rounded to
// nearest even; the library is built with FP contraction off.
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

// Unbiased binade exponent floor(log2 a) read from the FP32 bits (a >= 0);
// zero and FP32 subnormals give -127, below every clamp used here.
__device__ __forceinline__ int binade(float a) {
    return (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
}

// 2^e as an FP32 constant, for |e| < 127.
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// ---------------------------------------------------------------------------
// E4M3
// ---------------------------------------------------------------------------

// Positive E4M3 code -> value.
__device__ __forceinline__ float e4m3_pos_value(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Magnitude code of |v| on the E4M3 grid.  Rounding happens on t, the
// magnitude in units of the local grid step 2^(e-3), e = clamp(floor(log2|v|),
// -6, 8): q = rne(t) or floor(t + u).  The code is then ((e+7) << 3) + q - 8,
// which also covers the subnormal binade (e = -6 gives code q) and a carry
// into the next binade (q = 16); codes past 0x7E saturate at 448.
template <bool SR>
__device__ __forceinline__ uint32_t e4m3_mag_code(float a, float u) {
    int e = binade(a);
    e = e < -6 ? -6 : (e > 8 ? 8 : e);
    float t = a * pow2i(3 - e);                  // exact power-of-two scaling
    float q = SR ? floorf(t + u) : __builtin_rintf(t);
    q = fminf(q, 16.0f);
    int code = ((e + 7) << 3) + (int)q - 8;
    return (uint32_t)(code > 0x7E ? 0x7E : code);
}

template <bool SR>
__device__ __forceinline__ uint32_t e4m3_code(float v, float u) {
    return e4m3_mag_code<SR>(fabsf(v), u) | ((__float_as_uint(v) >> 24) & 0x80u);
}

// ---------------------------------------------------------------------------
// E2M1
// ---------------------------------------------------------------------------

// E2M1 magnitude code of |v|: e = clamp(floor(log2|v|), 0, 2), t = |v| / 2^(e-1),
// q = rne(t) or floor(t + u); code = min(q + 2e, 7) (q = 2..4 in the normal
// binades, 0..4 in the first; everything past 6 saturates at code 7).
template <bool SR>
__device__ __forceinline__ uint32_t e2m1_mag_code(float a, float u) {
    int e = binade(a);
    e = e < 0 ? 0 : (e > 2 ? 2 : e);
    float t = a * pow2i(1 - e);
    float q = SR ? floorf(t + u) : __builtin_rintf(t);
    q = fminf(q, 8.0f);
    int code = (int)q + 2 * e;
    return (uint32_t)(code > 7 ? 7 : code);
}

template <bool SR>
__device__ __forceinline__ uint32_t e2m1_code(float v, float u) {
    return e2m1_mag_code<SR>(fabsf(v), u) | ((__float_as_uint(v) >> 28) & 8u);
}

// E2M1 nibble -> FP32 value.
__device__ __forceinline__ float e2m1_value(uint32_t n) {
    uint32_t e = (n >> 1) & 3u, m = n & 1u;
    uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
    return __uint_as_float(bits | ((n & 8u) << 28));
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

// Block scale code: E4M3(rne((amax_b / 6) * s_enc)), never below code 1.
__device__ __forceinline__ uint32_t block_scale_code(float amax_b, float s_enc) {
    float t = (amax_b / 6.0f) * s_enc;
    uint32_t c = e4m3_mag_code<false>(t, 0.0f);
    return c ? c : 1u;
}

// s_enc_b = 1 / (E4M3(code) * s_dec).
__device__ __forceinline__ float block_enc_scale(uint32_t code, float s_dec) {
    return 1.0f / (e4m3_pos_value(code) * s_dec);
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

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) and the SR uniforms
// ---------------------------------------------------------------------------

struct u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // full 64-bit products (one v_mad_u64_u32 each)
        const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// The eight uniforms of elements 8n .. 8n+7 of one output copy:
// u_j = (16-bit lane j + 1/2) / 65536, lane j = word j/2, low half first.
__device__ __forceinline__ void sr_uniforms8(uint64_t seed, uint32_t stream, uint64_t n,
                                             float u[8]) {
    u32x4 w = philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), stream, 0u, (uint32_t)seed,
                            (uint32_t)(seed >> 32));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u[2 * j] = ((float)(ws[j] & 0xFFFFu) + 0.5f) * (1.0f / 65536.0f);
        u[2 * j + 1] = ((float)(ws[j] >> 16) + 0.5f) * (1.0f / 65536.0f);
    }
}

// ---------------------------------------------------------------------------
// 16-point random Hadamard transform: sign flips, four sum/difference stages
// with pair distance 1, 2, 4, 8, then one multiply by 1/4 (all FP32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rht16(float y[16], uint32_t signs) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if ((signs >> i) & 1u) y[i] = -y[i];
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
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = y[i] * 0.25f;
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

}  // namespace bbs

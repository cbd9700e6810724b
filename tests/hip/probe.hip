// Probes of gfx950 instruction behaviour that the library's kernels rely on
// or may rely on: the per-lane data / scale layout of the block-scaled FP8
// MFMA, and the rounding and scaling of the FP4 / FP8 conversion
// instructions.  Every probe only reads and writes the buffers it is given,
// with grids sized by the host wrapper.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// One wave per (hot lane L, hot byte J): the operand `which` (0 = A, 1 = B)
// holds E4M3 1.0 (0x38) only at byte J of lane L, the other operand is all
// 1.0.  The one-hot operand's scale in lane l is 2^(l/16) (byte 127 + l/16);
// the other operand's scales are 1.0.  out[wave][m][n] = the 16x16 result.
__global__ void mfma_scale_layout_kernel(int which, const int *one, float *out) {
    const int lane = threadIdx.x;
    const int L = blockIdx.x / 32, J = blockIdx.x % 32;
    uint8_t hot[32], ones[32];
    for (int j = 0; j < 32; ++j) {
        hot[j] = (lane == L && j == J) ? 0x38 : 0x00;
        ones[j] = 0x38;
    }
    i32x8 h, o;
    for (int v = 0; v < 8; ++v) {
        h[v] = (int)(hot[4 * v] | (hot[4 * v + 1] << 8) | (hot[4 * v + 2] << 16) | ((uint32_t)hot[4 * v + 3] << 24));
        o[v] = (int)(ones[4 * v] | (ones[4 * v + 1] << 8) | (ones[4 * v + 2] << 16) | ((uint32_t)ones[4 * v + 3] << 24));
    }
    const int s_var = 127 * one[0] + (lane >> 4);   // runtime values, not constants
    const int s_one = 127 * one[0];
    f32x4 acc = {0, 0, 0, 0};
    if (which == 0)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(h, o, acc, 0, 0, 0, s_var, 0, s_one);
    else
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o, h, acc, 0, 0, 0, s_one, 0, s_var);
    // store raw accumulator registers: out[wave][lane][v]
    for (int v = 0; v < 4; ++v) out[(blockIdx.x * 64 + lane) * 4 + v] = acc[v];
}

// cvt_scalef32_pk_bf16_fp4: for every scale s and source byte b, the two
// BF16 results for byte select 0..3 of a word holding b in every byte.
__global__ void cvt_bf16_fp4_kernel(const float *scales, int ns, uint32_t *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ns * 256) return;
    const int si = i / 256, b = i % 256;
    const uint32_t src = (uint32_t)b * 0x01010101u;
    const float s = scales[si];
    bf16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, s, 0);
    bf16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, s, 1);
    bf16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, s, 2);
    bf16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, s, 3);
    out[i * 4 + 0] = __builtin_bit_cast(uint32_t, r0);
    out[i * 4 + 1] = __builtin_bit_cast(uint32_t, r1);
    out[i * 4 + 2] = __builtin_bit_cast(uint32_t, r2);
    out[i * 4 + 3] = __builtin_bit_cast(uint32_t, r3);
}

// cvt_scalef32_pk_f16_fp4 at arbitrary FP32 scales: does the instruction
// multiply by the whole scale or by its power of two only?
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__global__ void cvt_f16_fp4_kernel(const float *scales, int ns, uint32_t *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ns * 256) return;
    const int si = i / 256, b = i % 256;
    const uint32_t src = (uint32_t)b * 0x01010101u;
    const float s = scales[si];
    f16x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, s, 0);
    out[i] = __builtin_bit_cast(uint32_t, r0);
}

// cvt_scalef32_pk_fp4_f32 with scale 1.0: the packed byte for (x[i], -x[i]).
__global__ void cvt_fp4_f32_kernel(const float *x, int n, const float *scale, uint8_t *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[i], -x[i], scale[0], 0);
    out[i] = (uint8_t)(r & 0xFF);
}

// cvt_scalef32_pk_fp8_f32 (E4M3) with scale 1.0: bytes for (x[i], -x[i]).
__global__ void cvt_fp8_f32_kernel(const float *x, int n, const float *scale, uint16_t *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    i16x2 old = {0, 0};
    i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, x[i], -x[i], scale[0], false);
    out[i] = (uint16_t)r[0];
}

// The same with E2M1 operands (format 4): the one-hot operand holds 1.0
// (code 2) only at nibble J of lane L's first 16 bytes, the other operand
// 1.0 in every nibble of its first 16 bytes (the upper 16 bytes are unused).
__global__ void mfma_scale_layout_fp4_kernel(int which, const int *one, float *out) {
    const int lane = threadIdx.x;
    const int L = blockIdx.x / 32, J = blockIdx.x % 32;
    i32x8 h, o;
    for (int v = 0; v < 8; ++v) {
        h[v] = 0;
        o[v] = v < 4 ? 0x22222222 : 0;
    }
    if (lane == L) h[J / 8] = 2 << (4 * (J % 8));
    const int s_var = 127 * one[0] + (lane >> 4);
    const int s_one = 127 * one[0];
    f32x4 acc = {0, 0, 0, 0};
    if (which == 0)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(h, o, acc, 4, 4, 0, s_var, 0, s_one);
    else
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(o, h, acc, 4, 4, 0, s_one, 0, s_var);
    for (int v = 0; v < 4; ++v) out[(blockIdx.x * 64 + lane) * 4 + v] = acc[v];
}

// The 32 x 32 x 64 form with E2M1 operands: one-hot nibble J (< 32) of lane
// L's first 16 bytes, scales 2^(lane / 32) on the one-hot operand.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__global__ void mfma32_scale_layout_fp4_kernel(int which, const int *one, float *out) {
    const int lane = threadIdx.x;
    const int L = blockIdx.x / 32, J = blockIdx.x % 32;
    i32x8 h, o;
    for (int v = 0; v < 8; ++v) {
        h[v] = 0;
        o[v] = v < 4 ? 0x22222222 : 0;
    }
    if (lane == L) h[J / 8] = 2 << (4 * (J % 8));
    const int s_var = 127 * one[0] + (lane >> 5);
    const int s_one = 127 * one[0];
    f32x16_t acc;
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    if (which == 0)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(h, o, acc, 4, 4, 0, s_var, 0, s_one);
    else
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o, h, acc, 4, 4, 0, s_one, 0, s_var);
    for (int v = 0; v < 16; ++v) out[(blockIdx.x * 64 + lane) * 16 + v] = acc[v];
}

extern "C" {
int probe_mfma32_scale_layout_fp4(int which, const int *one, float *out) {
    hipLaunchKernelGGL(mfma32_scale_layout_fp4_kernel, dim3(64 * 32), dim3(64), 0, 0, which, one,
                       out);
    return (int)hipDeviceSynchronize();
}
int probe_mfma_scale_layout_fp4(int which, const int *one, float *out) {
    hipLaunchKernelGGL(mfma_scale_layout_fp4_kernel, dim3(64 * 32), dim3(64), 0, 0, which, one,
                       out);
    return (int)hipDeviceSynchronize();
}
int probe_mfma_scale_layout(int which, const int *one, float *out) {
    hipLaunchKernelGGL(mfma_scale_layout_kernel, dim3(64 * 32), dim3(64), 0, 0, which, one, out);
    return (int)hipDeviceSynchronize();
}
int probe_cvt_bf16_fp4(const float *scales, int ns, uint32_t *out) {
    const int n = ns * 256;
    hipLaunchKernelGGL(cvt_bf16_fp4_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, scales, ns, out);
    return (int)hipDeviceSynchronize();
}
int probe_cvt_f16_fp4(const float *scales, int ns, uint32_t *out) {
    const int n = ns * 256;
    hipLaunchKernelGGL(cvt_f16_fp4_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, scales, ns, out);
    return (int)hipDeviceSynchronize();
}
int probe_cvt_fp4_f32(const float *x, int n, const float *scale, uint8_t *out) {
    hipLaunchKernelGGL(cvt_fp4_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, x, n, scale, out);
    return (int)hipDeviceSynchronize();
}
int probe_cvt_fp8_f32(const float *x, int n, const float *scale, uint16_t *out) {
    hipLaunchKernelGGL(cvt_fp8_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, x, n, scale, out);
    return (int)hipDeviceSynchronize();
}
}

// Stochastic conversions as the quantizers issue them: one value per
// instruction (+0 in the second slot of the FP4 pair), random operand
// (h << 16) | 0x8000 for a 16-bit uniform h, scale 1.0.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__global__ void cvt_sr_kernel(const float *x, const uint32_t *h, int n, const float *scale,
                              uint8_t *fp4, uint8_t *fp8) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t r = (h[i] << 16) | 0x8000u;
    f32x2 p = {x[i], 0.0f};
    fp4[i] = (uint8_t)(__builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, r, scale[0], 0) & 0xFF);
    fp8[i] = (uint8_t)(__builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, x[i], r, scale[0], 0) & 0xFF);
}

extern "C" int probe_cvt_sr(const float *x, const uint32_t *h, int n, const float *scale,
                            uint8_t *fp4, uint8_t *fp8) {
    hipLaunchKernelGGL(cvt_sr_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, x, h, n, scale, fp4,
                       fp8);
    return (int)hipDeviceSynchronize();
}

// The library's own GELU and exp (tanh form, Cody-Waite exp), element by
// element: the kernels' fused activation must equal the oracle's bit for bit.
#include "../../bit_block_scaled_amd/csrc/bbs_device.hpp"

__global__ void gelu_kernel(const float *x, int n, float *g, float *e) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    g[i] = bbs::gelu_tanh(x[i]);
    e[i] = bbs::exp_cw(x[i]);
}

extern "C" int probe_gelu(const float *x, int n, float *g, float *e) {
    hipLaunchKernelGGL(gelu_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, x, n, g, e);
    return (int)hipDeviceSynchronize();
}

// The quantizers' a / 6 (bbs::div6: constant reciprocal and one FMA
// correction) against IEEE division over every non-negative finite FP32 a
// (bit patterns 0 .. 0x7F7FFFFF); mismatches are counted.
__global__ void div6_kernel(unsigned long long *bad) {
    unsigned long long cnt = 0;
    for (uint64_t u = blockIdx.x * 256ull + threadIdx.x; u <= 0x7F7FFFFFull;
         u += (uint64_t)gridDim.x * 256ull) {
        const float a = __uint_as_float((uint32_t)u);
        if (__float_as_uint(bbs::div6(a)) != __float_as_uint(a / 6.0f)) ++cnt;
    }
    if (cnt) atomicAdd(bad, cnt);
}

// The MXFP8 exponent from the FP32 bits (bbs::e8m0_byte) against the frexp
// form of the rule (bbs::e8m0_k + 127) over every non-negative finite FP32.
__global__ void e8m0_kernel(unsigned long long *bad) {
    unsigned long long cnt = 0;
    for (uint64_t u = blockIdx.x * 256ull + threadIdx.x; u <= 0x7F7FFFFFull;
         u += (uint64_t)gridDim.x * 256ull) {
        const float a = __uint_as_float((uint32_t)u);
        if (bbs::e8m0_byte(a) != (uint32_t)(bbs::e8m0_k(a) + 127)) ++cnt;
    }
    if (cnt) atomicAdd(bad, cnt);
}

// FP8 conversions at scale 2^k (as the MXFP8 copies issue them, with the
// 2^-127 blocks doubled and converted at 2^-126) against the value divided
// by 2^k with ldexp and converted at scale 1.0, for every E8M0 byte 0..254
// and `per` hashed values x (|x 2^-k| <= 448, magnitudes from 2^-30 up) and
// random operands per byte; bad[0] counts stochastic mismatches, bad[1]
// nearest-even ones.
__device__ __forceinline__ uint32_t probe_hash(uint32_t h) {
    h ^= h >> 16; h *= 0x7feb352du; h ^= h >> 15; h *= 0x846ca68bu; h ^= h >> 16;
    return h;
}
__global__ void fp8_scale_kernel(int per, unsigned long long *bad) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= 255 * per) return;
    const uint32_t kb = (uint32_t)(i / per);
    const int k = (int)kb - 127;
    const uint32_t h1 = probe_hash(2u * i + 1u), h2 = probe_hash(2u * i + 2u);
    int e = (int)(h1 % 39u) - 30;                          // |x 2^-k| in [2^-30, 2^9)
    if (e + k > 126) e = 126 - k;                          // x stays finite
    float t = ldexpf(1.0f + (h2 >> 9) * 0x1p-23f, e);
    t = fminf(t, 448.0f);
    if (h1 & 1u) t = -t;
    const float x = ldexpf(t, k);                          // exact unless x is an FP32 subnormal
    const float xr = ldexpf(x, -k);                        // the value the copy must round
    const uint32_t r = probe_hash(i * 7u + 11u);
    const float y = kb == 0 ? x * 2.0f : x;
    const float cs = bbs::e8m0_cvt_scale(kb);
    const int a = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, xr, r, 1.0f, 0) & 0xFF;
    const int b = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, y, r, cs, 0) & 0xFF;
    const i16x2 ra = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2{0, 0}, xr, 0.0f, 1.0f, false);
    const i16x2 rb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2{0, 0}, y, 0.0f, cs, false);
    if (a != b) atomicAdd(&bad[0], 1ull);
    if ((ra[0] & 0xFF) != (rb[0] & 0xFF)) atomicAdd(&bad[1], 1ull);
}

extern "C" {
int probe_div6(unsigned long long *bad) {
    hipLaunchKernelGGL(div6_kernel, dim3(8192), dim3(256), 0, 0, bad);
    return (int)hipDeviceSynchronize();
}
int probe_e8m0(unsigned long long *bad) {
    hipLaunchKernelGGL(e8m0_kernel, dim3(8192), dim3(256), 0, 0, bad);
    return (int)hipDeviceSynchronize();
}
int probe_fp8_scale(int per, unsigned long long *bad) {
    const int n = 255 * per;
    hipLaunchKernelGGL(fp8_scale_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, per, bad);
    return (int)hipDeviceSynchronize();
}
}

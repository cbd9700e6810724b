// Combine wire format of the mixture-of-experts layer (4bit.vizuara.ai,
// section 11; End-to-End 4-Bit Training, "quantized communication"):
//   encode   s2f6_encode_kernel: each 32-value chunk of a row is rotated by
//            the 32-point RHT (sign flips, Sylvester butterflies, times
//            1/sqrt(32)) and stored as S2F6 (int8 / 64) with one E8M0 scale:
//            8.25 bits per value instead of 16.
//   combine  s2f6_combine_kernel: the receiver decodes the K copies of a
//            token (one per routed expert), sums them with their weights in
//            FP32, then undoes the rotation once (the RHT is linear).
// One 32-value chunk per lane: the transform stays in registers, a wave
// reads / writes 64 consecutive chunks of a row.
#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

constexpr int kCodecThreads = 256;
template <bool RHT>
__global__ __launch_bounds__(kCodecThreads) void s2f6_encode_kernel(const uint16_t *__restrict__ x,
                                                                    int64_t R, int64_t C, int64_t ld,
                                                                    uint32_t signs,
                                                                    int8_t *__restrict__ codes,
                                                                    uint8_t *__restrict__ scales) {
    const int64_t nb = C / 32;
    const int64_t b = (int64_t)blockIdx.x * kCodecThreads + threadIdx.x;
    if (b >= R * nb) return;
    const int64_t r = b / nb, cb = b - r * nb;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + r * ld + cb * 32);
    float y[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            y[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
            y[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
    if (RHT) {
        flip_signs32(y, signs);
        hadamard32(y);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[i]));
    const int k = s2f6_k(amax);
    uint32_t word[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        word[i] = pack_bytes4(s2f6_byte(y[4 * i], k), s2f6_byte(y[4 * i + 1], k),
                              s2f6_byte(y[4 * i + 2], k), s2f6_byte(y[4 * i + 3], k));
    uint4 *dst = reinterpret_cast<uint4 *>(codes + r * C + cb * 32);
    dst[0] = make_uint4(word[0], word[1], word[2], word[3]);
    dst[1] = make_uint4(word[4], word[5], word[6], word[7]);
    scales[b] = (uint8_t)(k + 127);
}

// out[t] chunk = inverse RHT of sum_j w[t][j] * decode(row src[t][j]);
// decode(code) = code * 2^(k-6) (exact); the weight multiply and every
// addition round once, in slot order; rows with a negative index (or one
// past the input) are skipped.  The inverse of the rotation is the same butterflies and
// multiply, then the sign flips.
template <bool RHT, bool WEIGHTS, bool BF16_OUT>
__global__ __launch_bounds__(kCodecThreads) void s2f6_combine_kernel(
    const int8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int64_t C,
    const int32_t *__restrict__ src, const float *__restrict__ w, int64_t T, int K,
    int64_t src_rows, uint32_t signs, void *__restrict__ out, int64_t ldo) {
    const int64_t nb = C / 32;
    const int64_t b = (int64_t)blockIdx.x * kCodecThreads + threadIdx.x;
    if (b >= T * nb) return;
    const int64_t t = b / nb, cb = b - t * nb;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
    for (int j = 0; j < K; ++j) {
        const int32_t row = src[t * K + j];
        if (row < 0 || row >= src_rows) continue;     // a dropped slot (or a bad index)
        const uint4 *p = reinterpret_cast<const uint4 *>(codes + (int64_t)row * C + cb * 32);
        const uint4 c0 = p[0], c1 = p[1];
        const float unit = ldexpf(1.0f, (int)scales[(int64_t)row * nb + cb] - 127 - 6);
        const float wt = WEIGHTS ? w[t * K + j] : 1.0f;
        const uint32_t word[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            // sign-extended byte i, times the power-of-two unit: exact
            const int q = (int)(word[i >> 2] << (24 - 8 * (i & 3))) >> 24;
            float d = (float)q * unit;
            if (WEIGHTS) d = wt * d;
            acc[i] = acc[i] + d;
        }
    }
    if (RHT) {
        hadamard32(acc);
        flip_signs32(acc, signs);
    }
    if (BF16_OUT) {
        uint32_t pk[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pk[i] = pk_bf16(acc[2 * i], acc[2 * i + 1]);
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + t * ldo + cb * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = make_uint4(pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]);
    } else {
        float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(out) + t * ldo + cb * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    }
}

hipError_t launch_s2f6_encode(const uint16_t *x, int64_t R, int64_t C, int64_t ld, bool rht,
                              uint32_t signs, int8_t *codes, uint8_t *scales, hipStream_t s) {
    const int64_t n = R * (C / 32);
    const dim3 grid((unsigned)((n + kCodecThreads - 1) / kCodecThreads));
    if (rht)
        hipLaunchKernelGGL((s2f6_encode_kernel<true>), grid, dim3(kCodecThreads), 0, s, x, R, C, ld,
                           signs, codes, scales);
    else
        hipLaunchKernelGGL((s2f6_encode_kernel<false>), grid, dim3(kCodecThreads), 0, s, x, R, C,
                           ld, signs, codes, scales);
    return hipGetLastError();
}

template <bool R_, bool W_, bool B_>
static void launch_comb(const S2F6CombineParams &p, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((s2f6_combine_kernel<R_, W_, B_>), grid, dim3(kCodecThreads), 0, s,
                       p.codes, p.scales, p.C, p.src, p.w, p.T, p.K, p.src_rows, p.signs, p.out,
                       p.ldo);
}

hipError_t launch_s2f6_combine(const S2F6CombineParams &p, bool rht, bool bf16_out,
                               hipStream_t s) {
    const int64_t n = p.T * (p.C / 32);
    const dim3 grid((unsigned)((n + kCodecThreads - 1) / kCodecThreads));
    const bool wt = p.w != nullptr;
    switch ((rht << 2) | (wt << 1) | bf16_out) {
        case 0b000: launch_comb<0, 0, 0>(p, grid, s); break;
        case 0b001: launch_comb<0, 0, 1>(p, grid, s); break;
        case 0b010: launch_comb<0, 1, 0>(p, grid, s); break;
        case 0b011: launch_comb<0, 1, 1>(p, grid, s); break;
        case 0b100: launch_comb<1, 0, 0>(p, grid, s); break;
        case 0b101: launch_comb<1, 0, 1>(p, grid, s); break;
        case 0b110: launch_comb<1, 1, 0>(p, grid, s); break;
        default: launch_comb<1, 1, 1>(p, grid, s); break;
    }
    return hipGetLastError();
}

}  // namespace bbs

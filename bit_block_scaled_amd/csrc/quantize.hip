// NVFP4 quantizer and MXFP8 requantizer kernels (gfx950).
//
// Quantize (Pretraining LLMs with NVFP4, "NVFP4 Format and Quantization
// Procedure", steps 1-4; 4bit.vizuara.ai sections 5-6, 13):
//   pass 1  amax_kernel / amax_rht_kernel: partial maxima of |x| (or of the
//           RHT'd column chunks) per workgroup, no atomics, no zeroing.
//   pass 2  quant_tile_kernel: every workgroup folds the partials into the
//           tensor amax (bit-identical everywhere), then each thread owns a
//           16-row x 8-column tile of x loaded with 16-byte rows, and writes
//           from that one read any of: the row-wise NVFP4 copy (block of 16 =
//           two neighbouring lanes), the column-wise NVFP4 copy (x^T: eight
//           full column blocks per thread, optional RHT), and the row-wise
//           MXFP8 copy (block of 32 = four lanes).
// Requantize (4bit.vizuara.ai sections 9-10): requant_kernel dequantizes a
// 32-row x 16-column tile of an NVFP4 matrix in FP32, and writes the 16
// transposed rows of 32 as MXFP8 (E8M0 per 32, E4M3 elements, RTN or SR).
#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

constexpr int kQuantThreads = 256;

// ---------------------------------------------------------------------------
// Pass 1: partial amax.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float block_max_256(float v, float *red) {
    // wave reduction through DPP-free shuffles, then across the 4 waves
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kQuantThreads / 64; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// max |x| over rows x cols; each thread reads 8 BF16 (16 bytes) per step.
__global__ __launch_bounds__(kQuantThreads) void amax_kernel(const uint16_t *__restrict__ x,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ld, float *__restrict__ part) {
    __shared__ float red[kQuantThreads / 64];
    const int64_t groups_per_row = cols / 8;
    const int64_t total = rows * groups_per_row;
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kQuantThreads) {
        const int64_t r = i / groups_per_row, g = i - r * groups_per_row;
        const uint4 v = *reinterpret_cast<const uint4 *>(x + r * ld + g * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m = fmaxf(m, fabsf(bf16_to_f32(w[j] & 0xFFFFu)));
            m = fmaxf(m, fabsf(bf16_to_f32(w[j] >> 16)));
        }
    }
    m = block_max_256(m, red);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// max |RHT(column chunk)| over the column-wise copy: the chunks are 16
// consecutive rows of one column.  Each thread takes a 16 x 8 tile.
__global__ __launch_bounds__(kQuantThreads) void amax_rht_kernel(const uint16_t *__restrict__ x,
                                                                 int64_t rows, int64_t cols,
                                                                 int64_t ld, uint32_t signs,
                                                                 float *__restrict__ part) {
    __shared__ float red[kQuantThreads / 64];
    const int64_t gpr = cols / 8;
    const int64_t total = (rows / 16) * gpr;
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kQuantThreads) {
        const int64_t band = i / gpr, g = i - band * gpr;
        uint4 v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            v[r] = *reinterpret_cast<const uint4 *>(x + (band * 16 + r) * ld + g * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t w = (&v[r].x)[j >> 1];
                y[r] = bf16_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
            }
            rht16(y, signs);
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(y[r]));
        }
    }
    m = block_max_256(m, red);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// ---------------------------------------------------------------------------
// Pass 2: encode.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float fold_partials(const float *part, int n, float *red) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += kQuantThreads) m = fmaxf(m, part[i]);
    return block_max_256(m, red);
}

// Encode 8 values of one row segment with block encode scale s; returns the
// 8 nibbles packed little-endian (element 0 in bits 3:0).
template <bool SR>
__device__ __forceinline__ uint32_t encode8_e2m1(const float v[8], float s, const float u[8]) {
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) packed |= e2m1_code<SR>(v[j] * s, SR ? u[j] : 0.0f) << (4 * j);
    return packed;
}

template <bool HAS_ROW, bool HAS_COL, bool HAS_MX, bool TILE2D, bool RHT>
__global__ __launch_bounds__(kQuantThreads) void quant_tile_kernel(QuantParams p) {
    __shared__ float red[kQuantThreads / 64];
    // Tensor scales, identical in every workgroup.
    float s_enc_plain = 1.0f, s_enc_col = 1.0f;
    if (HAS_ROW || (HAS_COL && !RHT)) s_enc_plain = tensor_s_enc(fold_partials(p.part, p.n_part, red));
    if (HAS_COL && RHT) s_enc_col = tensor_s_enc(fold_partials(p.part_rht, p.n_part_rht, red));
    if (HAS_COL && !RHT) s_enc_col = s_enc_plain;
    const float s_dec_row = 1.0f / s_enc_plain;
    const float s_dec_col = 1.0f / s_enc_col;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (HAS_ROW) p.row_sdec[0] = s_dec_row;
        if (HAS_COL) p.col_sdec[0] = s_dec_col;
    }

    const int lane = threadIdx.x & 63;
    const int64_t gpr = p.C / 8;                      // 8-column groups per row
    const int64_t waves_per_band = (gpr + 63) / 64;
    const int64_t wave = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) >> 6;
    const int64_t band = wave / waves_per_band;
    const int64_t g = (wave - band * waves_per_band) * 64 + lane;
    if (band >= p.R / 16) return;                    // whole wave leaves together
    const bool active = g < gpr;                      // groups of 4 lanes agree (C % 32 == 0
                                                     // whenever lane groups are combined)
    const int64_t r0 = band * 16, c0 = g * 8;

    uint4 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        v[r] = active ? *reinterpret_cast<const uint4 *>(p.x + (r0 + r) * p.ld + c0)
                      : make_uint4(0, 0, 0, 0);
    auto val = [&](int r, int j) -> float {
        const uint32_t w = (&v[r].x)[j >> 1];
        return bf16_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
    };

    // 16x16 tile amax (two lanes hold one tile).
    float tile_amax = 0.0f;
    if (TILE2D) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) tile_amax = fmaxf(tile_amax, fabsf(val(r, j)));
        tile_amax = max_lane_pair(tile_amax);
    }

    // ---- row-wise NVFP4 copy -------------------------------------------------
    if (HAS_ROW) {
        uint32_t tile_sc = 0;
        float tile_s = 0.0f;
        if (TILE2D) {
            tile_sc = block_scale_code(tile_amax, s_enc_plain);
            tile_s = block_enc_scale(tile_sc, s_dec_row);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x8[8];
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x8[j] = val(r, j);
                a = fmaxf(a, fabsf(x8[j]));
            }
            uint32_t sc;
            float s;
            if (TILE2D) {
                sc = tile_sc;
                s = tile_s;
            } else {
                a = max_lane_pair(a);
                sc = block_scale_code(a, s_enc_plain);
                s = block_enc_scale(sc, s_dec_row);
            }
            uint32_t packed;
            if (p.row_round == 1) {
                float u[8];
                sr_uniforms8(p.row_seed, p.row_stream, (uint64_t)((r0 + r) * gpr + g), u);
                packed = encode8_e2m1<true>(x8, s, u);
            } else {
                packed = encode8_e2m1<false>(x8, s, nullptr);
            }
            if (active) {
                *reinterpret_cast<uint32_t *>(p.row_codes + (r0 + r) * (p.C / 2) + g * 4) = packed;
                if ((lane & 1) == 0) {
                    if (!TILE2D) p.row_scales[(r0 + r) * (p.C / 16) + g / 2] = (uint8_t)sc;
                    else if (r == 0) p.row_scales[band * (p.C / 16) + g / 2] = (uint8_t)sc;
                }
            }
        }
    }

    // ---- row-wise MXFP8 copy -------------------------------------------------
    if (HAS_MX) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x8[8];
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x8[j] = val(r, j);
                a = fmaxf(a, fabsf(x8[j]));
            }
            a = max_lane_quad(a);
            const int k = e8m0_k(a);
            float u[8];
            const bool sr = p.mx_round == 1;
            if (sr) sr_uniforms8(p.mx_seed, p.mx_stream, (uint64_t)((r0 + r) * gpr + g), u);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float y = ldexpf(x8[j], -k);
                const uint32_t c = sr ? e4m3_code<true>(y, u[j]) : e4m3_code<false>(y, 0.0f);
                if (j < 4) lo |= c << (8 * j);
                else hi |= c << (8 * (j - 4));
            }
            if (active) {
                *reinterpret_cast<uint2 *>(p.mx_codes + (r0 + r) * p.C + c0) = make_uint2(lo, hi);
                if ((lane & 3) == 0) p.mx_scales[(r0 + r) * (p.C / 32) + g / 4] = (uint8_t)(k + 127);
            }
        }
    }

    // ---- column-wise NVFP4 copy (of x^T) ---------------------------------------
    if (HAS_COL) {
        uint32_t tile_sc = 0;
        float tile_s = 0.0f;
        if (TILE2D) {
            tile_sc = block_scale_code(tile_amax, s_enc_col);
            tile_s = block_enc_scale(tile_sc, s_dec_col);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] = val(r, j);
            if (RHT) rht16(y, p.rht_signs);
            uint32_t sc;
            float s;
            if (TILE2D) {
                sc = tile_sc;
                s = tile_s;
            } else {
                float a = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(y[r]));
                sc = block_scale_code(a, s_enc_col);
                s = block_enc_scale(sc, s_dec_col);
            }
            const int64_t c = c0 + j;                 // row of the transposed copy
            uint32_t w0, w1;
            if (p.col_round == 1) {
                const uint64_t n0 = (uint64_t)(c * p.R + r0) / 8;
                float u[8];
                sr_uniforms8(p.col_seed, p.col_stream, n0, u);
                w0 = encode8_e2m1<true>(y, s, u);
                sr_uniforms8(p.col_seed, p.col_stream, n0 + 1, u);
                w1 = encode8_e2m1<true>(y + 8, s, u);
            } else {
                w0 = encode8_e2m1<false>(y, s, nullptr);
                w1 = encode8_e2m1<false>(y + 8, s, nullptr);
            }
            if (active) {
                *reinterpret_cast<uint2 *>(p.col_codes + c * (p.R / 2) + r0 / 2) = make_uint2(w0, w1);
                if (!TILE2D) p.col_scales[c * (p.R / 16) + band] = (uint8_t)sc;
                else if (j == 0 && (lane & 1) == 0)
                    p.col_scales[(c / 16) * (p.R / 16) + band] = (uint8_t)sc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Requantize: NVFP4 [R x C] -> MXFP8 of the transpose [C x R].
// Each thread: 32 source rows x 16 source columns (8 code bytes per row).
// ---------------------------------------------------------------------------
template <bool SR>
__global__ __launch_bounds__(kQuantThreads) void requant_kernel(RequantParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t gpr = p.C / 16;                    // 16-column groups per source row
    const int64_t waves_per_band = (gpr + 63) / 64;
    const int64_t wave = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) >> 6;
    const int64_t band = wave / waves_per_band;      // 32-row band of the source
    const int64_t g = (wave - band * waves_per_band) * 64 + lane;
    if (band >= p.R / 32 || g >= gpr) return;        // no cross-lane traffic here
    const int64_t r0 = band * 32, c0 = g * 16;
    const float s_dec = p.s_dec[0];

    uint2 cw[32];
    uint32_t sc[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        cw[r] = *reinterpret_cast<const uint2 *>(p.codes + (r0 + r) * (p.C / 2) + c0 / 2);
        const int64_t srow = p.tile2d ? (r0 + r) / 16 : (r0 + r);
        sc[r] = p.scales[srow * (p.C / 16) + g];
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll 1
    for (int jj = 0; jj < 8; ++jj) {
        const int j = half * 8 + jj;
        float x[32];
        float a = 0.0f;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const uint32_t w = half ? cw[r].y : cw[r].x;
            const uint32_t nib = (w >> (4 * jj)) & 0xFu;
            // (E2M1 x E4M3) is exact; the multiply by s_dec is one FP32 rounding.
            x[r] = (e2m1_value(nib) * e4m3_pos_value(sc[r])) * s_dec;
            a = fmaxf(a, fabsf(x[r]));
        }
        const int k = e8m0_k(a);
        const int64_t c = c0 + j;                    // destination row
        uint32_t out[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float u[8];
            if (SR) sr_uniforms8(p.seed, p.stream, (uint64_t)(c * p.R + r0) / 8 + q, u);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t word = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int e = q * 8 + h * 4 + b;
                    const float y = ldexpf(x[e], -k);
                    word |= e4m3_code<SR>(y, SR ? u[h * 4 + b] : 0.0f) << (8 * b);
                }
                out[q * 2 + h] = word;
            }
        }
        uint4 *dst = reinterpret_cast<uint4 *>(p.out_codes + c * p.R + r0);
        dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
        dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
        p.out_scales[c * (p.R / 32) + band] = (uint8_t)(k + 127);
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after argument checks).
// ---------------------------------------------------------------------------

int amax_grid(int64_t work_items) {
    int64_t g = (work_items + kQuantThreads * 8 - 1) / (kQuantThreads * 8);
    if (g < 1) g = 1;
    if (g > kAmaxPartials) g = kAmaxPartials;
    return (int)g;
}

hipError_t launch_amax(const uint16_t *x, int64_t R, int64_t C, int64_t ld, float *part,
                       int *n_part, hipStream_t s) {
    const int grid = amax_grid(R * (C / 8));
    *n_part = grid;
    hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(kQuantThreads), 0, s, x, R, C, ld, part);
    return hipGetLastError();
}

hipError_t launch_amax_rht(const uint16_t *x, int64_t R, int64_t C, int64_t ld, uint32_t signs,
                           float *part, int *n_part, hipStream_t s) {
    const int grid = amax_grid((R / 16) * (C / 8) * 16);
    *n_part = grid;
    hipLaunchKernelGGL(amax_rht_kernel, dim3(grid), dim3(kQuantThreads), 0, s, x, R, C, ld,
                       signs, part);
    return hipGetLastError();
}

template <bool R_, bool C_, bool M_, bool T_, bool H_>
static void launch_tile(const QuantParams &p, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((quant_tile_kernel<R_, C_, M_, T_, H_>), grid, dim3(kQuantThreads), 0, s, p);
}

hipError_t launch_quant_tile(const QuantParams &p, bool has_row, bool has_col, bool has_mx,
                             bool tile2d, bool rht, hipStream_t s) {
    const int64_t gpr = p.C / 8;
    const int64_t waves = (p.R / 16) * ((gpr + 63) / 64);
    const dim3 grid((unsigned)((waves + 3) / 4));
    // The combinations the quantizer supports (RHT only on a 1x16 column copy).
    const int key = (has_row << 4) | (has_col << 3) | (has_mx << 2) | (tile2d << 1) | rht;
    switch (key) {
        case 0b10000: launch_tile<1, 0, 0, 0, 0>(p, grid, s); break;
        case 0b10010: launch_tile<1, 0, 0, 1, 0>(p, grid, s); break;
        case 0b11000: launch_tile<1, 1, 0, 0, 0>(p, grid, s); break;
        case 0b11010: launch_tile<1, 1, 0, 1, 0>(p, grid, s); break;
        case 0b11001: launch_tile<1, 1, 0, 0, 1>(p, grid, s); break;
        case 0b01000: launch_tile<0, 1, 0, 0, 0>(p, grid, s); break;
        case 0b01010: launch_tile<0, 1, 0, 1, 0>(p, grid, s); break;
        case 0b01001: launch_tile<0, 1, 0, 0, 1>(p, grid, s); break;
        case 0b00100: launch_tile<0, 0, 1, 0, 0>(p, grid, s); break;
        case 0b10100: launch_tile<1, 0, 1, 0, 0>(p, grid, s); break;
        case 0b10110: launch_tile<1, 0, 1, 1, 0>(p, grid, s); break;
        case 0b01100: launch_tile<0, 1, 1, 0, 0>(p, grid, s); break;
        case 0b01101: launch_tile<0, 1, 1, 0, 1>(p, grid, s); break;
        case 0b11100: launch_tile<1, 1, 1, 0, 0>(p, grid, s); break;
        case 0b11101: launch_tile<1, 1, 1, 0, 1>(p, grid, s); break;
        case 0b01110: launch_tile<0, 1, 1, 1, 0>(p, grid, s); break;
        case 0b11110: launch_tile<1, 1, 1, 1, 0>(p, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_requant(const RequantParams &p, bool sr, hipStream_t s) {
    const int64_t gpr = p.C / 16;
    const int64_t waves = (p.R / 32) * ((gpr + 63) / 64);
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (sr) hipLaunchKernelGGL(requant_kernel<true>, grid, dim3(kQuantThreads), 0, s, p);
    else hipLaunchKernelGGL(requant_kernel<false>, grid, dim3(kQuantThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace bbs

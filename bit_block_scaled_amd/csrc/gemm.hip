// Block-scaled GEMMs on CDNA4 matrix cores (gfx950).
//
// NVFP4 x NVFP4 (Pretraining LLMs with NVFP4, "NVFP4 Format and Quantization
// Procedure", step 5): C = s_dec,A * s_dec,B * sum_b E4M3_A,b * E4M3_B,b *
// sum_{k in b} a_k * b_k, FP32 accumulation.
//
// Mapping onto the matrix cores.  gfx950's block-scaled MFMA takes one
// power-of-two (E8M0) scale per 32 K-values, while NVFP4 carries an E4M3
// scale per 16.  An E2M1 code times its E4M3 scale has up to 6 significant
// bits (2 x 4), so it is exact in BF16 (8 bits) and in no FP8/FP6/FP4 operand
// type.  The kernel therefore keeps the packed 4-bit codes and the scale
// bytes in LDS, expands code x scale to BF16 in registers right before each
// MFMA (exact), and runs v_mfma_f32_32x32x16_bf16, whose K = 16 is exactly
// one NVFP4 block.  The two FP32 tensor decode scales are applied once in the
// epilogue.  The products are exact and only the FP32 accumulation rounds.
//
// MXFP8 x MXFP8: E4M3 elements with one E8M0 scale per 32 along K map exactly
// onto v_mfma_scale_f32_16x16x128_f8f6f4 (FP8 operands, per-lane scale byte).
#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 128, kBN = 128, kBK = 64;     // block tile (K in elements)
constexpr int kGemmThreads = 256;                 // 4 waves, 2 x 2, 64 x 64 each
constexpr int kRowBytes = kBK / 2;                // packed codes per tile row
constexpr int kLdsStride = kRowBytes + 4;         // padded row (bank spread)
constexpr int kSBlocks = kBK / 16;                // scale bytes per tile row

// Expand 8 E2M1 codes (one 32-bit word, element 0 in bits 3:0) times a
// positive E4M3 scale into 8 BF16 values.  code x scale has <= 6 significant
// bits, so taking the upper half of the FP32 product is exact.
__device__ __forceinline__ bf16x8 expand8(uint32_t codes, float scale) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = e2m1_value((codes >> (8 * j)) & 0xFu) * scale;
        const float hi = e2m1_value((codes >> (8 * j + 4)) & 0xFu) * scale;
        w[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

struct TileSmem {
    uint8_t a[kBM * kLdsStride];
    uint8_t b[kBN * kLdsStride];
    uint8_t as[kBM * kSBlocks];
    uint8_t bs[kBN * kSBlocks];
};

// Load one K-slab of packed codes for a 128-row operand tile into LDS.
// Thread t handles row t/2, 32 codes (16 bytes) starting at code half*32,
// as two 8-byte granules (16 codes = one NVFP4 block each).
__device__ __forceinline__ void load_codes(uint8_t *dst, const uint8_t *codes, int64_t K,
                                           int64_t grow, bool row_ok, int64_t k0) {
    const int t = threadIdx.x;
    const int row = t >> 1, half = t & 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int64_t kk = k0 + half * 32 + q * 16;
        uint2 v = make_uint2(0, 0);
        if (row_ok && kk < K) v = *reinterpret_cast<const uint2 *>(codes + grow * (K / 2) + kk / 2);
        uint32_t *d = reinterpret_cast<uint32_t *>(dst + row * kLdsStride + half * 16 + q * 8);
        d[0] = v.x;
        d[1] = v.y;
    }
}

__device__ __forceinline__ void load_scales(uint8_t *dst, const uint8_t *scales, int64_t K,
                                            int64_t grow, bool row_ok, int tile2d, int row,
                                            int64_t k0) {
    const int64_t nkb = K / 16;
    const int64_t srow = tile2d ? grow / 16 : grow;
#pragma unroll
    for (int j = 0; j < kSBlocks; ++j) {
        const int64_t kb = k0 / 16 + j;
        dst[row * kSBlocks + j] = (row_ok && kb < nkb) ? scales[srow * nkb + kb] : (uint8_t)0;
    }
}

// One 128 x 128 output tile of C = A * B^T over the full K range.
// a_row(i) maps tile row i to the source row of A (or -1 for no row).
template <bool BF16_OUT, typename RowMap>
__device__ __forceinline__ void gemm_tile(TileSmem &sm, const Fp4View &A, const Fp4View &B,
                                          int64_t K, int64_t m0, int64_t m_end, int64_t n0,
                                          int64_t n_end, RowMap a_row, float out_scale, void *C,
                                          int64_t ldc) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // rows this thread stages
    const int crow = t >> 1;
    const int64_t a_src = (m0 + crow < m_end) ? a_row(m0 + crow) : -1;
    const int64_t b_src = n0 + crow;
    const bool b_ok = b_src < n_end;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};

    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
        load_codes(sm.a, A.codes, K, a_src, a_src >= 0, k0);
        load_codes(sm.b, B.codes, K, b_src, b_ok, k0);
        if (t < kBM) {
            const int64_t src = (m0 + t < m_end) ? a_row(m0 + t) : -1;
            load_scales(sm.as, A.scales, K, src, src >= 0, A.tile2d, t, k0);
        } else {
            const int r = t - kBM;
            load_scales(sm.bs, B.scales, K, n0 + r, n0 + r < n_end, B.tile2d, r, k0);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kSBlocks; ++kk) {
            bf16x8 af[2], bfr[2];
            const int half = lane >> 5;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                const uint32_t c =
                    *reinterpret_cast<const uint32_t *>(sm.a + r * kLdsStride + kk * 8 + half * 4);
                af[i] = expand8(c, e4m3_pos_value(sm.as[r * kSBlocks + kk]));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn * 64 + j * 32 + (lane & 31);
                const uint32_t c =
                    *reinterpret_cast<const uint32_t *>(sm.b + r * kLdsStride + kk * 8 + half * 4);
                bfr[j] = expand8(c, e4m3_pos_value(sm.bs[r * kSBlocks + kk]));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // Epilogue: lane holds column n = lane % 32 and rows 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < m_end && n < n_end) {
                    const float y = acc[i][j][v] * out_scale;
                    if (BF16_OUT)
                        reinterpret_cast<uint16_t *>(C)[m * ldc + n] = (uint16_t)f32_to_bf16(y);
                    else
                        reinterpret_cast<float *>(C)[m * ldc + n] = y;
                }
            }
        }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(kGemmThreads) void nvfp4_gemm_kernel(GemmParams p) {
    __shared__ TileSmem sm;
    const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
    const float out_scale = p.a.s_dec[0] * p.b.s_dec[0];
    gemm_tile<BF16_OUT>(sm, p.a, p.b, p.K, m0, p.M, n0, p.N, [](int64_t r) { return r; },
                        out_scale, p.c, p.ldc);
}

// Grouped GEMM: a persistent grid walks the tiles of all groups.  Every
// workgroup derives the per-group tile counts from group_offsets itself, so
// no host round trip is needed; each workgroup stops when the tile index
// passes the total.
constexpr int kMaxGroups = 1024;

template <bool BF16_OUT>
__global__ __launch_bounds__(kGemmThreads) void grouped_nvfp4_gemm_kernel(GemmParams p) {
    __shared__ TileSmem sm;
    __shared__ int64_t tile_start[kMaxGroups + 1];
    __shared__ int64_t row_start[kMaxGroups + 1];
    const int64_t n_tiles_n = (p.N + kBN - 1) / kBN;
    if (threadIdx.x == 0) {
        int64_t acc = 0, prev = 0;
        for (int g = 0; g <= p.G; ++g) {
            int64_t off = p.group_offsets[g];
            off = off < prev ? prev : off;                  // keep offsets monotone
            off = off > p.max_rows ? p.max_rows : off;      // never past C
            row_start[g] = off;
            if (g > 0) acc += ((off - prev + kBM - 1) / kBM) * n_tiles_n;
            tile_start[g] = acc;   // tiles before group g (g >= 1: through group g-1)
            prev = off;
        }
    }
    __syncthreads();
    // tile_start[g] holds the tile count of groups 0..g-1 for g >= 1; group g
    // owns tiles [tile_start[g], tile_start[g+1]).
    const int64_t total = tile_start[p.G];
    for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
        int g = 0;
        while (g + 1 < p.G && tile_start[g + 1] <= tile) ++g;
        const int64_t local = tile - tile_start[g];
        const int64_t mt = local / n_tiles_n, nt = local - mt * n_tiles_n;
        const int64_t rs = row_start[g], re = row_start[g + 1];
        const int64_t m0 = rs + mt * kBM, n0 = nt * kBN;
        Fp4View B = p.b;
        B.codes = p.b.codes + (int64_t)g * p.N * (p.K / 2);
        B.scales = p.b.scales + (int64_t)g * (B.tile2d ? (p.N / 16) : p.N) * (p.K / 16);
        const float out_scale = p.a.s_dec[0] * p.b.s_dec[g];
        const int32_t *ri = p.row_index;
        const int64_t src_rows = p.a_src_rows;
        gemm_tile<BF16_OUT>(
            sm, p.a, B, p.K, m0, re, n0, p.N,
            [ri, src_rows](int64_t r) -> int64_t {
                const int64_t s = ri ? (int64_t)ri[r] : r;
                return (s >= 0 && s < src_rows) ? s : -1;
            },
            out_scale, p.c, p.ldc);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// MXFP8 x MXFP8 with v_mfma_scale_f32_16x16x128_f8f6f4.
// Tile 128 x 128, K-slab 128 (one MFMA deep); wave tile 64 x 64 = 4 x 4 MFMAs.
// Operand layout of the 16x16x128 MFMA with 8-bit elements (measured on
// gfx950): lane l holds row l%16; its bytes 0-15 are K = 16g .. 16g+15 and its
// bytes 16-31 are K = 64 + 16g .. 64 + 16g + 15, g = l/16.  The E8M0 scale of
// the 32-block b (K = 32b .. 32b+31) is byte 0 of the scale operand of lane
// group b.  So lane group g loads slab bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) and supplies the scale of the slab's block g.
// ---------------------------------------------------------------------------
constexpr int kMxBK = 128;
constexpr int kMxStride = kMxBK + 16;

struct MxSmem {
    uint8_t a[kBM * kMxStride];
    uint8_t b[kBN * kMxStride];
    uint8_t as[kBM * 4];
    uint8_t bs[kBN * 4];
};

template <bool BF16_OUT>
__global__ __launch_bounds__(kGemmThreads) void mxfp8_gemm_kernel(Mx8GemmParams p) {
    __shared__ MxSmem sm;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
    const int64_t nkb = p.K / 32;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0};

    for (int64_t k0 = 0; k0 < p.K; k0 += kMxBK) {
        // codes: 128 rows x 128 bytes per operand = 256 threads x 4 x 16 B
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int idx = q * kGemmThreads + t;     // 0 .. 1023
            const int row = idx >> 3, seg = idx & 7;  // 8 x 16 B per row
            const int64_t kk = k0 + seg * 16;
            uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
            if (m0 + row < p.M && kk < p.K)
                va = *reinterpret_cast<const uint4 *>(p.a_codes + (m0 + row) * p.K + kk);
            if (n0 + row < p.N && kk < p.K)
                vb = *reinterpret_cast<const uint4 *>(p.b_codes + (n0 + row) * p.K + kk);
            *reinterpret_cast<uint4 *>(sm.a + row * kMxStride + seg * 16) = va;
            *reinterpret_cast<uint4 *>(sm.b + row * kMxStride + seg * 16) = vb;
        }
        {
            const int row = t & 127;
            const bool isb = t >= 128;
            const int64_t gr = (isb ? n0 : m0) + row;
            const int64_t lim = isb ? p.N : p.M;
            const uint8_t *sc = isb ? p.b_scales : p.a_scales;
            uint8_t *dst = isb ? sm.bs : sm.as;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t kb = k0 / 32 + j;
                dst[row * 4 + j] = (gr < lim && kb < nkb) ? sc[gr * nkb + kb] : (uint8_t)0;
            }
        }
        __syncthreads();
        const int kg = lane >> 4;                     // K-block of this lane
        i32x8 af[4], bfr[4];
        int as_[4], bs_[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + i * 16 + (lane & 15);
            const uint8_t *row = sm.a + r * kMxStride;
            const uint4 x0 = *reinterpret_cast<const uint4 *>(row + 16 * kg);
            const uint4 x1 = *reinterpret_cast<const uint4 *>(row + 64 + 16 * kg);
            af[i] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            as_[i] = sm.as[r * 4 + kg];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn * 64 + j * 16 + (lane & 15);
            const uint8_t *row = sm.b + r * kMxStride;
            const uint4 x0 = *reinterpret_cast<const uint4 *>(row + 16 * kg);
            const uint4 x1 = *reinterpret_cast<const uint4 *>(row + 64 + 16 * kg);
            bfr[j] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                           (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            bs_[j] = sm.bs[r * 4 + kg];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], bfr[j], acc[i][j], 0, 0, 0, as_[i], 0, bs_[j]);
        __syncthreads();
    }

    // 16x16 output: lane holds column lane%16, rows 4*(lane/16) + v.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + v;
                if (m < p.M && n < p.N) {
                    const float y = acc[i][j][v];
                    if (BF16_OUT)
                        reinterpret_cast<uint16_t *>(p.c)[m * p.ldc + n] = (uint16_t)f32_to_bf16(y);
                    else
                        reinterpret_cast<float *>(p.c)[m * p.ldc + n] = y;
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

hipError_t launch_nvfp4_gemm_big(const GemmParams &p, bool bf16_out, hipStream_t s);
hipError_t launch_grouped_nvfp4_gemm_big(const GemmParams &p, bool bf16_out, hipStream_t s);

// The large-tile kernel needs K % 128 == 0, 8-byte aligned scale rows and
// 16-byte aligned output rows (its epilogue stores 16-byte row segments).
bool big_ok(const GemmParams &p, bool bf16_out) {
    auto al = [](const void *q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) % a) == 0; };
    const int64_t es = bf16_out ? 2 : 4;
    return p.K % 128 == 0 && al(p.a.codes, 16) && al(p.b.codes, 16) && al(p.a.scales, 8) &&
           al(p.b.scales, 8) && al(p.c, 16) && (p.ldc * es) % 16 == 0;
}

hipError_t launch_nvfp4_gemm(const GemmParams &p, bool bf16_out, hipStream_t s) {
    if (big_ok(p, bf16_out)) return launch_nvfp4_gemm_big(p, bf16_out, s);
    const dim3 grid((unsigned)((p.N + kBN - 1) / kBN), (unsigned)((p.M + kBM - 1) / kBM));
    if (bf16_out) hipLaunchKernelGGL(nvfp4_gemm_kernel<true>, grid, dim3(kGemmThreads), 0, s, p);
    else hipLaunchKernelGGL(nvfp4_gemm_kernel<false>, grid, dim3(kGemmThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_grouped_nvfp4_gemm(const GemmParams &p, bool bf16_out, hipStream_t s) {
    if (p.G > kMaxGroups) return hipErrorInvalidValue;
    if (big_ok(p, bf16_out)) return launch_grouped_nvfp4_gemm_big(p, bf16_out, s);
    const dim3 grid(1024);
    if (bf16_out)
        hipLaunchKernelGGL(grouped_nvfp4_gemm_kernel<true>, grid, dim3(kGemmThreads), 0, s, p);
    else
        hipLaunchKernelGGL(grouped_nvfp4_gemm_kernel<false>, grid, dim3(kGemmThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_mxfp8_gemm_big(const Mx8GemmParams &p, bool bf16_out, hipStream_t s);

hipError_t launch_mxfp8_gemm(const Mx8GemmParams &p, bool bf16_out, hipStream_t s) {
    auto al = [](const void *q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) % a) == 0; };
    // the large-tile kernel stores groups of four output columns at once
    if (p.K % 128 == 0 && al(p.a_codes, 16) && al(p.b_codes, 16) && al(p.a_scales, 4) &&
        al(p.b_scales, 4) && p.N % 4 == 0 && al(p.c, 16) && p.ldc % 4 == 0)
        return launch_mxfp8_gemm_big(p, bf16_out, s);
    const dim3 grid((unsigned)((p.N + kBN - 1) / kBN), (unsigned)((p.M + kBM - 1) / kBM));
    if (bf16_out) hipLaunchKernelGGL(mxfp8_gemm_kernel<true>, grid, dim3(kGemmThreads), 0, s, p);
    else hipLaunchKernelGGL(mxfp8_gemm_kernel<false>, grid, dim3(kGemmThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace bbs

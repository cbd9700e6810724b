// NVFP4 x NVFP4 GEMM, large-tile kernel for K % 128 == 0 (gfx950).
//
// C = s_dec,A * s_dec,B * sum_b E4M3_A,b * E4M3_B,b * sum_{k in b} a_k b_k
// (Pretraining LLMs with NVFP4, "NVFP4 Format and Quantization Procedure",
// step 5), FP32 accumulation.
//
// Tiling: a workgroup (4 waves, 2 x 2) owns a 256 x 256 tile of C; each wave
// owns 128 x 128 = 4 x 4 v_mfma_f32_32x32x16_f16 accumulators (256 FP32 per
// lane).  K advances in slabs of 128 (8 NVFP4 blocks), double-buffered in LDS:
// while a slab is consumed, the next one is fetched from global memory into
// registers and stored to the other buffer.  LDS holds the packed 4-bit codes
// as they are in HBM (64 bytes per row and slab) and the block scales already
// converted to FP16 pairs.
//
// Exact expansion: v_cvt_scalef32_pk_f16_fp4 (scale 1.0) turns two E2M1 codes
// into two FP16 values and one v_pk_mul_f16 applies the FP16 copy of the E4M3
// block scale.  code x scale has at most 6 significant bits and lies in
// [2^-10, 2688], so both steps are exact in FP16; the MFMA products are exact
// in FP32 and only the accumulation rounds.
//
// K order inside a slab: lane half h of an MFMA step takes 8 codes from the
// 16-byte group [16h, 16h+16) of the current 32-byte chunk (4 steps per
// chunk), so one ds_read_b128 feeds four MFMA steps.  A and B use the same
// order, so the sum is unchanged; each lane's 8 codes always lie in one block.
//
// Tile order is XCD-aware: workgroup i runs on XCD i % 8, so each XCD is given
// a contiguous range of tile ids, and ids walk 8 M-tiles down before moving
// along N, keeping operand panels shared inside one XCD's L2.
#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace big {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NT = 256;
constexpr int CS = 80;            // LDS row stride of the codes: 64 bytes + 16 pad
constexpr int SB = BK / 16;       // scale blocks per row and slab (8)
constexpr int GROUP_M = 8;

struct Stage {
    uint8_t a[BM * CS];
    uint8_t b[BN * CS];
    uint32_t as[BM * SB];         // FP16 pair (scale, scale) per row and block
    uint32_t bs[BN * SB];
};
struct Smem {
    Stage st[2];
};

// E4M3 byte (positive) -> FP16 bits of the same value.  Normal codes map by
// a shift and an exponent rebias; the subnormal codes m * 2^-9 (m = 1..7) go
// through an integer-to-FP16 conversion and a 9-binade shift.
__device__ __forceinline__ uint32_t e4m3_to_f16_bits(uint32_t b) {
    const uint32_t normal = (b << 7) + 0x2000u;
    const uint32_t sub = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)b) - 0x2400u;
    return b >= 8u ? normal : (b ? sub : 0u);
}

__device__ __forceinline__ uint32_t f16_pair(uint32_t b) {
    const uint32_t h = e4m3_to_f16_bits(b);
    return h | (h << 16);
}

// Eight E2M1 codes of one 32-bit word times an FP16 scale pair -> 8 FP16.
__device__ __forceinline__ f16x8 expand8_f16(uint32_t w, uint32_t scale_pair) {
    const f16x2 s = __builtin_bit_cast(f16x2, scale_pair);
    const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// Per-thread staging registers of one slab.
struct Regs {
    uint4 a[4], b[4];
    uint2 sa, sb;
};

// Source offsets this thread stages each slab (fixed for the whole tile).
struct Plan {
    const uint8_t *a_row[4];      // code row of A for chunk q (nullptr = zero row)
    const uint8_t *b_row[4];
    const uint8_t *sa_row;        // scale row (nullptr = none)
    const uint8_t *sb_row;
};

template <typename RowMap>
__device__ __forceinline__ Plan make_plan(const Fp4View &A, const Fp4View &B, int64_t K,
                                          int64_t m0, int64_t m_end, int64_t n0, int64_t n_end,
                                          RowMap a_row) {
    Plan pl;
    const int t = threadIdx.x;
    const int64_t kb = K / 2, ks = K / 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = (q * NT + t) >> 2;
        const int64_t m = m0 + row;
        const int64_t src = (m < m_end) ? a_row(m) : -1;
        pl.a_row[q] = src >= 0 ? A.codes + src * kb + (t & 3) * 16 : nullptr;
        const int64_t n = n0 + row;
        pl.b_row[q] = n < n_end ? B.codes + n * kb + (t & 3) * 16 : nullptr;
    }
    {
        const int64_t m = m0 + t;
        const int64_t src = (m < m_end) ? a_row(m) : -1;
        pl.sa_row = src >= 0 ? A.scales + (A.tile2d ? src / 16 : src) * ks : nullptr;
        // B: 1x16 -> one scale row per tile row; 16x16 -> 16 tile rows per tile
        const int brows = B.tile2d ? BN / 16 : BN;
        const int64_t n = B.tile2d ? n0 / 16 + t : n0 + t;
        const int64_t lim = B.tile2d ? (n_end + 15) / 16 : n_end;
        pl.sb_row = (t < brows && n < lim) ? B.scales + n * ks : nullptr;
    }
    return pl;
}

__device__ __forceinline__ void fetch(Regs &r, const Plan &pl, int64_t k0) {
    const int64_t cb = k0 / 2, sbk = k0 / 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        r.a[q] = pl.a_row[q] ? *reinterpret_cast<const uint4 *>(pl.a_row[q] + cb) : make_uint4(0, 0, 0, 0);
        r.b[q] = pl.b_row[q] ? *reinterpret_cast<const uint4 *>(pl.b_row[q] + cb) : make_uint4(0, 0, 0, 0);
    }
    r.sa = pl.sa_row ? *reinterpret_cast<const uint2 *>(pl.sa_row + sbk) : make_uint2(0, 0);
    r.sb = pl.sb_row ? *reinterpret_cast<const uint2 *>(pl.sb_row + sbk) : make_uint2(0, 0);
}

__device__ __forceinline__ void store(Stage &st, const Regs &r, bool b_tile2d) {
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = q * NT + t, row = c >> 2, seg = c & 3;
        *reinterpret_cast<uint4 *>(st.a + row * CS + seg * 16) = r.a[q];
        *reinterpret_cast<uint4 *>(st.b + row * CS + seg * 16) = r.b[q];
    }
    uint32_t s[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s[j] = f16_pair((r.sa.x >> (8 * j)) & 0xFFu);
        s[4 + j] = f16_pair((r.sa.y >> (8 * j)) & 0xFFu);
    }
    *reinterpret_cast<uint4 *>(st.as + t * SB) = make_uint4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<uint4 *>(st.as + t * SB + 4) = make_uint4(s[4], s[5], s[6], s[7]);
    if (!b_tile2d || t < BN / 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j] = f16_pair((r.sb.x >> (8 * j)) & 0xFFu);
            s[4 + j] = f16_pair((r.sb.y >> (8 * j)) & 0xFFu);
        }
        *reinterpret_cast<uint4 *>(st.bs + t * SB) = make_uint4(s[0], s[1], s[2], s[3]);
        *reinterpret_cast<uint4 *>(st.bs + t * SB + 4) = make_uint4(s[4], s[5], s[6], s[7]);
    }
}

// One slab: 2 chunks x 4 MFMA steps x (4 x 4) MFMAs per wave.
__device__ __forceinline__ void compute(const Stage &st, f32x16 (&acc)[4][4], bool b_tile2d,
                                        int wm, int wn, int lane) {
    const int h = lane >> 5, rl = lane & 31;
#pragma unroll
    for (int chunk = 0; chunk < 2; ++chunk) {
        uint4 ca[4], cb[4];
        uint2 sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + rl;
            ca[i] = *reinterpret_cast<const uint4 *>(st.a + r * CS + chunk * 32 + h * 16);
            sa[i] = *reinterpret_cast<const uint2 *>(st.as + r * SB + chunk * 4 + 2 * h);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn * 128 + j * 32 + rl;
            const int sr = b_tile2d ? (r >> 4) : r;
            cb[j] = *reinterpret_cast<const uint4 *>(st.b + r * CS + chunk * 32 + h * 16);
            sb[j] = *reinterpret_cast<const uint2 *>(st.bs + sr * SB + chunk * 4 + 2 * h);
        }
#pragma unroll
        for (int step = 0; step < 4; ++step) {
            f16x8 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = step == 0 ? ca[i].x : step == 1 ? ca[i].y : step == 2 ? ca[i].z : ca[i].w;
                af[i] = expand8_f16(w, (step >> 1) ? sa[i].y : sa[i].x);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = step == 0 ? cb[j].x : step == 1 ? cb[j].y : step == 2 ? cb[j].z : cb[j].w;
                bf[j] = expand8_f16(w, (step >> 1) ? sb[j].y : sb[j].x);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
}

template <bool BF16_OUT, typename RowMap>
__device__ __forceinline__ void tile(Smem &sm, const Fp4View &A, const Fp4View &B, int64_t K,
                                     int64_t m0, int64_t m_end, int64_t n0, int64_t n_end,
                                     RowMap a_row, float out_scale, void *C, int64_t ldc) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool bt = B.tile2d != 0;
    const Plan pl = make_plan(A, B, K, m0, m_end, n0, n_end, a_row);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0};

    Regs r;
    fetch(r, pl, 0);
    store(sm.st[0], r, bt);
    __syncthreads();
    const int64_t nslab = K / BK;
    for (int64_t s = 0; s < nslab; ++s) {
        const bool more = s + 1 < nslab;
        if (more) fetch(r, pl, (s + 1) * BK);
        compute(sm.st[s & 1], acc, bt, wm, wn, lane);
        if (more) store(sm.st[(s + 1) & 1], r, bt);
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane holds column lane % 32 and rows
    // 8 * (v / 4) + 4 * (lane / 32) + v % 4.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
            if (n >= n_end) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < m_end) {
                    const float y = acc[i][j][v] * out_scale;
                    if (BF16_OUT)
                        reinterpret_cast<uint16_t *>(C)[m * ldc + n] = (uint16_t)f32_to_bf16(y);
                    else
                        reinterpret_cast<float *>(C)[m * ldc + n] = y;
                }
            }
        }
}

}  // namespace big

template <bool BF16_OUT>
__global__ __launch_bounds__(big::NT) void nvfp4_gemm_big_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    big::Smem &sm = *reinterpret_cast<big::Smem *>(smem_raw);
    const int64_t tm = (p.M + big::BM - 1) / big::BM, tn = (p.N + big::BN - 1) / big::BN;
    const int64_t T = tm * tn;
    // XCD-contiguous tile ranges
    const int64_t bid = blockIdx.x, x = bid % 8, j = bid / 8;
    const int64_t per = T / 8, rem = T % 8;
    const int64_t tid = x * per + (x < rem ? x : rem) + j;
    // grouped order: GROUP_M tiles down M, then along N
    const int64_t gsize = big::GROUP_M * tn;
    const int64_t g = tid / gsize, in = tid - g * gsize;
    const int64_t gm = (tm - g * big::GROUP_M) < big::GROUP_M ? (tm - g * big::GROUP_M) : big::GROUP_M;
    const int64_t mt = g * big::GROUP_M + in % gm, nt = in / gm;
    const float out_scale = p.a.s_dec[0] * p.b.s_dec[0];
    big::tile<BF16_OUT>(sm, p.a, p.b, p.K, mt * big::BM, p.M, nt * big::BN, p.N,
                        [](int64_t r) { return r; }, out_scale, p.c, p.ldc);
}

constexpr int kMaxGroupsBig = 1024;

template <bool BF16_OUT>
__global__ __launch_bounds__(big::NT) void grouped_nvfp4_gemm_big_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    big::Smem &sm = *reinterpret_cast<big::Smem *>(smem_raw);
    __shared__ int64_t tile_start[kMaxGroupsBig + 1];
    __shared__ int64_t row_start[kMaxGroupsBig + 1];
    const int64_t n_tiles_n = (p.N + big::BN - 1) / big::BN;
    if (threadIdx.x == 0) {
        int64_t acc = 0, prev = 0;
        for (int g = 0; g <= p.G; ++g) {
            int64_t off = p.group_offsets[g];
            off = off < prev ? prev : off;
            off = off > p.max_rows ? p.max_rows : off;
            row_start[g] = off;
            if (g > 0) acc += ((off - prev + big::BM - 1) / big::BM) * n_tiles_n;
            tile_start[g] = acc;
            prev = off;
        }
    }
    __syncthreads();
    const int64_t total = tile_start[p.G];
    for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
        int g = 0;
        while (g + 1 < p.G && tile_start[g + 1] <= tile) ++g;
        const int64_t local = tile - tile_start[g];
        const int64_t mt = local / n_tiles_n, nt = local - mt * n_tiles_n;
        const int64_t re = row_start[g + 1];
        const int64_t m0 = row_start[g] + mt * big::BM, n0 = nt * big::BN;
        Fp4View B = p.b;
        B.codes = p.b.codes + (int64_t)g * p.N * (p.K / 2);
        B.scales = p.b.scales + (int64_t)g * (B.tile2d ? (p.N / 16) : p.N) * (p.K / 16);
        const float out_scale = p.a.s_dec[0] * p.b.s_dec[g];
        const int32_t *ri = p.row_index;
        const int64_t src_rows = p.a_src_rows;
        big::tile<BF16_OUT>(
            sm, p.a, B, p.K, m0, re, n0, p.N,
            [ri, src_rows](int64_t r) -> int64_t {
                const int64_t s = ri ? (int64_t)ri[r] : r;
                return (s >= 0 && s < src_rows) ? s : -1;
            },
            out_scale, p.c, p.ldc);
        __syncthreads();
    }
}

hipError_t launch_nvfp4_gemm_big(const GemmParams &p, bool bf16_out, hipStream_t s) {
    const int64_t T = ((p.M + big::BM - 1) / big::BM) * ((p.N + big::BN - 1) / big::BN);
    const size_t shm = sizeof(big::Smem);
    if (bf16_out) {
        hipFuncSetAttribute(reinterpret_cast<const void *>(nvfp4_gemm_big_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        hipLaunchKernelGGL(nvfp4_gemm_big_kernel<true>, dim3((unsigned)T), dim3(big::NT), shm, s, p);
    } else {
        hipFuncSetAttribute(reinterpret_cast<const void *>(nvfp4_gemm_big_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        hipLaunchKernelGGL(nvfp4_gemm_big_kernel<false>, dim3((unsigned)T), dim3(big::NT), shm, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_grouped_nvfp4_gemm_big(const GemmParams &p, bool bf16_out, hipStream_t s) {
    if (p.G > kMaxGroupsBig) return hipErrorInvalidValue;
    const size_t shm = sizeof(big::Smem);
    const dim3 grid(512);
    if (bf16_out) {
        hipFuncSetAttribute(reinterpret_cast<const void *>(grouped_nvfp4_gemm_big_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        hipLaunchKernelGGL(grouped_nvfp4_gemm_big_kernel<true>, grid, dim3(big::NT), shm, s, p);
    } else {
        hipFuncSetAttribute(reinterpret_cast<const void *>(grouped_nvfp4_gemm_big_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        hipLaunchKernelGGL(grouped_nvfp4_gemm_big_kernel<false>, grid, dim3(big::NT), shm, s, p);
    }
    return hipGetLastError();
}

}  // namespace bbs

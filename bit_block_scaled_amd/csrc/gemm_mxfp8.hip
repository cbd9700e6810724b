// MXFP8 x MXFP8 GEMM, large-tile kernel for K % 128 == 0 (gfx950).
//
// C = sum over 32-blocks b of 2^(sa_b - 127) * 2^(sb_b - 127) * sum_{k in b}
// a_k b_k with E4M3 elements (the dgrad GEMM of the backward pass,
// 4bit.vizuara.ai sections 9-10).  This maps exactly onto
// v_mfma_scale_f32_16x16x128_f8f6f4: FP8 (E4M3) operands, one E8M0 scale per
// 32 K-values and row / column.
//
// A workgroup (4 waves, 2 x 2) owns a 256 x 256 tile of C; a wave owns
// 128 x 128 = 8 x 8 MFMAs (256 FP32 accumulators per lane).  K advances in
// slabs of 128 (one MFMA deep), double-buffered in LDS.  Slabs are copied
// global -> LDS with global_load_lds_dwordx4 (no staging registers): each
// instruction fills 1 KB of LDS, 16 bytes per lane in lane order, so a wave
// writes 8 rows of 128 bytes per instruction.  Within a row the 16-byte chunk
// c is stored at position c ^ ((row >> 1) & 7): the 16 rows that one fragment
// read touches then fall on 16 distinct bank groups.
//
// Operand layout of the MFMA (measured): lane l holds row l % 16; its bytes
// 0-15 are K = 16g .. 16g+15 and bytes 16-31 are K = 64+16g .. 64+16g+15,
// g = l / 16; the scale of block b comes from byte 0 of lane group b's scale
// operand.  So lane group g reads chunks g and 4 + g of its row and supplies
// the scale of the slab's block g.
#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

namespace mx {

constexpr int BM = 256, BN = 256, BK = 128, NT = 256;
constexpr int GROUP_M = 8;

struct Stage {
    uint8_t a[BM * BK];
    uint8_t b[BN * BK];
    uint32_t as[BM];              // 4 E8M0 bytes (the slab's 4 blocks) per row
    uint32_t bs[BN];
};
struct Smem {
    Stage st[2];
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Per-lane source offsets (bytes, relative to the tile's first row) of the
// eight 1 KB copies of each operand, and of the scale row.  Rows past M (N)
// are clamped to the last valid row: they only feed outputs that are never
// written.
struct Plan {
    const uint8_t *a_base, *b_base, *sa_base, *sb_base;
    uint32_t a_off[8], b_off[8];
    uint32_t sa_off, sb_off;
};

__device__ __forceinline__ Plan make_plan(const Mx8GemmParams &p, int64_t m0, int64_t n0) {
    Plan pl;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    pl.a_base = p.a_codes + m0 * p.K;
    pl.b_base = p.b_codes + n0 * p.K;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = (w * 8 + q) * 8 + (lane >> 3);     // tile row this lane fills
        const int pos = lane & 7;                          // LDS chunk position
        const int c = swz(row, pos);                       // global chunk stored there
        const int64_t am = min(m0 + row, p.M - 1) - m0, bn = min(n0 + row, p.N - 1) - n0;
        pl.a_off[q] = (uint32_t)(am * p.K + 16 * c);
        pl.b_off[q] = (uint32_t)(bn * p.K + 16 * c);
    }
    const int64_t nkb = p.K / 32;
    pl.sa_base = p.a_scales + m0 * nkb;
    pl.sb_base = p.b_scales + n0 * nkb;
    pl.sa_off = (uint32_t)((min(m0 + t, p.M - 1) - m0) * nkb);
    pl.sb_off = (uint32_t)((min(n0 + t, p.N - 1) - n0) * nkb);
    return pl;
}

// Enqueue the copies of one slab into one LDS stage (asynchronous).
__device__ __forceinline__ void issue(Stage &st, const Plan &pl, int64_t k0) {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int seg = (w * 8 + q) * 1024;
        copy_lds16(pl.a_base + k0 + pl.a_off[q], st.a + seg);
        copy_lds16(pl.b_base + k0 + pl.b_off[q], st.b + seg);
    }
    copy_lds4(pl.sa_base + k0 / 32 + pl.sa_off, st.as + w * 64);
    copy_lds4(pl.sb_base + k0 / 32 + pl.sb_off, st.bs + w * 64);
}

__device__ __forceinline__ i32x8 frag(const uint8_t *tile, int r, int g) {
    const uint8_t *row = tile + r * BK;
    const uint4 x0 = *reinterpret_cast<const uint4 *>(row + 16 * swz(r, g));
    const uint4 x1 = *reinterpret_cast<const uint4 *>(row + 16 * swz(r, 4 + g));
    return i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                 (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// The MFMAs of one slab.  The copies of the next slab into stage nx are
// issued along the way, four 1 KB copies after each of the first four row
// blocks' MFMAs (and the scale copies after the fourth): the wave never
// waits on one long burst of copy issues, and the copies still have half a
// slab of MFMAs to land in.
__device__ __forceinline__ void compute(const Stage &st, f32x4 (&acc)[8][8], int wm, int wn,
                                        int lane, Stage &nx, const Plan &pl, int64_t kn) {
    const int w = threadIdx.x >> 6;
    const int g = lane >> 4, rl = lane & 15;
    i32x8 bf[8];
    int bsc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = wn * 128 + j * 16 + rl;
        bf[j] = frag(st.b, r, g);
        bsc[j] = (int)((st.bs[r] >> (8 * g)) & 0xFFu);
    }
    // A fragments are double-buffered by hand: row block i + 1 is read while
    // the MFMAs of row block i run; the scheduling barrier keeps the compiler
    // from hoisting every fragment read at once.
    int r0 = wm * 128 + rl;
    i32x8 an = frag(st.a, r0, g);
    int ans = (int)((st.as[r0] >> (8 * g)) & 0xFFu);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const i32x8 af = an;
        const int asc = ans;
        if (i + 1 < 8) {
            const int r = wm * 128 + (i + 1) * 16 + rl;
            an = frag(st.a, r, g);
            ans = (int)((st.as[r] >> (8 * g)) & 0xFFu);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0,
                                                                         bsc[j], 0, asc);
        if (i < 4) {
#pragma unroll
            for (int q = 2 * i; q < 2 * i + 2; ++q) {
                copy_lds16(pl.a_base + kn + pl.a_off[q], nx.a + (w * 8 + q) * 1024);
                copy_lds16(pl.b_base + kn + pl.b_off[q], nx.b + (w * 8 + q) * 1024);
            }
        }
        if (i == 3) {
            copy_lds4(pl.sa_base + kn / 32 + pl.sa_off, nx.as + w * 64);
            copy_lds4(pl.sb_base + kn / 32 + pl.sb_off, nx.bs + w * 64);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace mx

template <bool BF16_OUT>
__global__ __launch_bounds__(mx::NT) void mxfp8_gemm_big_kernel(Mx8GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    mx::Smem &sm = *reinterpret_cast<mx::Smem *>(smem_raw);
    const int64_t tm = (p.M + mx::BM - 1) / mx::BM, tn = (p.N + mx::BN - 1) / mx::BN;
    const int64_t T = tm * tn;
    const int64_t bid = blockIdx.x, x = bid % 8, j = bid / 8;
    const int64_t per = T / 8, rem = T % 8;
    const int64_t tid = x * per + (x < rem ? x : rem) + j;
    const int64_t gsize = mx::GROUP_M * tn;
    const int64_t g = tid / gsize, in = tid - g * gsize;
    const int64_t gm = (tm - g * mx::GROUP_M) < mx::GROUP_M ? (tm - g * mx::GROUP_M) : mx::GROUP_M;
    const int64_t m0 = (g * mx::GROUP_M + in % gm) * mx::BM, n0 = (in / gm) * mx::BN;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const mx::Plan pl = mx::make_plan(p, m0, n0);

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[i][jj] = f32x4{0, 0, 0, 0};

    mx::issue(sm.st[0], pl, 0);
    __builtin_amdgcn_s_waitcnt(0x3F70);               // vmcnt(0)
    __syncthreads();
    const int64_t nslab = p.K / mx::BK;
    for (int64_t s = 0; s < nslab; ++s) {
        // slab s + 1 goes to the other stage (past the end the last slab is
        // copied again into the stage nobody reads any more: no branch)
        const int64_t kn = (s + 1 < nslab ? s + 1 : s) * mx::BK;
        mx::compute(sm.st[s & 1], acc, wm, wn, lane, sm.st[(s + 1) & 1], pl, kn);
        __builtin_amdgcn_s_waitcnt(0x3F70);           // the next slab's copies have landed
        __syncthreads();
    }

    // The MFMAs take the B fragment first, so block (i, jj) holds the
    // transposed 16 x 16 product: lane l has output row l % 16 and columns
    // 4 * (l / 16) + v, four consecutive columns stored at once.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t m = m0 + wm * 128 + i * 16 + (lane & 15);
        if (m >= p.M) continue;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int64_t n = n0 + wn * 128 + jj * 16 + 4 * (lane >> 4);
            if (n >= p.N) continue;
            const f32x4 y = acc[i][jj];
            if (BF16_OUT) {
                const uint2 w = make_uint2(f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16),
                                           f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16));
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.c) + m * p.ldc + n) = w;
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.c) + m * p.ldc + n) =
                    make_float4(y[0], y[1], y[2], y[3]);
            }
        }
    }
}

hipError_t launch_mxfp8_gemm_big(const Mx8GemmParams &p, bool bf16_out, hipStream_t s) {
    const int64_t T = ((p.M + mx::BM - 1) / mx::BM) * ((p.N + mx::BN - 1) / mx::BN);
    const size_t shm = sizeof(mx::Smem);
    if (bf16_out) {
        hipFuncSetAttribute(reinterpret_cast<const void *>(mxfp8_gemm_big_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        hipLaunchKernelGGL(mxfp8_gemm_big_kernel<true>, dim3((unsigned)T), dim3(mx::NT), shm, s, p);
    } else {
        hipFuncSetAttribute(reinterpret_cast<const void *>(mxfp8_gemm_big_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        hipLaunchKernelGGL(mxfp8_gemm_big_kernel<false>, dim3((unsigned)T), dim3(mx::NT), shm, s, p);
    }
    return hipGetLastError();
}

}  // namespace bbs

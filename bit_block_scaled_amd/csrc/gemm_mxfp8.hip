// MXFP8 x MXFP8 GEMM, large-tile kernel for K % 128 == 0, and MXFP4 x MXFP4
// for K % 256 == 0 (gfx950).
//
// C = sum over 32-blocks b of 2^(sa_b - 127) * 2^(sb_b - 127) * sum_{k in b}
// a_k b_k with E4M3 elements (the dgrad GEMM of the backward pass,
// 4bit.vizuara.ai sections 9-10).  This maps exactly onto
// v_mfma_scale_f32_16x16x128_f8f6f4: FP8 (E4M3) operands, one E8M0 scale per
// 32 K-values and row / column.
//
// A workgroup (4 waves, 2 x 2) owns a 256 x 256 tile of C; a wave owns
// 128 x 128 = 8 x 8 MFMAs (256 FP32 accumulators per lane).  K advances in
// slabs of 128 (one MFMA deep) through two LDS stages (a slab is 66 KB, so
// no third fits); each wave holds all of a slab's fragments in registers,
// read two MFMA shells ahead of their use, which frees the stage after one
// barrier and lets the copies of the slab two ahead go into it.  Slabs are
// copied global -> LDS with global_load_lds_dwordx4 (no staging registers):
// each instruction fills 1 KB of LDS, 16 bytes per lane in lane order, so a
// wave writes 8 rows of 128 bytes per instruction.  Within a row the 16-byte chunk
// c is stored at position c ^ ((row >> 1) & 7): the 16 rows that one fragment
// read touches then fall on 16 distinct bank groups.
//
// Operand layout of the MFMA (measured): lane l holds row l % 16; its bytes
// 0-15 are K = 16g .. 16g+15 and bytes 16-31 are K = 64+16g .. 64+16g+15,
// g = l / 16; the scale of block b comes from byte 0 of lane group b's scale
// operand.  So lane group g reads chunks g and 4 + g of its row and supplies
// the scale of the slab's block g.
//
// The same tiles, LDS ring and copy plan run MXFP4 x MXFP4 (FP4 Training on
// Blackwell, 'The scaling math, worked'; the OCP format with E2M1 elements)
// on v_mfma_scale_f32_32x32x64_f8f6f4 with operand format 4, where lane l's
// first 16 bytes hold the 32 values of block l / 32 of row l % 32
// (measured).  A slab is still 128 bytes of every row, now 256 K-values: four
// 64-value MFMA steps, with 8 scale bytes per row.
#include <type_traits>

#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;
namespace mx {

constexpr int BM = 256, BN = 256, BK = 128, NT = 256;
constexpr int GROUP_M = 8;

// BK is in bytes of a row: 128 FP8 values or 256 FP4 values per slab.
template <bool FP4>
struct Stage {
    uint8_t a[BM * BK];
    uint8_t b[BN * BK];
    uint32_t as[FP4 ? 2 : 1][BM];   // the slab's E8M0 bytes per row: 4 (FP8) or 8 (FP4)
    uint32_t bs[FP4 ? 2 : 1][BN];
};
template <bool FP4>
struct Smem {
    Stage<FP4> st[2];
};

// Scale bytes (= 32-blocks) per row in one slab.
template <bool FP4>
constexpr int slab_blocks() { return FP4 ? 8 : 4; }

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

template <bool FP4>
__device__ __forceinline__ Plan make_plan(const Mx8GemmParams &p, int64_t m0, int64_t n0) {
    Plan pl;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t rb = FP4 ? p.K / 2 : p.K;            // bytes per row
    pl.a_base = p.a_codes + m0 * rb;
    pl.b_base = p.b_codes + n0 * rb;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = (w * 8 + q) * 8 + (lane >> 3);     // tile row this lane fills
        const int pos = lane & 7;                          // LDS chunk position
        const int c = swz(row, pos);                       // global chunk stored there
        const int64_t am = min(m0 + row, p.M - 1) - m0, bn = min(n0 + row, p.N - 1) - n0;
        pl.a_off[q] = (uint32_t)(am * rb + 16 * c);
        pl.b_off[q] = (uint32_t)(bn * rb + 16 * c);
    }
    const int64_t nkb = p.K / 32;
    pl.sa_base = p.a_scales + m0 * nkb;
    pl.sb_base = p.b_scales + n0 * nkb;
    // FP8: LDS word t holds the scales of row 128 (t / 128) + 16 k + rl with
    // rl = (t / 8) % 16 and k = (t % 8) ^ (4 (rl / 8)), so the eight rows
    // rl + 16 k of a lane's half are adjacent, their halves swapped for
    // rl >= 8 (lanes rl and rl + 8 then read different banks)
    const int s_rl = (t >> 3) & 15;
    const int srow = FP4 ? t : (t >> 7) * 128 + ((t & 7) ^ ((s_rl >> 3) << 2)) * 16 + s_rl;
    pl.sa_off = (uint32_t)((min(m0 + srow, p.M - 1) - m0) * nkb);
    pl.sb_off = (uint32_t)((min(n0 + srow, p.N - 1) - n0) * nkb);
    return pl;
}

// The scale copies of slab s (4 bytes per row per copy).
template <bool FP4>
__device__ __forceinline__ void issue_scales(Stage<FP4> &st, const Plan &pl, int64_t s) {
    const int w = threadIdx.x >> 6;
    const int64_t blk = s * slab_blocks<FP4>();
#pragma unroll
    for (int h = 0; h < (FP4 ? 2 : 1); ++h) {
        copy_lds4(pl.sa_base + blk + 4 * h + pl.sa_off, st.as[h] + w * 64);
        copy_lds4(pl.sb_base + blk + 4 * h + pl.sb_off, st.bs[h] + w * 64);
    }
}

// Enqueue the copies of slab s into one LDS stage (asynchronous).
template <bool FP4>
__device__ __forceinline__ void issue(Stage<FP4> &st, const Plan &pl, int64_t s) {
    const int w = threadIdx.x >> 6;
    const int64_t k0 = s * BK;                          // byte offset in a row
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int seg = (w * 8 + q) * 1024;
        copy_lds16(pl.a_base + k0 + pl.a_off[q], st.a + seg);
        copy_lds16(pl.b_base + k0 + pl.b_off[q], st.b + seg);
    }
    issue_scales(st, pl, s);
}

// One 16-byte chunk c of row r (FP4: the 32 values of one block); the upper
// half of the operand is not read by the instruction.
__device__ __forceinline__ i32x8 frag4(const uint8_t *tile, int r, int c) {
    const uint4 x = *reinterpret_cast<const uint4 *>(tile + r * BK + 16 * swz(r, c));
    return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
}

__device__ __forceinline__ i32x8 frag(const uint8_t *tile, int r, int g) {
    const uint8_t *row = tile + r * BK;
    const uint4 x0 = *reinterpret_cast<const uint4 *>(row + 16 * swz(r, g));
    const uint4 x1 = *reinterpret_cast<const uint4 *>(row + 16 * swz(r, 4 + g));
    return i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                 (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// s_waitcnt vmcnt(n), other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | (((N >> 4) & 3) << 14));
}

// Copies one wave issues per FP8 slab: 8 + 8 code copies, 2 scale copies.
constexpr int kIssued8 = 18;

// The MFMAs of one FP8 slab (8 A + 8 B fragments, 128 VGPRs).  The MFMAs
// run in growing squares (shell k = the blocks that need fragments k and
// below), and the fragment reads go two shells ahead of the MFMAs that use
// them, so a shell waits only for the reads issued before the previous
// shell's, not for all 20 of the slab (the LDS wait counter tracks at most
// 15, and with more in flight the compiler waits for all).  After shell 5 the
// wave's reads are all issued; after one barrier at shell 6 the stage is free
// and the copies of slab sn (two slabs ahead) go into it during shells 6-7:
// they get most of two slabs to land, where copying into the other stage of a
// two-stage ring gives them one.
__device__ __forceinline__ void compute_held(Stage<false> &st, f32x4 (&acc)[8][8], int wm,
                                             int wn, int lane, const Plan &pl, int64_t sn) {
    const int w = threadIdx.x >> 6;
    const int g = lane >> 4, rl = lane & 15;
    const int64_t kn = sn * BK;
    i32x8 af[8], bf[8];
    // the lane's eight scale words per operand, adjacent in the stage (rows
    // rl + 16 k for k = 0-3 in one half, 4-7 in the other: swapped for rl >= 8)
    const int h0 = rl * 8 + ((rl >> 3) << 2), h1 = rl * 8 + 4 - ((rl >> 3) << 2);
    const uint4 sa0 = *reinterpret_cast<const uint4 *>(&st.as[0][wm * 128 + h0]);
    const uint4 sa1 = *reinterpret_cast<const uint4 *>(&st.as[0][wm * 128 + h1]);
    const uint4 sb0 = *reinterpret_cast<const uint4 *>(&st.bs[0][wn * 128 + h0]);
    const uint4 sb1 = *reinterpret_cast<const uint4 *>(&st.bs[0][wn * 128 + h1]);
    auto read = [&](int k) {
        af[k] = frag(st.a, wm * 128 + k * 16 + rl, g);
        bf[k] = frag(st.b, wn * 128 + k * 16 + rl, g);
    };
    read(0);
    read(1);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t saw[8] = {sa0.x, sa0.y, sa0.z, sa0.w, sa1.x, sa1.y, sa1.z, sa1.w};
    const uint32_t sbw[8] = {sb0.x, sb0.y, sb0.z, sb0.w, sb1.x, sb1.y, sb1.z, sb1.w};
    auto byte_of = [&](uint32_t v) { return (int)((v >> (8 * g)) & 0xFFu); };
    int c = 0;                                         // copies issued
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k + 2 < 8) {
            read(k + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (k == 6) {
            // every read of this wave is complete; once every wave's are,
            // nobody reads the stage again in this slab
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < 2 * k + 1; ++e) {
            const int i = e < k ? e : k, j = e < k ? k : e - k;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bf[j], af[i], acc[i][j], 0, 0, 0, byte_of(sbw[j]), 0, byte_of(saw[i]));
            // shell 6: a copy after every MFMA, shell 7 after every second
            // (A and B in turn), then the scale copies
            if (k == 6 || (k == 7 && (e & 1))) {
                if (c < 16) {
                    const int q = c >> 1;
                    if (c & 1) copy_lds16(pl.b_base + kn + pl.b_off[q], st.b + (w * 8 + q) * 1024);
                    else copy_lds16(pl.a_base + kn + pl.a_off[q], st.a + (w * 8 + q) * 1024);
                } else if (c == 16) {
                    issue_scales(st, pl, sn);
                }
                ++c;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// FP4 slabs on v_mfma_scale_f32_32x32x64_f8f6f4, the full-rate form for
// E2M1 operands (the 16 x 16 x 128 form issues E2M1 at about half its rate,
// measured): lane l feeds row l % 32 and block l / 32 of a 64-value step (its
// 16 bytes of the row's chunk 2 * ks + l / 32), with that block's scale.  A
// wave's 128 x 128 tile is 4 x 4 MFMA blocks of 32 x 32; a slab is 4 steps.

// Copies one wave issues per FP4 slab: 8 + 8 code copies, 4 scale copies.
constexpr int kIssued4 = 20;

// The FP4 slab with every fragment held in registers, as compute_held: the
// 16 code chunks (4 steps x (4 A + 4 B) x 16 bytes, 128 VGPRs) and the
// slab's scale words are read at its start; after step 0's row block 1 the
// stage is free and the copies of slab sn go into it.  An MFMA operand is
// the chunk in the low half of eight registers (the instruction reads only
// those 16 bytes for E2M1).
__device__ __forceinline__ void compute4_held(Stage<true> &st, f32x16 (&acc)[4][4], int wm,
                                              int wn, int lane, const Plan &pl, int64_t sn) {
    const int w = threadIdx.x >> 6;
    const int h = lane >> 5, rl = lane & 31;
    const int64_t kn = sn * BK;
    uint4 ad[4][4], bd[4][4];                      // [step][row block]
    uint32_t as0[4], as1[4], bs0[4], bs1[4];       // the slab's 8 scale bytes per row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + rl;
        as0[i] = st.as[0][r];
        as1[i] = st.as[1][r];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + rl;
        bs0[j] = st.bs[0][r];
        bs1[j] = st.bs[1][r];
    }
    // the chunks in step order (each step's MFMAs then wait only for their
    // own reads and those before)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int c = 2 * ks + h;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn * 128 + j * 32 + rl;
            bd[ks][j] = *reinterpret_cast<const uint4 *>(st.b + r * BK + 16 * swz(r, c));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + rl;
            ad[ks][i] = *reinterpret_cast<const uint4 *>(st.a + r * BK + 16 * swz(r, c));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int c = 2 * ks + h;                      // the lane's 16-byte chunk
        const int sh = 8 * (c & 3);                    // its scale byte within the word
        i32x8 bf[4];
        int bsc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 x = bd[ks][j];
            bf[j] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
            bsc[j] = (int)((((c >> 2) ? bs1[j] : bs0[j]) >> sh) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 x = ad[ks][i];
            const i32x8 af = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
            const int asc = (int)((((c >> 2) ? as1[i] : as0[i]) >> sh) & 0xFFu);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af, acc[i][j], 4, 4,
                                                                            0, bsc[j], 0, asc);
            const int slot = ks * 4 + i;
            if (slot == 1) {
                // this wave's reads are complete; once every wave's are, the
                // stage is free for the copies of slab sn
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __syncthreads();
            }
            if (slot >= 2 && slot < 10) {
                const int q = slot - 2;
                copy_lds16(pl.a_base + kn + pl.a_off[q], st.a + (w * 8 + q) * 1024);
                copy_lds16(pl.b_base + kn + pl.b_off[q], st.b + (w * 8 + q) * 1024);
            }
            if (slot == 9) issue_scales(st, pl, sn);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace mx

template <bool FP4, bool BF16_OUT>
__device__ __forceinline__ void mx_gemm_big(const Mx8GemmParams &p, uint8_t *smem_raw) {
    mx::Smem<FP4> &sm = *reinterpret_cast<mx::Smem<FP4> *>(smem_raw);
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
    const mx::Plan pl = mx::make_plan<FP4>(p, m0, n0);

    // FP8: 8 x 8 blocks of 16 x 16; FP4: 4 x 4 blocks of 32 x 32 (256 FP32 each)
    typedef std::conditional_t<FP4, f32x16[4][4], f32x4[8][8]> Acc;
    Acc acc;
    if constexpr (FP4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f32x16{0};
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) acc[i][jj] = f32x4{0, 0, 0, 0};
    }

    const int64_t nslab = p.K / (FP4 ? 2 * mx::BK : mx::BK);
    if constexpr (!FP4) {
        // Slab s lives in stage s % 2 and is copied while slab s - 2 is
        // multiplied (compute_held); past the end the last slab is copied
        // again into the freed stage, which keeps the loop free of branches.
        mx::issue(sm.st[0], pl, 0);
        mx::issue(sm.st[1], pl, nslab > 1 ? 1 : 0);
        mx::wait_vmcnt<mx::kIssued8>();                // slab 0 has landed
        __syncthreads();
        // no scalar load in flight into the loop: with one pending the LDS
        // counter is out of order and every fragment wait becomes lgkmcnt(0)
        // (the epilogue's arguments are loaded here, not under the loop)
        asm volatile("" ::"s"(p.c), "s"(p.ldc), "s"(p.M), "s"(p.N));
        __builtin_amdgcn_s_waitcnt(0xC07F);
        for (int64_t s = 0; s < nslab; ++s) {
            const int64_t sn = s + 2 < nslab ? s + 2 : nslab - 1;
            mx::compute_held(sm.st[s & 1], acc, wm, wn, lane, pl, sn);
            mx::wait_vmcnt<mx::kIssued8>();            // slab s + 1 has landed
            __syncthreads();
        }
        mx::wait_vmcnt<0>();
    }
    if constexpr (FP4) {
        // the same two-stage schedule for FP4 slabs
        mx::issue(sm.st[0], pl, 0);
        mx::issue(sm.st[1], pl, nslab > 1 ? 1 : 0);
        mx::wait_vmcnt<mx::kIssued4>();                // slab 0 has landed
        __syncthreads();
        asm volatile("" ::"s"(p.c), "s"(p.ldc), "s"(p.M), "s"(p.N));
        __builtin_amdgcn_s_waitcnt(0xC07F);           // as for FP8
        for (int64_t s = 0; s < nslab; ++s) {
            const int64_t sn = s + 2 < nslab ? s + 2 : nslab - 1;
            mx::compute4_held(sm.st[s & 1], acc, wm, wn, lane, pl, sn);
            mx::wait_vmcnt<mx::kIssued4>();            // slab s + 1 has landed
            __syncthreads();
        }
        mx::wait_vmcnt<0>();
    }

    auto store4 = [&](int64_t m, int64_t n, float y0, float y1, float y2, float y3) {
        if (BF16_OUT) {
            const uint2 w = make_uint2(pk_bf16(y0, y1), pk_bf16(y2, y3));
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.c) + m * p.ldc + n) = w;
        } else {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.c) + m * p.ldc + n) =
                make_float4(y0, y1, y2, y3);
        }
    };
    if constexpr (FP4) {
        // block (i, jj) holds the transposed 32 x 32 product: lane l has output
        // row l % 32 and columns 8 * (v / 4) + 4 * (l / 32) + v % 4
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
            if (m >= p.M) continue;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int64_t n = n0 + wn * 128 + jj * 32 + 8 * gq + 4 * (lane >> 5);
                    if (n >= p.N) continue;
                    const f32x16 &y = acc[i][jj];
                    store4(m, n, y[4 * gq], y[4 * gq + 1], y[4 * gq + 2], y[4 * gq + 3]);
                }
        }
        return;
    } else {
    // The MFMAs take the B fragment first, so block (i, jj) holds the
    // transposed 16 x 16 product: lane l has output row l % 16 and columns
    // 4 * (l / 16) + v, four consecutive columns stored at once.  A tile
    // wholly inside C stores without bounds tests, each row block from one
    // address (the column blocks at immediate offsets).
    const int64_t nl = n0 + wn * 128 + 4 * (lane >> 4);       // column of block 0
    auto row_blocks = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t m = m0 + wm * 128 + i * 16 + (lane & 15);
            if (!FULL && m >= p.M) continue;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                if (!FULL && nl + jj * 16 >= p.N) continue;
                const f32x4 y = acc[i][jj];
                if (BF16_OUT) {
                    uint16_t *row = reinterpret_cast<uint16_t *>(p.c) + m * p.ldc + nl;
                    *reinterpret_cast<uint2 *>(row + jj * 16) =
                        make_uint2(pk_bf16(y[0], y[1]), pk_bf16(y[2], y[3]));
                } else {
                    float *row = reinterpret_cast<float *>(p.c) + m * p.ldc + nl;
                    *reinterpret_cast<float4 *>(row + jj * 16) = make_float4(y[0], y[1], y[2], y[3]);
                }
            }
        }
    };
    if (m0 + mx::BM <= p.M && n0 + mx::BN <= p.N) row_blocks(std::true_type{});
    else row_blocks(std::false_type{});
    }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(mx::NT) void mxfp8_gemm_big_kernel(Mx8GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    mx_gemm_big<false, BF16_OUT>(p, smem_raw);
}

template <bool BF16_OUT>
__global__ __launch_bounds__(mx::NT) void mxfp4_gemm_big_kernel(Mx8GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    mx_gemm_big<true, BF16_OUT>(p, smem_raw);
}

// The kernel's dynamic LDS limit is raised once per kernel (thread-safe
// static initialisation).
template <auto Kernel>
static void launch_big(size_t shm, const Mx8GemmParams &p, hipStream_t s) {
    const int64_t T = ((p.M + mx::BM - 1) / mx::BM) * ((p.N + mx::BN - 1) / mx::BN);
    static const bool attr_set = [shm] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(Kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        return true;
    }();
    (void)attr_set;
    hipLaunchKernelGGL(Kernel, dim3((unsigned)T), dim3(mx::NT), shm, s, p);
}

hipError_t launch_mxfp8_gemm_big(const Mx8GemmParams &p, bool bf16_out, hipStream_t s) {
    const size_t shm = sizeof(mx::Smem<false>);
    if (bf16_out) launch_big<mxfp8_gemm_big_kernel<true>>(shm, p, s);
    else launch_big<mxfp8_gemm_big_kernel<false>>(shm, p, s);
    return hipGetLastError();
}

hipError_t launch_mxfp4_gemm(const Mx8GemmParams &p, bool bf16_out, hipStream_t s) {
    const size_t shm = sizeof(mx::Smem<true>);
    if (bf16_out) launch_big<mxfp4_gemm_big_kernel<true>>(shm, p, s);
    else launch_big<mxfp4_gemm_big_kernel<false>>(shm, p, s);
    return hipGetLastError();
}

}  // namespace bbs

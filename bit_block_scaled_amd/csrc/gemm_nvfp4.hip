// NVFP4 x NVFP4 GEMM, large-tile kernel for K % 128 == 0 (gfx950).
//
// C = s_dec,A * s_dec,B * sum_b E4M3_A,b * E4M3_B,b * sum_{k in b} a_k b_k
// (Pretraining LLMs with NVFP4, "NVFP4 Format and Quantization Procedure",
// step 5), FP32 accumulation.
//
// Tiling: a workgroup (4 waves, 2 x 2) owns a 256 x 256 tile of C; each wave
// owns 128 x 128 = 4 x 4 v_mfma_f32_32x32x16_f16 accumulators (256 FP32 per
// lane).  K advances in slabs of 128 (8 NVFP4 blocks).  Each slab is copied
// global -> LDS with global_load_lds (asynchronous, no staging registers) into
// one of three LDS stages (two slabs in flight ahead of the one consumed): the packed 4-bit codes exactly as stored in HBM (64
// bytes per row) and the raw E4M3 scale bytes (8 per row).
//
// Exact expansion: v_cvt_scalef32_pk_f16_fp4 (scale 1.0) turns two E2M1 codes
// into two FP16 values and one v_pk_mul_f16 applies the block scale, decoded
// to FP16 by v_cvt_scalef32_pk_f16_fp8 (two blocks per instruction).  code x scale
// has at most 6 significant bits and lies in [2^-10, 2688], so both steps are
// exact in FP16; the MFMA products are exact in FP32 and only the
// accumulation rounds.  The expansion of MFMA step s + 1 is interleaved with
// the MFMAs of step s.
//
// K order inside a slab: lane half h of an MFMA step takes 8 codes from the
// 16-byte group 2c + h of the row (c = 32-byte chunk, 4 steps per chunk), so
// one ds_read_b128 feeds four MFMA steps.  A and B use the same order, so the
// sum is unchanged; each lane's 8 codes always lie in one block.  In LDS the
// 16-byte group p of row r sits at position p ^ ((r >> 2) & 3), which puts the
// 16 rows of one fragment read on 16 distinct bank groups.
//
// Tile order is XCD-aware: workgroup i runs on XCD i % 8, so each XCD is given
// a contiguous range of tile ids, and ids walk 8 M-tiles down before moving
// along N, keeping operand panels shared inside one XCD's L2.  The kernels
// are persistent: one workgroup per CU takes its XCD's tiles in turn, and
// the slab ring runs on from one tile into the next (run_tiles).
#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

namespace big {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NT = 256;
constexpr int RB = BK / 2;        // code bytes per row and slab (64)
constexpr int SB = BK / 16;       // scale bytes per row and slab (8)
constexpr int GROUP_M = 8;

struct Stage {
    uint8_t a[BM * RB];
    uint8_t b[BN * RB];
    uint8_t as[BM * SB];
    uint8_t bs[BN * SB];
};
struct Smem {
    Stage st[3];
};

__device__ __forceinline__ int swz(int row, int pos) { return pos ^ ((row >> 2) & 3); }

// Eight E2M1 codes of one 32-bit word times one FP16 scale -> 8 FP16.
__device__ __forceinline__ f16x8 expand8_f16(uint32_t w, _Float16 scale) {
    const f16x2 s = {scale, scale};
    const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// Per-lane global sources of the copies of one slab (K offset added later).
// Rows past the operand's end are clamped to a valid row: they only feed
// outputs that are never written.
struct Plan {
    const uint8_t *a[4], *b[4];   // code copies: 16 rows x 64 bytes per instruction
    const uint8_t *sa[2], *sb[2]; // scale copies: 32 rows x 8 bytes per instruction
};

// The A rows one lane copies for a tile: 4 code rows, 2 scale rows (source
// rows after the row map; a row map miss reads row 0).
struct ARows {
    int32_t c[4], s[2];
};

template <typename RowMap>
__device__ __forceinline__ ARows a_rows(int64_t m0, int64_t m_end, RowMap a_row) {
    ARows ar;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    auto arow = [&](int r) -> int32_t {
        const int64_t m = min(m0 + r, m_end - 1);
        const int64_t s = a_row(m);
        return s < 0 ? 0 : (int32_t)s;
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) ar.c[q] = arow((w * 4 + q) * 16 + (lane >> 2));
#pragma unroll
    for (int q = 0; q < 2; ++q) ar.s[q] = arow((w * 2 + q) * 32 + (lane >> 1));
    return ar;
}

// NJ: 32-column blocks per wave (4: a 256 x 256 tile; 2: a 256 x 128 half
// tile, whose B side is 128 rows: NJ code copies and NJ / 2 scale copies
// per wave).
template <int NJ>
__device__ __forceinline__ Plan make_plan(const Fp4View &A, const Fp4View &B, int64_t K,
                                          const ARows &ar, int64_t n0, int64_t n_end) {
    Plan pl;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t kb = K / 2, ks = K / 16;
    auto brow = [&](int r) -> int64_t { return min(n0 + r, n_end - 1); };
    const int pos = swz(lane >> 2, lane & 3);     // (row >> 2) & 3 == (lane >> 4) & 3 here
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = (w * 4 + q) * 16 + (lane >> 2);
        pl.a[q] = A.codes + (int64_t)ar.c[q] * kb + 16 * pos;
    }
#pragma unroll
    for (int q = 0; q < NJ; ++q) {
        const int r = (w * NJ + q) * 16 + (lane >> 2);
        pl.b[q] = B.codes + brow(r) * kb + 16 * pos;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int64_t sa_row = A.tile2d ? ar.s[q] / 16 : ar.s[q];
        pl.sa[q] = A.scales + sa_row * ks + 4 * (lane & 1);
    }
    if (B.tile2d) {
        // 16 tile rows: lanes 0..31 (the upper lanes repeat them)
        const int tr = (lane >> 1) & 15;
        const int64_t n = min(n0 / 16 + tr, (n_end - 1) / 16);
        pl.sb[0] = pl.sb[1] = B.scales + n * ks + 4 * (lane & 1);
    } else {
#pragma unroll
        for (int q = 0; q < NJ / 2; ++q) {
            const int r = (w * (NJ / 2) + q) * 32 + (lane >> 1);
            pl.sb[q] = B.scales + brow(r) * ks + 4 * (lane & 1);
        }
    }
    return pl;
}

// The copies of one slab, in three parts that the main loop spreads over
// MFMA steps: 0 = A codes (4 instructions per wave), 1 = B codes (4),
// 2 = scales (2 + 2, or 2 + 1 when B has 16x16 tiles).
template <int PART, bool BT, int NJ>
__device__ __forceinline__ void issue_part(Stage &st, const Plan &pl, int64_t k0) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // LDS offsets in SGPRs
    const int64_t cb = k0 / 2, sk = k0 / 16;
    if (PART == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            copy_lds16(pl.a[q] + cb, st.a + (w * 4 + q) * 1024);
    } else if (PART == 1) {
#pragma unroll
        for (int q = 0; q < NJ; ++q)
            copy_lds16(pl.b[q] + cb, st.b + (w * NJ + q) * 1024);
    } else {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            copy_lds4(pl.sa[q] + sk, st.as + (w * 2 + q) * 256);
        if (!BT) {
#pragma unroll
            for (int q = 0; q < NJ / 2; ++q)
                copy_lds4(pl.sb[q] + sk, st.bs + (w * (NJ / 2) + q) * 256);
        } else {
            // the 16 tile rows (128 bytes); every wave writes the same bytes
            copy_lds4(pl.sb[0] + sk, st.bs);
        }
    }
}

template <bool BT, int NJ>
__device__ __forceinline__ void issue(Stage &st, const Plan &pl, int64_t k0) {
    issue_part<0, BT, NJ>(st, pl, k0);
    issue_part<1, BT, NJ>(st, pl, k0);
    issue_part<2, BT, NJ>(st, pl, k0);
}

// Code words of one 32-byte chunk of a slab for the wave's 4 + 4 fragment
// rows (16 bytes per lane each: four MFMA steps).
struct Chunk {
    uint4 ca[4], cb[4];
};

// FP16 block scales of one chunk: the two blocks of each fragment row that
// the lane's 16 code bytes span (steps 0-1 use the first, steps 2-3 the
// second).  v_cvt_scalef32_pk_f16_fp8 (scale 1.0) decodes two E4M3 bytes at
// once, exactly (every E4M3 value is a normal FP16 number).
struct Pairs {
    f16x2 pa[4], pb[4];
};

template <int NJ>
__device__ __forceinline__ void load_chunk(Chunk &c, const Stage &st, int chunk, int wm, int wn,
                                           int lane) {
    const int h = lane >> 5, rl = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + rl;
        c.ca[i] = *reinterpret_cast<const uint4 *>(st.a + r * RB + 16 * swz(r, 2 * chunk + h));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = wn * NJ * 32 + j * 32 + rl;
        c.cb[j] = *reinterpret_cast<const uint4 *>(st.b + r * RB + 16 * swz(r, 2 * chunk + h));
    }
}

template <bool BT, int NJ>
__device__ __forceinline__ void load_scales(uint2 (&sca)[4], uint2 (&scb)[4], const Stage &st,
                                            int wm, int wn, int lane) {
    const int rl = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sca[i] = *reinterpret_cast<const uint2 *>(st.as + (wm * 128 + i * 32 + rl) * SB);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = wn * NJ * 32 + j * 32 + rl;
        scb[j] = *reinterpret_cast<const uint2 *>(st.bs + (BT ? (r >> 4) : r) * SB);
    }
}

template <int NJ>
__device__ __forceinline__ void load_pairs(Pairs &p, const uint2 (&sca)[4], const uint2 (&scb)[4],
                                           int chunk, int lane) {
    const int sh = 16 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        p.pa[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((chunk ? sca[i].y : sca[i].x) >> sh, 1.0f, false);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        p.pb[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((chunk ? scb[j].y : scb[j].x) >> sh, 1.0f, false);
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int s) {
    return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// Expanded operands of MFMA step s (0..3) of a chunk.
template <int NJ>
__device__ __forceinline__ void expand_step(f16x8 (&af)[4], f16x8 (&bf)[4], const Chunk &c,
                                            const Pairs &p, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = expand8_f16(word(c.ca[i], s), p.pa[i][s >> 1]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bf[j] = expand8_f16(word(c.cb[j], s), p.pb[j][s >> 1]);
}

template <int NJ>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[4][NJ], const f16x8 (&af)[4],
                                          const f16x8 (&bf)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
}

// Interleave: one MFMA, then four VALU, sixteen times.
__device__ __forceinline__ void interleave_1_4() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
}

// One MFMA, then one vector-memory instruction (the first N times), then
// four VALU, sixteen times: the slab copies issue under the MFMAs.
template <int N>
__device__ __forceinline__ void interleave_1_vmem_4() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k < N) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
}

// One MFMA, one LDS read, four VALU: the next slab's fragment reads issue
// early, under the MFMAs.
__device__ __forceinline__ void interleave_1_ds_4() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
}

// One MFMA step in four quarters, fenced from each other: quarter q expands
// operand pair q of the next step (A row block q, and B column block q when
// q < NJ: 16 or 8 VALU), issues the NJ MFMAs of row block q of this step
// (interleaved with that expansion) and then copy(q), a slab copy or
// nothing.  The fences keep each copy between MFMAs instead of letting the
// scheduler gather them into one burst that stalls the wave.
template <int NJ, typename Copy>
__device__ __forceinline__ void step_q(f32x16 (&acc)[4][NJ], const f16x8 (&af)[4],
                                       const f16x8 (&bf)[4], f16x8 (&an)[4], f16x8 (&bn)[4],
                                       const Chunk &c, const Pairs &p, int s, Copy copy) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        an[q] = expand8_f16(word(c.ca[q], s), p.pa[q][s >> 1]);
        if (q < NJ) bn[q] = expand8_f16(word(c.cb[q], s), p.pb[q][s >> 1]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[q][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[q], acc[q][j], 0, 0, 0);
        copy(q);
        // VALU after each MFMA: the quarter's 16 (q < NJ) or 8 spread evenly
        if (q < NJ) {
#pragma unroll
            for (int k = 0; k < NJ; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 16 / NJ, 0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NJ; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8 / NJ, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// s_waitcnt vmcnt(n), other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | (((N >> 4) & 3) << 14));
}

// Epilogue.  The MFMAs take the B fragment as their first operand, so block
// (i, j) of the accumulators holds the transposed 32 x 32 product: lane l has
// output row l % 32 and columns 8 * (v / 4) + 4 * (l / 32) + v % 4, i.e. each
// group of four registers is four consecutive columns of one row.  Each wave
// writes those groups (8 bytes of BF16, 16 of FP32) into its own staging rows
// in the ring stage the tile's last slab used (the next tile's first two
// slabs are meanwhile copied into the other two), then stores whole rows, 16
// bytes per lane, so
// every store instruction writes complete 256- or 512-byte row segments.
// Rows m < m_end and columns n < n_end are written; N being a multiple of 16
// keeps every 16-byte segment wholly in or out.
//
// Output modes: OUT_F32, OUT_BF16, and the quantizing modes OUT_Q / OUT_QG
// (4bit.vizuara.ai, section 13; End-to-End 4-Bit Training, kernels for
// low-precision training: the quantize rides in the GEMM's epilogue so the
// output never makes a round trip through memory).  These stage FP32 rows as
// OUT_BF16 does (the BF16 values the plain GEMM stores); on read-back each
// lane takes one 1x16 block of a row (16 consecutive values), applies GELU
// by the quantizers' table (OUT_QG; the workgroup copies it from
// q.gelu_tab to LDS past the ring once), and encodes the block with the given
// tensor scale exactly as the quantizer does: E4M3 block scale of
// (amax_b / 6) * s_enc (never below code 1), E2M1 codes of x * s_enc_b to
// nearest even.  The result is bit for bit the BF16 GEMM followed by the
// quantizer with that scale.  The largest |value| is folded into q.amax.
//
// OUT_S2F6 encodes the staged BF16 rows in the combine wire format instead
// (4bit.vizuara.ai, section 11; End-to-End 4-Bit Training, "quantized
// communication"): each lane takes 32 consecutive values of a row, rotates
// them by the 32-point RHT (q.rht) and stores the S2F6 codes and E8M0 scale,
// so the BF16 output of an expert never goes to memory.  Bit for bit the
// BF16 GEMM followed by the combine encode.
constexpr int OUT_F32 = 0, OUT_BF16 = 1, OUT_Q = 2, OUT_QG = 3, OUT_S2F6 = 4;

// Order a wave's LDS writes and later reads (or reads and later writes) of
// the same staging rows: wait for its LDS operations and fence the compiler.
__device__ __forceinline__ void lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// DROP: output rows may be dropped slots of a grouped GEMM, whose scale is
// 0; adding +0 turns their -0 products into +0, so they come out as the
// zero rows (and zero blocks) the header promises.
// NJ: the wave's 32-column blocks (4, or 2 in a 256 x 128 half tile of the
// plain output modes).
template <int OUT, bool DROP, int NJ, typename ScaleFn>
__device__ __forceinline__ void epilogue(uint8_t *stage, const float *tab,
                                         const f32x16 (&acc)[4][NJ], int64_t m0, int64_t m_end,
                                         int64_t n0, int64_t n_end, ScaleFn scale_of, void *C,
                                         int64_t ldc, int wm, int wn, int lane,
                                         const QuantOut &qo) {
    constexpr bool NVQ = OUT == OUT_Q || OUT == OUT_QG;   // NVFP4 encode
    constexpr bool S2 = OUT == OUT_S2F6;                   // combine wire format
    constexpr bool QUANT = NVQ || S2;
    static_assert(NJ == 4 || !QUANT, "the encoding epilogues take whole 256-column tiles");
    constexpr bool BF16_OUT = OUT == OUT_BF16 || QUANT;    // BF16 staging
    constexpr int WC = NJ * 32;                       // the wave's output columns
    constexpr int ES = BF16_OUT ? 2 : 4;              // bytes per element
    constexpr int RS = WC * ES + 16;                  // staging row stride
    constexpr int PR = BF16_OUT ? 32 : 16;            // rows per piece
    constexpr int LPR = WC * ES / 16;                 // lanes per row on read-back
    constexpr int RPI = 64 / LPR;                     // rows per read-back instruction
    // plain output: pieces alternate between the stage and a second buffer
    // past the ring (where the GELU modes keep their table), so a piece's
    // read-back needs no wait before the next piece is staged
    uint8_t *const buf0 = stage + (threadIdx.x >> 6) * (PR * RS);
    uint8_t *const buf1 = reinterpret_cast<uint8_t *>(const_cast<float *>(tab)) +
                          (threadIdx.x >> 6) * (PR * RS);
    const int64_t mw = m0 + wm * 128, nw = n0 + wn * WC;
    const int lr = lane & 31;                          // the lane's row in a 32-row block
    float s_enc = 1.0f, s_dec = 1.0f, amax = 0.0f;
    if (NVQ) {
        s_enc = qo.s_enc[0];
        s_dec = 1.0f / s_enc;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // output scale of the lane's row: s_dec,A (of that row) * s_dec,B
        const int64_t mr = mw + i * 32 + lr;
        const float out_scale = scale_of(mr < m_end ? mr : m_end - 1);
#pragma unroll
        for (int piece = 0; piece < 32 / PR; ++piece) {
            uint8_t *const buf = (!QUANT && ((i * (32 / PR) + piece) & 1)) ? buf1 : buf0;
            if (lr / PR == piece) {
                uint8_t *row = buf + (lr - piece * PR) * RS;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c = j * 32 + 8 * g + 4 * (lane >> 5);
                        float y0 = acc[i][j][4 * g] * out_scale;
                        float y1 = acc[i][j][4 * g + 1] * out_scale;
                        float y2 = acc[i][j][4 * g + 2] * out_scale;
                        float y3 = acc[i][j][4 * g + 3] * out_scale;
                        if constexpr (DROP) {
                            y0 = y0 + 0.0f;
                            y1 = y1 + 0.0f;
                            y2 = y2 + 0.0f;
                            y3 = y3 + 0.0f;
                        }
                        if constexpr (BF16_OUT)
                            *reinterpret_cast<uint2 *>(row + c * 2) =
                                make_uint2(pk_bf16(y0, y1), pk_bf16(y2, y3));
                        else
                            *reinterpret_cast<float4 *>(row + c * 4) = make_float4(y0, y1, y2, y3);
                    }
            }
            // a wave reads back only its own rows, written by other lanes of
            // the same wave: LDS executes a wave's operations in order, and
            // the barrier keeps the compiler from moving reads above writes
            lds_order();
            if constexpr (!QUANT) {
#pragma unroll
                for (int q = 0; q < PR / RPI; ++q) {
                    const int r = q * RPI + lane / LPR;
                    const int cb = (lane % LPR) * 16;
                    const uint4 val = *reinterpret_cast<const uint4 *>(buf + r * RS + cb);
                    const int64_t m = mw + i * 32 + piece * PR + r;
                    const int64_t n = nw + cb / ES;
                    if (m < m_end && n < n_end)
                        *reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(C) + (m * ldc + n) * ES) = val;
                }
            } else if constexpr (S2) {
                // 32 rows x 4 chunks of 32 BF16 values: two chunks per lane
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int r = q * 16 + lane / 4, c = lane % 4;
                    const uint4 *src = reinterpret_cast<const uint4 *>(buf + r * RS + c * 64);
                    float y[32];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint4 w = src[v];
                        const uint32_t hw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            y[8 * v + 2 * e] = __uint_as_float(hw[e] << 16);
                            y[8 * v + 2 * e + 1] = __uint_as_float(hw[e] & 0xFFFF0000u);
                        }
                    }
                    if (qo.rht) {
                        flip_signs32(y, qo.signs);
                        hadamard32(y);
                    }
                    float a = 0.0f;
#pragma unroll
                    for (int v = 0; v < 32; ++v) a = fmaxf(a, fabsf(y[v]));
                    const int k = s2f6_k(a);
                    uint32_t wd[8];
#pragma unroll
                    for (int v = 0; v < 8; ++v)
                        wd[v] = pack_bytes4(s2f6_byte(y[4 * v], k), s2f6_byte(y[4 * v + 1], k),
                                            s2f6_byte(y[4 * v + 2], k), s2f6_byte(y[4 * v + 3], k));
                    const int64_t m = mw + i * 32 + piece * PR + r;
                    const int64_t n = nw + c * 32;
                    if (m < m_end && n < n_end) {
                        uint4 *dst = reinterpret_cast<uint4 *>(qo.codes + m * n_end + n);
                        dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                        dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
                        qo.scales[m * (n_end / 32) + n / 32] = (uint8_t)(k + 127);
                    }
                }
            } else {
                // 32 rows x 8 blocks of 16 BF16 values: four blocks per lane
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = q * 8 + lane / 8, b = lane % 8;
                    const uint4 *src = reinterpret_cast<const uint4 *>(buf + r * RS + b * 32);
                    // the BF16 value the plain GEMM stores, GELU of it by the table
                    float f[16];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const uint4 w = src[v];
                        const uint32_t hw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint32_t hb = (e & 1) ? (hw[e >> 1] >> 16) : (hw[e >> 1] & 0xFFFFu);
                            f[8 * v + e] = OUT == OUT_QG ? gelu_bf16_select(hb, tab) : bf16_to_f32(hb);
                        }
                    }
                    const int64_t m = mw + i * 32 + piece * PR + r;
                    const int64_t n = nw + b * 16;
                    if (m < m_end && n < n_end) {
                        float a = 0.0f;
#pragma unroll
                        for (int v = 0; v < 16; ++v) a = fmaxf(a, fabsf(f[v]));
                        amax = fmaxf(amax, a);
                        const uint32_t sc = block_scale_code(a, s_enc);
                        const float se = block_enc_scale(sc, s_dec);
                        *reinterpret_cast<uint2 *>(qo.codes + m * (n_end / 2) + n / 2) =
                            make_uint2(e2m1_rne8(f, se), e2m1_rne8(f + 8, se));
                        qo.scales[m * (n_end / 16) + n / 16] = (uint8_t)sc;
                    }
                }
            }
            if constexpr (QUANT) lds_order();     // before the next piece is staged
        }
    }
    if (NVQ && qo.amax) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        if (lane == 0) atomicMax(qo.amax, __float_as_uint(amax));
    }
}

// One output tile of a workgroup's sequence: rows [m0, m_end) of the
// (row-mapped) A, columns [n0, n0 + BN) of group g's B.
struct TileRef {
    int64_t m0, m_end, n0;
    int g;
};

// A persistent workgroup (one per CU) takes its tiles one after another, and
// the slab ring runs on across them: while a tile's last two slabs are
// multiplied, the next tile's first two slabs are copied into the stages
// they free, and the epilogue stages its output in the third.  The slab loop
// itself is the single-tile one; only its last two iterations (peeled)
// switch the copies to the next tile.
//   next_tile(TileRef &)   the workgroup's next tile, false when done
//   b_view(g)              group g's B operand
//   a_row(m)               source row of A for output row m (< 0: none)
//   scale_of(m, g)         output scale of row m in group g's tile
template <int OUT, bool BT, bool DROP, int NJ, typename Next, typename BView, typename RowMap,
          typename ScaleFn>
__device__ __forceinline__ void run_tiles(Smem &sm, float *tab, const GemmParams &p,
                                          Next next_tile, BView b_view, RowMap a_row,
                                          ScaleFn scale_of) {
    // the wave index is uniform: the copies' LDS offsets live in scalar registers
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t K = p.K, N = p.N;
    // global_load_lds instructions one wave issues per slab
    constexpr int kIssued = 4 + NJ + 2 + (BT ? 1 : NJ / 2);
    const int64_t nslab = K / BK;

    TileRef cur;
    if (!next_tile(cur)) return;
    if (OUT == OUT_QG) gelu_table_load(tab, p.q.gelu_tab);   // ordered by the first barrier
    Plan pl = make_plan<NJ>(p.a, b_view(cur.g), K, a_rows(cur.m0, cur.m_end, a_row), cur.n0, N);
    int cs = 0;                                   // stage holding the current slab
    issue<BT, NJ>(sm.st[0], pl, 0);
    if (nslab > 1) issue<BT, NJ>(sm.st[1], pl, BK);

    for (;;) {
        // the next tile (the last tile repeats itself: its copies land in
        // stages nobody reads again)
        TileRef nxt;
        const bool more = next_tile(nxt);
        if (!more) nxt = cur;
        const ARows nar = a_rows(nxt.m0, nxt.m_end, a_row);
        // this tile's first slabs have landed (the previous tile's stores too:
        // vmcnt counts both)
        wait_vmcnt<0>();
        __syncthreads();

        f32x16 acc[4][NJ];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{0};

        uint2 sca[4], scb[4];
        Chunk c0, c1;
        Pairs p0, p1;
        f16x8 af[4], bf[4], an[4], bn[4];
        load_scales<BT, NJ>(sca, scb, sm.st[cs], wm, wn, lane);
        load_chunk<NJ>(c0, sm.st[cs], 0, wm, wn, lane);
        load_pairs<NJ>(p0, sca, scb, 0, lane);
        expand_step<NJ>(af, bf, c0, p0, 0);

        // The 8 MFMA steps of the current slab, with the expansion of step
        // k + 1 under the MFMAs of step k, and the copies of the slab at
        // byte offset kn (two ahead) into stage dst during the first steps.
        // Stage cs is read only by the chunk and scale loads at its start,
        // so the slab barrier can come after step 4: the last three steps
        // then cover the next slab's LDS reads.
        auto slab = [&](int64_t kn, Stage &dst) __attribute__((always_inline)) {
            const int ns = cs == 2 ? 0 : cs + 1;      // stage of the next slab
            auto none = [](int) {};
            auto copy_a = [&](int q) {
                copy_lds16(pl.a[q] + kn / 2, dst.a + (wave * 4 + q) * 1024);
            };
            auto copy_b = [&](int q) {
                if (q < NJ) copy_lds16(pl.b[q] + kn / 2, dst.b + (wave * NJ + q) * 1024);
            };
            auto copy_s = [&](int q) {
                if (q < 2) copy_lds4(pl.sa[q] + kn / 16, dst.as + (wave * 2 + q) * 256);
                else if (!BT) {
                    if (q - 2 < NJ / 2)
                        copy_lds4(pl.sb[q - 2] + kn / 16, dst.bs + (wave * (NJ / 2) + q - 2) * 256);
                } else if (q == 2) copy_lds4(pl.sb[0] + kn / 16, dst.bs);
            };
            load_chunk<NJ>(c1, sm.st[cs], 1, wm, wn, lane);
            load_pairs<NJ>(p1, sca, scb, 1, lane);
            step_q(acc, af, bf, an, bn, c0, p0, 1, copy_a);
            step_q(acc, an, bn, af, bf, c0, p0, 2, copy_b);
            step_q(acc, af, bf, an, bn, c0, p0, 3, copy_s);
            step_q(acc, an, bn, af, bf, c1, p1, 0, none);
            step_q(acc, af, bf, an, bn, c1, p1, 1, none);
            // the next slab is complete once every wave has seen its own copies land
            wait_vmcnt<kIssued>();
            __syncthreads();
            load_scales<BT, NJ>(sca, scb, sm.st[ns], wm, wn, lane);
            load_chunk<NJ>(c0, sm.st[ns], 0, wm, wn, lane);
            step_q(acc, an, bn, af, bf, c1, p1, 2, none);
            step_q(acc, af, bf, an, bn, c1, p1, 3, none);
            load_pairs<NJ>(p0, sca, scb, 0, lane);
            step_q(acc, an, bn, af, bf, c0, p0, 0, none);
            cs = ns;
        };
        auto two_ahead = [&]() -> Stage & {
            const int ns = cs == 2 ? 0 : cs + 1;
            return sm.st[ns == 2 ? 0 : ns + 1];
        };
        for (int64_t s = 0; s + 2 < nslab; ++s) slab((s + 2) * BK, two_ahead());
        if (nslab > 1) {
            // the second-to-last slab: its look-ahead copy is the next tile's slab 0
            pl = make_plan<NJ>(p.a, b_view(nxt.g), K, nar, nxt.n0, N);
            slab(0, two_ahead());
        }
        // The last slab, copying the next tile's slab 1 into the stage the
        // slab before used (a single-slab tile: the next tile's slab 0 into
        // the free stage).
        {
            const int c1s = cs == 2 ? 0 : cs + 1, c2s = c1s == 2 ? 0 : c1s + 1;
            if (nslab == 1) pl = make_plan<NJ>(p.a, b_view(nxt.g), K, nar, nxt.n0, N);
            const int64_t kl = nslab > 1 ? BK : 0;
            Stage &dst = sm.st[nslab > 1 ? c2s : c1s];
            auto none = [](int) {};
            auto copy_a = [&](int q) {
                copy_lds16(pl.a[q] + kl / 2, dst.a + (wave * 4 + q) * 1024);
            };
            auto copy_b = [&](int q) {
                if (q < NJ) copy_lds16(pl.b[q] + kl / 2, dst.b + (wave * NJ + q) * 1024);
            };
            auto copy_s = [&](int q) {
                if (q < 2) copy_lds4(pl.sa[q] + kl / 16, dst.as + (wave * 2 + q) * 256);
                else if (!BT) {
                    if (q - 2 < NJ / 2)
                        copy_lds4(pl.sb[q - 2] + kl / 16, dst.bs + (wave * (NJ / 2) + q - 2) * 256);
                } else if (q == 2) copy_lds4(pl.sb[0] + kl / 16, dst.bs);
            };
            load_chunk<NJ>(c1, sm.st[cs], 1, wm, wn, lane);
            load_pairs<NJ>(p1, sca, scb, 1, lane);
            step_q(acc, af, bf, an, bn, c0, p0, 1, copy_a);
            step_q(acc, an, bn, af, bf, c0, p0, 2, copy_b);
            step_q(acc, af, bf, an, bn, c0, p0, 3, copy_s);
            step_q(acc, an, bn, af, bf, c1, p1, 0, none);
            step_q(acc, af, bf, an, bn, c1, p1, 1, none);
            step_q(acc, an, bn, af, bf, c1, p1, 2, none);
            step_q(acc, af, bf, an, bn, c1, p1, 3, none);
            mfma_step(acc, an, bn);
        }
        // every wave is done reading stage cs: it becomes the staging area
        __syncthreads();
        const int g = cur.g;
        epilogue<OUT, DROP, NJ>(reinterpret_cast<uint8_t *>(&sm.st[cs]), tab, acc, cur.m0, cur.m_end,
                      cur.n0, N, [&](int64_t m) { return scale_of(m, g); }, p.c, p.ldc, wm, wn,
                      lane, p.q);
        if (!more) break;
        cur = nxt;
        cs = cs == 2 ? 0 : cs + 1;                // the next tile's slab 0
    }
    // the last tile's repeated copies land before the workgroup ends
    wait_vmcnt<0>();
}

}  // namespace big

// A persistent workgroup's share of a tile sequence: workgroup b runs on XCD
// b % 8, each XCD owns one contiguous eighth of the sequence (so the tiles in
// flight on an XCD share operand panels in its L2), and the workgroups of an
// XCD take its tiles in turn.
struct TileWalk {
    int64_t next, last, stride;
    __device__ TileWalk(int64_t total) {
        const int64_t x = blockIdx.x % 8, grid = gridDim.x;
        const int64_t share = total / 8, extra = total % 8;
        const int64_t first = x * share + (x < extra ? x : extra);
        last = first + share + (x < extra ? 1 : 0);
        stride = (grid - x + 7) / 8;              // workgroups on this XCD
        next = first + blockIdx.x / 8;
    }
    __device__ bool take(int64_t &tile) {
        if (next >= last) return false;
        tile = next;
        next += stride;
        return true;
    }
};

template <int OUT>
__device__ __forceinline__ void dense_body(const GemmParams &p, uint8_t *smem_raw) {
    big::Smem &sm = *reinterpret_cast<big::Smem *>(smem_raw);
    float *tab = reinterpret_cast<float *>(smem_raw + sizeof(big::Smem));
    if ((OUT == big::OUT_Q || OUT == big::OUT_QG) && blockIdx.x == 0 && threadIdx.x == 0)
        p.q.s_dec[0] = 1.0f / p.q.s_enc[0];
    const int64_t tm = (p.M + big::BM - 1) / big::BM, tn = (p.N + big::BN - 1) / big::BN;
    const int64_t total = tm * tn, grid = gridDim.x;
    // A last round of whole tiles that would leave more than half the
    // workgroups idle is run as twice as many 256 x 128 half tiles (plain
    // output modes): every workgroup then takes one half, and the round
    // costs about half a tile instead of a whole one.
    constexpr bool kHalves = OUT == big::OUT_F32 || OUT == big::OUT_BF16;
    const int64_t rem = total % grid;
    const bool split = kHalves && rem > 0 && 2 * rem <= grid;
    const int64_t n_whole = split ? total - rem : total;
    const int64_t M = p.M;
    auto tile_at = [&](int64_t tid, big::TileRef &r) {
        // grouped order: GROUP_M tiles down M, then along N
        const int64_t gsize = big::GROUP_M * tn;
        const int64_t g = tid / gsize, in = tid - g * gsize;
        const int64_t gm = (tm - g * big::GROUP_M) < big::GROUP_M ? (tm - g * big::GROUP_M) : big::GROUP_M;
        r.m0 = (g * big::GROUP_M + in % gm) * big::BM;
        r.m_end = M;
        r.n0 = (in / gm) * big::BN;
        r.g = 0;
    };
    TileWalk walk(n_whole);
    auto next_tile = [&](big::TileRef &r) -> bool {
        int64_t tid;
        if (!walk.take(tid)) return false;
        tile_at(tid, r);
        return true;
    };
    // half h: tile n_whole + h / 2, columns 128 * (h % 2) onwards (both
    // halves of a tile fall in one XCD's contiguous share)
    TileWalk half_walk(split ? 2 * rem : 0);
    auto next_half = [&](big::TileRef &r) -> bool {
        int64_t h;
        if (!half_walk.take(h)) return false;
        tile_at(n_whole + (h >> 1), r);
        r.n0 += (h & 1) * (big::BN / 2);
        return true;
    };
    const Fp4View B = p.b;
    auto b_view = [B](int) { return B; };
    auto ident = [](int64_t r) { return r; };
    const float sb = p.b.s_dec[0];
    auto run = [&](auto scale_of) {
        if (p.b.tile2d)
            big::run_tiles<OUT, true, false, 4>(sm, tab, p, next_tile, b_view, ident, scale_of);
        else
            big::run_tiles<OUT, false, false, 4>(sm, tab, p, next_tile, b_view, ident, scale_of);
        if constexpr (kHalves) {
            if (split) {
                // the last whole tile's epilogue has read its staging rows
                // before the ring is refilled
                __syncthreads();
                if (p.b.tile2d)
                    big::run_tiles<OUT, true, false, 2>(sm, tab, p, next_half, b_view, ident,
                                                        scale_of);
                else
                    big::run_tiles<OUT, false, false, 2>(sm, tab, p, next_half, b_view, ident,
                                                         scale_of);
            }
        }
    };
    if (p.a.sdec_rows) {
        const float *sa = p.a.s_dec;
        run([sa, sb](int64_t m, int) { return sa[m] * sb; });
    } else {
        const float out_scale = p.a.s_dec[0] * sb;
        run([out_scale](int64_t, int) { return out_scale; });
    }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(big::NT) void nvfp4_gemm_big_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    dense_body<BF16_OUT ? big::OUT_BF16 : big::OUT_F32>(p, smem_raw);
}

template <bool GELU>
__global__ __launch_bounds__(big::NT) void nvfp4_gemm_quant_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    dense_body<GELU ? big::OUT_QG : big::OUT_Q>(p, smem_raw);
}

__global__ __launch_bounds__(big::NT) void nvfp4_gemm_s2f6_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    dense_body<big::OUT_S2F6>(p, smem_raw);
}

constexpr int kMaxGroupsBig = 1024;

template <int OUT>
__device__ __forceinline__ void grouped_body(const GemmParams &p, uint8_t *smem_raw,
                                             int64_t *tile_start, int64_t *row_start) {
    big::Smem &sm = *reinterpret_cast<big::Smem *>(smem_raw);
    float *tab = reinterpret_cast<float *>(smem_raw + sizeof(big::Smem));
    if ((OUT == big::OUT_Q || OUT == big::OUT_QG) && blockIdx.x == 0 && threadIdx.x == 0)
        p.q.s_dec[0] = 1.0f / p.q.s_enc[0];
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
    TileWalk walk(tile_start[p.G]);
    const int G = p.G;
    auto next_tile = [&](big::TileRef &r) -> bool {
        int64_t tile;
        if (!walk.take(tile)) return false;
        int g = 0;
        while (g + 1 < G && tile_start[g + 1] <= tile) ++g;
        const int64_t local = tile - tile_start[g];
        const int64_t mt = local / n_tiles_n, nt = local - mt * n_tiles_n;
        r.m0 = row_start[g] + mt * big::BM;
        r.m_end = row_start[g + 1];
        r.n0 = nt * big::BN;
        r.g = g;
        return true;
    };
    const Fp4View B0 = p.b;
    const int64_t b_codes = p.N * (p.K / 2), b_scales = (B0.tile2d ? (p.N / 16) : p.N) * (p.K / 16);
    auto b_view = [B0, b_codes, b_scales](int g) {
        Fp4View B = B0;
        B.codes = B0.codes + (int64_t)g * b_codes;
        B.scales = B0.scales + (int64_t)g * b_scales;
        return B;
    };
    const int32_t *ri = p.row_index;
    const int64_t src_rows = p.a_src_rows;
    auto gather = [ri, src_rows](int64_t r) -> int64_t {
        const int64_t s = ri ? (int64_t)ri[r] : r;
        return (s >= 0 && s < src_rows) ? s : -1;
    };
    const float *sdb = p.b.s_dec;
    auto run = [&](auto scale_of) {
        if (B0.tile2d)
            big::run_tiles<OUT, true, true, 4>(sm, tab, p, next_tile, b_view, gather, scale_of);
        else
            big::run_tiles<OUT, false, true, 4>(sm, tab, p, next_tile, b_view, gather, scale_of);
    };
    // the output scale of row m: the decode scale of the A row it was
    // computed from times the expert's; 0 for a dropped slot (its copies
    // read A row 0 in place of a row the map misses)
    if (p.a.sdec_rows) {
        const float *sa = p.a.s_dec;
        run([sa, sdb, gather](int64_t m, int g) {
            const int64_t s = gather(m);
            return s < 0 ? 0.0f : sa[s] * sdb[g];
        });
    } else {
        const float sa0 = p.a.s_dec[0];
        run([sa0, sdb, gather](int64_t m, int g) { return gather(m) < 0 ? 0.0f : sa0 * sdb[g]; });
    }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(big::NT) void grouped_nvfp4_gemm_big_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    __shared__ int64_t tile_start[kMaxGroupsBig + 1];
    __shared__ int64_t row_start[kMaxGroupsBig + 1];
    grouped_body<BF16_OUT ? big::OUT_BF16 : big::OUT_F32>(p, smem_raw, tile_start, row_start);
}

template <bool GELU>
__global__ __launch_bounds__(big::NT) void grouped_nvfp4_gemm_quant_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    __shared__ int64_t tile_start[kMaxGroupsBig + 1];
    __shared__ int64_t row_start[kMaxGroupsBig + 1];
    grouped_body<GELU ? big::OUT_QG : big::OUT_Q>(p, smem_raw, tile_start, row_start);
}

__global__ __launch_bounds__(big::NT) void grouped_nvfp4_gemm_s2f6_kernel(GemmParams p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    __shared__ int64_t tile_start[kMaxGroupsBig + 1];
    __shared__ int64_t row_start[kMaxGroupsBig + 1];
    grouped_body<big::OUT_S2F6>(p, smem_raw, tile_start, row_start);
}

__global__ void clear_amax_kernel(unsigned *amax) { *amax = 0u; }

// Persistent grid: one workgroup per CU of the stream's device (the LDS ring
// admits one), a multiple of 8 so every XCD holds the same number; never
// more than the tiles when those are known.
static int64_t persistent_grid(int64_t tiles, hipStream_t s) {
    const int n = device_cus(s);
    const int64_t g = n >= 8 ? n / 8 * 8 : 8;
    return tiles > 0 && tiles < g ? tiles : g;
}

// Launch with `shm` bytes of dynamic LDS; the kernel's limit is raised once
// per kernel (thread-safe static initialisation).
template <auto Kernel>
static void launch_with_smem(int64_t grid, size_t shm, const GemmParams &p, hipStream_t s) {
    static const bool attr_set = [shm] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(Kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        return true;
    }();
    (void)attr_set;
    hipLaunchKernelGGL(Kernel, dim3((unsigned)grid), dim3(big::NT), shm, s, p);
}

static int64_t dense_tiles(const GemmParams &p) {
    return ((p.M + big::BM - 1) / big::BM) * ((p.N + big::BN - 1) / big::BN);
}

constexpr size_t kSmemBig = sizeof(big::Smem);
// plain output: the second staging buffer (4 waves x 32 rows x 272 bytes)
constexpr size_t kSmemPlain = sizeof(big::Smem) + 4 * 32 * 272;
constexpr size_t kSmemGelu = sizeof(big::Smem) + kGeluTabSize * sizeof(float);

hipError_t launch_nvfp4_gemm_quant(const GemmParams &p, bool gelu, hipStream_t s) {
    if (p.q.amax) hipLaunchKernelGGL(clear_amax_kernel, dim3(1), dim3(1), 0, s, p.q.amax);
    if (gelu) {
        const hipError_t e = launch_gelu_table(const_cast<float *>(p.q.gelu_tab), s);
        if (e != hipSuccess) return e;
    }
    const int64_t grid = persistent_grid(dense_tiles(p), s);
    if (gelu) launch_with_smem<nvfp4_gemm_quant_kernel<true>>(grid, kSmemGelu, p, s);
    else launch_with_smem<nvfp4_gemm_quant_kernel<false>>(grid, kSmemBig, p, s);
    return hipGetLastError();
}

hipError_t launch_grouped_nvfp4_gemm_quant(const GemmParams &p, bool gelu, hipStream_t s) {
    if (p.G > kMaxGroupsBig) return hipErrorInvalidValue;
    if (p.q.amax) hipLaunchKernelGGL(clear_amax_kernel, dim3(1), dim3(1), 0, s, p.q.amax);
    if (gelu) {
        const hipError_t e = launch_gelu_table(const_cast<float *>(p.q.gelu_tab), s);
        if (e != hipSuccess) return e;
    }
    const int64_t grid = persistent_grid(0, s);
    if (gelu) launch_with_smem<grouped_nvfp4_gemm_quant_kernel<true>>(grid, kSmemGelu, p, s);
    else launch_with_smem<grouped_nvfp4_gemm_quant_kernel<false>>(grid, kSmemBig, p, s);
    return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_s2f6(const GemmParams &p, hipStream_t s) {
    launch_with_smem<nvfp4_gemm_s2f6_kernel>(persistent_grid(dense_tiles(p), s), kSmemBig, p, s);
    return hipGetLastError();
}

hipError_t launch_grouped_nvfp4_gemm_s2f6(const GemmParams &p, hipStream_t s) {
    if (p.G > kMaxGroupsBig) return hipErrorInvalidValue;
    launch_with_smem<grouped_nvfp4_gemm_s2f6_kernel>(persistent_grid(0, s), kSmemBig, p, s);
    return hipGetLastError();
}

hipError_t launch_nvfp4_gemm_big(const GemmParams &p, bool bf16_out, hipStream_t s) {
    // up to two workgroups per tile, so that fewer tiles than CUs run as
    // half tiles
    const int64_t grid = persistent_grid(2 * dense_tiles(p), s);
    if (bf16_out) launch_with_smem<nvfp4_gemm_big_kernel<true>>(grid, kSmemPlain, p, s);
    else launch_with_smem<nvfp4_gemm_big_kernel<false>>(grid, kSmemPlain, p, s);
    return hipGetLastError();
}

hipError_t launch_grouped_nvfp4_gemm_big(const GemmParams &p, bool bf16_out, hipStream_t s) {
    if (p.G > kMaxGroupsBig) return hipErrorInvalidValue;
    const int64_t grid = persistent_grid(0, s);
    if (bf16_out) launch_with_smem<grouped_nvfp4_gemm_big_kernel<true>>(grid, kSmemPlain, p, s);
    else launch_with_smem<grouped_nvfp4_gemm_big_kernel<false>>(grid, kSmemPlain, p, s);
    return hipGetLastError();
}

}  // namespace bbs

// NVFP4 quantizer and MXFP8 requantizer kernels (gfx950).
//
// Quantize (Pretraining LLMs with NVFP4, "NVFP4 Format and Quantization
// Procedure", steps 1-4; 4bit.vizuara.ai sections 5-6, 13):
//   pass 1  amax_kernel: per-workgroup maxima of |x| and / or of the RHT'd
//           16-row column chunks, from one read of x; no atomics, no zeroing.
//   pass 2  quant_kernel: every wave folds the partials into the tensor amax
//           (bit-identical everywhere).  A workgroup owns a 256-row x
//           128-column tile of x; each thread a 16 x 8 piece of it, loaded as
//           16 rows of 16 bytes.  From that one read it writes any of: the
//           row-wise NVFP4 copy (a 1x16 block is two neighbouring lanes), the
//           column-wise NVFP4 copy of x^T (eight full column blocks per
//           thread, optional RHT), and the row-wise MXFP8 copy (a block of 32
//           is four lanes).  With 256 tile rows, each transposed row's 128
//           code bytes are written by one workgroup, so HBM sees whole lines.
//           Block scales are gathered in LDS and written as contiguous runs.
// Requantize (4bit.vizuara.ai sections 9-10): requant_kernel dequantizes a
// 32-row x 8-column piece of an NVFP4 matrix in FP32 and writes its 8
// transposed rows of 32 as MXFP8 (E8M0 per 32, E4M3 elements, RTN or SR).
//
// Workgroups are mapped to tiles so that each of the 8 XCDs works through a
// contiguous run of tiles (neighbouring tiles share output lines in L2).
#include <type_traits>

#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

constexpr int kQT = 256;                       // threads per workgroup
constexpr int kTileR = 256, kTileC = 128;      // quantizer tile of x
constexpr int kAmaxGrid = 512;                 // workgroups (= partials) of pass 1
constexpr int kReqR = 128, kReqC = 512;        // requantizer tile of the source

static_assert(kAmaxGrid <= kAmaxPartials, "amax partials exceed the workspace");
static_assert(kGeluTabOffset + kGeluTabSize <= kWorkspaceFloats, "GELU table exceeds the workspace");
static_assert(kGeluTabOffset % 4 == 0, "GELU table must stay 16-byte aligned");

// Tile t of T when workgroup b runs on XCD b % 8: XCD x takes a contiguous
// run of tiles.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t T) {
    const int64_t x = b % 8, j = b / 8, per = T / 8, rem = T % 8;
    return x * per + (x < rem ? x : rem) + j;
}

// A thread's 16 x 8 piece of a quantizer tile.
struct Piece {
    int64_t R0, C0;   // the tile's first row / column
    int64_t r0, c0;   // the piece's first row / column
    int band, cg;     // 16-row band and 8-column group inside the tile
    bool in;          // the piece lies inside x (R, C are multiples of 16)
};

__device__ __forceinline__ Piece piece_of(int64_t tile, int64_t R, int64_t C) {
    const int64_t tiles_c = (C + kTileC - 1) / kTileC;
    const int64_t tr = tile / tiles_c;
    Piece q;
    q.R0 = tr * kTileR;
    q.C0 = (tile - tr * tiles_c) * kTileC;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    q.band = w * 4 + (lane >> 4);
    q.cg = lane & 15;
    q.r0 = q.R0 + q.band * 16;
    q.c0 = q.C0 + q.cg * 8;
    q.in = q.r0 < R && q.c0 < C;
    return q;
}

// 16 rows of 16 bytes.  A piece outside x reads a valid piece instead (its
// results are never stored), so the loads need no branches.
__device__ __forceinline__ void load_piece(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                           const Piece &q, uint4 v[16]) {
    const int64_t r = q.r0 < R ? q.r0 : R - 16;
    const int64_t c = q.c0 < C ? q.c0 : C - 8;
    const uint16_t *src = x + r * ld + c;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const uint4 *>(src + i * ld);
}

// Element j (compile-time) of a row of 8 BF16 values, as FP32.
__device__ __forceinline__ float elem(const uint4 &row, int j) {
    const uint32_t w = j < 2 ? row.x : (j < 4 ? row.y : (j < 6 ? row.z : row.w));
    return (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}

// Element j (compile-time) of a row of 8 BF16 values, as BF16 bits.
__device__ __forceinline__ uint32_t elem_bits(const uint4 &row, int j) {
    const uint32_t w = j < 2 ? row.x : (j < 4 ? row.y : (j < 6 ? row.z : row.w));
    return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    return m;
}

// ---------------------------------------------------------------------------
// Pass 1: partial amax of |x| (PLAIN) and of |RHT(column chunks)| (RHT).
// ---------------------------------------------------------------------------
// GELU: the partials are maxima of |GELU(x)|, found without evaluating GELU
// on most elements.  GELU is non-decreasing for x >= 0, so the largest value
// over the non-negative elements is GELU of their maximum; every negative
// element has |GELU| < kGeluNegBound, so the negative elements of a wave's
// pieces are evaluated only when GELU of the wave's largest element is below
// that bound (wave-uniform branch).  The result is the exact maximum.
template <bool PLAIN, bool RHT, bool GELU>
__global__ __launch_bounds__(kQT) void amax_kernel(const uint16_t *__restrict__ x, int64_t R,
                                                   int64_t C, int64_t ld, uint32_t signs,
                                                   float *__restrict__ part,
                                                   float *__restrict__ part_rht,
                                                   float *__restrict__ gelu_tab) {
    static_assert(!GELU || (!PLAIN && !RHT), "GELU partials replace the plain ones");
    if (GELU)
        for (int i = blockIdx.x * kQT + threadIdx.x; i < kGeluTabSize; i += gridDim.x * kQT)
            gelu_tab[i] = gelu_table_entry(i);
    __shared__ float red[2][kQT / 64];
    const int64_t T = ((R + kTileR - 1) / kTileR) * ((C + kTileC - 1) / kTileC);
    float m = 0.0f, mr = 0.0f;
    float mx = 0.0f;     // GELU: largest element seen (0 if none is positive)
    // The next tile's piece is loaded while this one is reduced.
    int64_t tile = blockIdx.x;
    Piece q = piece_of(tile, R, C);
    uint4 v[16];
    if (tile < T) load_piece(x, R, C, ld, q, v);
    while (tile < T) {
        const int64_t next = tile + gridDim.x;
        const Piece qn = piece_of(next < T ? next : tile, R, C);
        uint4 vn[16];
        if (next < T) load_piece(x, R, C, ld, qn, vn);
        if (q.in) {
        if (PLAIN) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem(v[r], j)));
        }
        if (RHT) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float y[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) y[r] = elem(v[r], j);
                rht16_butterflies(y, signs);
#pragma unroll
                for (int r = 0; r < 16; ++r) mr = fmaxf(mr, fabsf(y[r]));
            }
        }
        }
        if (GELU) {
            float pm = 0.0f;
            if (q.in) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int j = 0; j < 8; ++j) pm = fmaxf(pm, elem(v[r], j));
            }
            mx = fmaxf(mx, pm);
            if (gelu_tanh(wave_max(pm)) < kGeluNegBound && q.in) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(gelu_tanh(elem(v[r], j))));
            }
        }
        tile = next;
        q = qn;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = vn[i];
    }
    // The transform's final multiply by 1/4 is monotonic, so the maximum of
    // the scaled values is the scaled maximum (bit for bit).
    mr = mr * 0.25f;
    if (GELU) m = fmaxf(m, gelu_tanh(mx));
    m = wave_max(m);
    mr = wave_max(mr);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][w] = m;
        red[1][w] = mr;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0][0], b = red[1][0];
        for (int i = 1; i < kQT / 64; ++i) {
            a = fmaxf(a, red[0][i]);
            b = fmaxf(b, red[1][i]);
        }
        if (PLAIN || GELU) part[blockIdx.x] = a;
        if (RHT) part_rht[blockIdx.x] = b;
    }
}

// ---------------------------------------------------------------------------
// Pass 2: encode.
// ---------------------------------------------------------------------------

// The tensor amax: the maximum of n <= kAmaxPartials partials, in every lane.
__device__ __forceinline__ float fold_partials(const float *part, int n) {
    float m = 0.0f;
    for (int i = threadIdx.x & 63; i < n; i += 64) m = fmaxf(m, part[i]);
    return wave_max(m);
}

// Copy n bytes from LDS to global memory: one vector store when the run is
// whole and aligned, else byte stores.
template <int N>
__device__ __forceinline__ void put_run(uint8_t *dst, const uint8_t *src, int64_t n) {
    if (n == N && (reinterpret_cast<uintptr_t>(dst) % N) == 0) {
        if constexpr (N == 16) *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
        if constexpr (N == 8) *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(src);
        if constexpr (N == 4)
            *reinterpret_cast<uint32_t *>(dst) = *reinterpret_cast<const uint32_t *>(src);
    } else {
        for (int64_t i = 0; i < n; ++i) dst[i] = src[i];
    }
}

// GELU: the row-wise copies are of GELU(x), evaluated once per element in
// FP32 (the pages' fused activation + quantize); the amax partials are those
// of |GELU(x)|.
template <bool HAS_ROW, bool HAS_COL, bool HAS_MX, bool TILE2D, bool RHT, bool GELU>
__global__ __launch_bounds__(kQT) void quant_kernel(QuantParams p) {
    static_assert(!GELU || (!HAS_COL && !TILE2D && !RHT), "GELU feeds the row-wise copies");
    __shared__ __align__(16) uint8_t s_row[kTileR * 8];    // row copy scales
    __shared__ __align__(16) uint8_t s_col[kTileC * 16];   // column copy scales
    __shared__ __align__(16) uint8_t s_mx[kTileR * 4];     // MXFP8 scales
    __shared__ __align__(16) float s_gelu[GELU ? kGeluTabSize : 1];
    const int64_t T = ((p.R + kTileR - 1) / kTileR) * ((p.C + kTileC - 1) / kTileC);
    const Piece q = piece_of(xcd_tile(blockIdx.x, T), p.R, p.C);
    uint4 v[16];
    load_piece(p.x, p.R, p.C, p.ld, q, v);

    // Tensor scales, identical in every wave.
    float s_enc_row = 1.0f, s_enc_col = 1.0f;
    if (HAS_ROW || (HAS_COL && !RHT)) s_enc_row = tensor_s_enc(fold_partials(p.part, p.n_part));
    if (HAS_COL) s_enc_col = RHT ? tensor_s_enc(fold_partials(p.part_rht, p.n_part_rht)) : s_enc_row;
    const float s_dec_row = 1.0f / s_enc_row;
    const float s_dec_col = 1.0f / s_enc_col;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (HAS_ROW) p.row_sdec[0] = s_dec_row;
        if (HAS_COL) p.col_sdec[0] = s_dec_col;
    }
    const int lane = threadIdx.x & 63;
    if constexpr (GELU) {
        gelu_table_load(s_gelu, p.gelu_tab);        // while the piece is in flight
        __syncthreads();
    }
    // Element j of row r of the piece, as the row-wise copies see it (GELU:
    // looked up where it is used, so the piece stays in its BF16 registers).
    auto val = [&](int r, int j) -> float __attribute__((always_inline)) {
        if constexpr (GELU) return gelu_bf16(elem_bits(v[r], j), s_gelu);
        else return elem(v[r], j);
    };


    // 16x16 tile amax (two lanes hold one tile; TILE2D excludes RHT).
    float tile_amax = 0.0f;
    if (TILE2D) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) tile_amax = fmaxf(tile_amax, fabsf(elem(v[r], j)));
        tile_amax = max_lane_pair(tile_amax);
    }

    // ---- row-wise copies (NVFP4 and MXFP8), one row of the piece at a time ----
    uint32_t tsc = 0;
    float ts = 0.0f;
    if (HAS_ROW && TILE2D) {
        tsc = block_scale_code(tile_amax, s_enc_row);
        ts = block_enc_scale(tsc, s_dec_row);
    }
    // NVFP4 copy of row r of the piece (values f)
    auto row_copy = [&](auto sr_tag, int r, const float f[8]) __attribute__((always_inline)) {
        constexpr bool SR = decltype(sr_tag)::value;
        uint32_t sc = tsc;
        float s = ts;
        if (!TILE2D) {
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
            sc = block_scale_code(max_lane_pair(a), s_enc_row);
            s = block_enc_scale(sc, s_dec_row);
            if ((lane & 1) == 0) s_row[(q.band * 16 + r) * 8 + (q.cg >> 1)] = (uint8_t)sc;
        }
        uint32_t packed;
        if (SR) {
            uint32_t w[4];
            sr_block(p.row_seed, p.row_stream, (uint64_t)((q.r0 + r) * p.C + q.c0) / 8, w);
            packed = e2m1_sr8(f, s, w);
        } else {
            packed = e2m1_rne8(f, s);
        }
        if (q.in) *reinterpret_cast<uint32_t *>(p.row_codes + (q.r0 + r) * (p.C / 2) + q.c0 / 2) =
            packed;
    };
    // MXFP8 copy of row r of the piece (values f)
    auto mx_copy = [&](auto sr_tag, int r, const float f[8]) __attribute__((always_inline)) {
        constexpr bool SR = decltype(sr_tag)::value;
        float y[8];
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
        const int k = e8m0_k(max_lane_quad(a));
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = ldexpf(f[j], -k);   // exact
        uint32_t lo, hi;
        if (SR) {
            uint32_t w[4];
            sr_block(p.mx_seed, p.mx_stream, (uint64_t)((q.r0 + r) * p.C + q.c0) / 8, w);
            lo = e4m3_sr4(y[0], y[1], y[2], y[3], sr_word_lo(w[0]), sr_word_hi(w[0]),
                          sr_word_lo(w[1]), sr_word_hi(w[1]));
            hi = e4m3_sr4(y[4], y[5], y[6], y[7], sr_word_lo(w[2]), sr_word_hi(w[2]),
                          sr_word_lo(w[3]), sr_word_hi(w[3]));
        } else {
            lo = e4m3_rne4(y[0], y[1], y[2], y[3]);
            hi = e4m3_rne4(y[4], y[5], y[6], y[7]);
        }
        if (q.in) *reinterpret_cast<uint2 *>(p.mx_codes + (q.r0 + r) * p.C + q.c0) = make_uint2(lo, hi);
        if ((lane & 3) == 0) s_mx[(q.band * 16 + r) * 4 + (q.cg >> 2)] = (uint8_t)(k + 127);
    };
    // (two loops of 8 rows: each stays under the compiler's full-unroll
    // limit, so the piece's registers are never indexed at run time)
    auto rows = [&](auto row_sr, auto mx_sr) __attribute__((always_inline)) {
        auto one = [&](int r) __attribute__((always_inline)) {
            float f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = val(r, j);
            if (HAS_ROW) row_copy(row_sr, r, f);
            if (HAS_MX) mx_copy(mx_sr, r, f);
        };
#pragma unroll
        for (int r = 0; r < 8; ++r) one(r);
#pragma unroll
        for (int r = 8; r < 16; ++r) one(r);
    };
    if (HAS_ROW || HAS_MX) {
        const bool row_sr = HAS_ROW && p.row_round == 1, mx_sr = HAS_MX && p.mx_round == 1;
        if (row_sr && mx_sr) rows(std::true_type{}, std::true_type{});
        else if (row_sr) rows(std::true_type{}, std::false_type{});
        else if (mx_sr) rows(std::false_type{}, std::true_type{});
        else rows(std::false_type{}, std::false_type{});
    }
    if (HAS_ROW && TILE2D && (lane & 1) == 0) s_row[q.band * 8 + (q.cg >> 1)] = (uint8_t)tsc;

    // ---- column-wise NVFP4 copy (of x^T) ---------------------------------------
    if (HAS_COL) {
        uint32_t tsc = 0;
        float ts = 0.0f;
        if (TILE2D) {
            tsc = block_scale_code(tile_amax, s_enc_col);
            ts = block_enc_scale(tsc, s_dec_col);
        }
        auto cols = [&](auto sr_tag) {
            constexpr bool SR = decltype(sr_tag)::value;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float y[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) y[r] = elem(v[r], j);
                if (RHT) rht16(y, p.rht_signs);
                uint32_t sc = tsc;
                float s = ts;
                if (!TILE2D) {
                    float a = 0.0f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(y[r]));
                    sc = block_scale_code(a, s_enc_col);
                    s = block_enc_scale(sc, s_dec_col);
                    s_col[(q.cg * 8 + j) * 16 + q.band] = (uint8_t)sc;
                }
                const int64_t c = q.c0 + j;                 // row of the transposed copy
                uint32_t w0, w1;
                if (SR) {
                    const uint64_t n0 = (uint64_t)(c * p.R + q.r0) / 8;
                    uint32_t w[4];
                    sr_block(p.col_seed, p.col_stream, n0, w);
                    w0 = e2m1_sr8(y, s, w);
                    sr_block(p.col_seed, p.col_stream, n0 + 1, w);
                    w1 = e2m1_sr8(y + 8, s, w);
                } else {
                    w0 = e2m1_rne8(y, s);
                    w1 = e2m1_rne8(y + 8, s);
                }
                if (q.in)
                    *reinterpret_cast<uint2 *>(p.col_codes + c * (p.R / 2) + q.r0 / 2) =
                        make_uint2(w0, w1);
            }
        };
        if (p.col_round == 1) cols(std::true_type{});
        else cols(std::false_type{});
        if (TILE2D && (lane & 1) == 0) s_col[(q.cg >> 1) * 16 + q.band] = (uint8_t)tsc;
    }

    // ---- block scales, as contiguous runs ------------------------------------
    __syncthreads();
    const int t = threadIdx.x;
    const int64_t nb_row = (p.C - q.C0) / 16, nb_col = (p.R - q.R0) / 16;
    if (HAS_ROW) {
        if (!TILE2D) {
            if (q.R0 + t < p.R)
                put_run<8>(p.row_scales + (q.R0 + t) * (p.C / 16) + q.C0 / 16, s_row + t * 8,
                           nb_row < 8 ? nb_row : 8);
        } else if (t < 16 && q.R0 / 16 + t < p.R / 16) {
            put_run<8>(p.row_scales + (q.R0 / 16 + t) * (p.C / 16) + q.C0 / 16, s_row + t * 8,
                       nb_row < 8 ? nb_row : 8);
        }
    }
    if (HAS_MX && q.R0 + t < p.R) {
        const int64_t nb = (p.C - q.C0) / 32;
        put_run<4>(p.mx_scales + (q.R0 + t) * (p.C / 32) + q.C0 / 32, s_mx + t * 4,
                   nb < 4 ? nb : 4);
    }
    if (HAS_COL) {
        if (!TILE2D) {
            if (t < kTileC && q.C0 + t < p.C)
                put_run<16>(p.col_scales + (q.C0 + t) * (p.R / 16) + q.R0 / 16, s_col + t * 16,
                            nb_col < 16 ? nb_col : 16);
        } else if (t < kTileC / 16 && q.C0 / 16 + t < p.C / 16) {
            put_run<16>(p.col_scales + (q.C0 / 16 + t) * (p.R / 16) + q.R0 / 16, s_col + t * 16,
                        nb_col < 16 ? nb_col : 16);
        }
    }
}

// ---------------------------------------------------------------------------
// Activation copy: per-token outer scale and / or Four Over Six
// (4bit.vizuara.ai, section 11; End-to-End 4-Bit Training, recipe details).
// One wave per row; in chunk k of 512 columns lane l holds columns
// 512k + 8l .. 512k + 8l + 7, so a 1x16 block is two neighbouring lanes.
// With a per-token scale the row amax comes first (the first 8 chunks stay
// in registers; longer rows are read again).  Four Over Six encodes every
// block with its top-6 and its top-4 scale and keeps the encoding with the
// smaller squared error, computed in FP32 as the sum over the block's first
// eight values (the even lane) plus the sum over its last eight (the odd
// lane), each in element order; the top-6 encoding is kept on ties.
// ---------------------------------------------------------------------------
constexpr int kActChunks = 8;

__device__ __forceinline__ void load_chunk8(const uint16_t *row, int64_t C, int64_t k, int lane,
                                            uint4 &v) {
    const int64_t c = k * 512 + lane * 8;
    v = c < C ? *reinterpret_cast<const uint4 *>(row + c) : make_uint4(0, 0, 0, 0);
}

// Squared error of 8 values f against their E2M1 codes (packed nibbles)
// dequantized as (code * S) * s_dec, summed in element order.
__device__ __forceinline__ float half_err(const float f[8], uint32_t packed, float S,
                                          float s_dec) {
    const f32x2_t g[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 1),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 2),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 3)};
    float e = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float d = f[j] - (g[j >> 1][j & 1] * S) * s_dec;    // code * S is exact
        e = e + d * d;
    }
    return e;
}

// A lane's 8 values of a chunk: x, or GELU(x) (tab: the LDS GELU table).
template <bool GELU>
__device__ __forceinline__ void act_values(const uint4 &v, float f[8], const float *tab) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = GELU ? gelu_bf16(elem_bits(v, j), tab) : elem(v, j);
}

template <bool FOUR_SIX>
__device__ __forceinline__ void act_encode_chunk(const float f[8], float s_enc, float s_dec,
                                                 int lane, uint32_t &packed, uint32_t &sc) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
    a = max_lane_pair(a);
    const uint32_t sc6 = block_scale_code(a, s_enc, 6.0f);
    packed = e2m1_rne8(f, block_enc_scale(sc6, s_dec));
    sc = sc6;
    if (FOUR_SIX) {
        const uint32_t sc4 = block_scale_code(a, s_enc, 4.0f);
        const uint32_t p4 = e2m1_rne8(f, block_enc_scale(sc4, s_dec));
        const float S6 = __builtin_amdgcn_cvt_scalef32_f32_fp8((int)sc6, 1.0f, 0);
        const float S4 = __builtin_amdgcn_cvt_scalef32_f32_fp8((int)sc4, 1.0f, 0);
        const float h6 = half_err(f, packed, S6, s_dec), h4 = half_err(f, p4, S4, s_dec);
        // the partner lane's half (quad_perm [1,0,3,2]); low half + high half
        const float o6 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(h6), 0xB1, 0xF, 0xF, false));
        const float o4 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(h4), 0xB1, 0xF, 0xF, false));
        const bool lo = (lane & 1) == 0;
        const float e6 = lo ? h6 + o6 : o6 + h6;
        const float e4 = lo ? h4 + o4 : o4 + h4;
        if (e4 < e6) {
            packed = p4;
            sc = sc4;
        }
    }
}

// GELU: the copy is of GELU(x); the per-token amax uses the same shortcut as
// the amax pass (GELU of the row's largest element, and the negative
// elements only when that is below kGeluNegBound).
template <bool PER_TOKEN, bool FOUR_SIX, bool GELU>
__global__ __launch_bounds__(kQT) void quant_act_kernel(QuantParams p) {
    __shared__ __align__(16) float s_gelu[GELU ? kGeluTabSize : 1];
    const int lane = threadIdx.x & 63;
    float s_enc_t = 1.0f;                             // the tensor's, without PER_TOKEN
    if (!PER_TOKEN) {
        s_enc_t = tensor_s_enc(fold_partials(p.part, p.n_part));
        if (blockIdx.x == 0 && threadIdx.x == 0) p.row_sdec[0] = 1.0f / s_enc_t;
    }
    const int64_t r = ((int64_t)blockIdx.x * kQT + threadIdx.x) >> 6;
    const bool live = r < p.R;
    float s_enc = s_enc_t;
    const uint16_t *row = p.x + (live ? r : 0) * p.ld;
    const int64_t nch = (p.C + 511) / 512;
    uint4 v[kActChunks];
#pragma unroll
    for (int k = 0; k < kActChunks; ++k)
        if (k < nch) load_chunk8(row, p.C, k, lane, v[k]);
    if constexpr (GELU) {
        gelu_table_load(s_gelu, p.gelu_tab);        // while the row is in flight
        __syncthreads();
    }
    if (!live) return;                                // whole waves leave together
    if (PER_TOKEN) {
        // GELU: m is the largest element (at least 0), else the largest |x|
        // (chunks past the row's end hold zeros)
        auto fold = [&](float m, const uint4 &w) {
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, GELU ? elem(w, j) : fabsf(elem(w, j)));
            return m;
        };
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < kActChunks; ++k)
            if (k < nch) m = fold(m, v[k]);
        for (int64_t k = kActChunks; k < nch; ++k) {
            uint4 w;
            load_chunk8(row, p.C, k, lane, w);
            m = fold(m, w);
        }
        float amax = wave_max(m);
        if (GELU) {
            amax = gelu_tanh(amax);
            if (amax < kGeluNegBound) {                 // wave-uniform
                float mn = 0.0f;
                auto fold_neg = [&](const uint4 &w) {
                    float f[8];
                    act_values<true>(w, f, s_gelu);
#pragma unroll
                    for (int j = 0; j < 8; ++j) mn = fmaxf(mn, fabsf(f[j]));
                };
#pragma unroll
                for (int k = 0; k < kActChunks; ++k)
                    if (k < nch) fold_neg(v[k]);
                for (int64_t k = kActChunks; k < nch; ++k) {
                    uint4 w;
                    load_chunk8(row, p.C, k, lane, w);
                    fold_neg(w);
                }
                amax = fmaxf(amax, wave_max(mn));
            }
        }
        s_enc = tensor_s_enc(amax);
        if (lane == 0) p.row_sdec[r] = 1.0f / s_enc;
    }
    const float s_dec = 1.0f / s_enc;
    uint8_t *codes = p.row_codes + r * (p.C / 2);
    uint8_t *scales = p.row_scales + r * (p.C / 16);
    auto emit = [&](const uint4 &w, int64_t k) {
        uint32_t packed, sc;
        float f[8];
        act_values<GELU>(w, f, s_gelu);
        act_encode_chunk<FOUR_SIX>(f, s_enc, s_dec, lane, packed, sc);
        const int64_t c = k * 512 + lane * 8;
        if (c < p.C) {
            *reinterpret_cast<uint32_t *>(codes + c / 2) = packed;
            if ((lane & 1) == 0) scales[c / 16] = (uint8_t)sc;
        }
    };
#pragma unroll
    for (int k = 0; k < kActChunks; ++k)
        if (k < nch) emit(v[k], k);
    for (int64_t k = kActChunks; k < nch; ++k) {
        uint4 w;
        load_chunk8(row, p.C, k, lane, w);
        emit(w, k);
    }
}

// ---------------------------------------------------------------------------
// Requantize: NVFP4 [R x C] -> MXFP8 of the transpose [C x R].
// A workgroup takes 128 source rows (a 32-row band per wave) x 512 source
// columns (8 per lane), so each destination row's 128 bytes come from one
// workgroup.  Each lane: 32 rows x 8 columns -> 8 destination rows of 32.
// ---------------------------------------------------------------------------
template <bool SR, bool TILE2D>
__global__ __launch_bounds__(kQT) void requant_kernel(RequantParams p) {
    const int64_t tiles_c = (p.C + kReqC - 1) / kReqC;
    const int64_t T = ((p.R + kReqR - 1) / kReqR) * tiles_c;
    const int64_t tile = xcd_tile(blockIdx.x, T);
    const int64_t tr = tile / tiles_c, tc = tile - tr * tiles_c;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r0 = tr * kReqR + w * 32, c0 = tc * kReqC + lane * 8;
    if (r0 >= p.R || c0 >= p.C) return;              // no barriers or lane exchange below
    const float s_dec = p.s_dec[0];
    const int64_t nsb = p.C / 16;                    // scale bytes per scale row

    uint32_t cw[32];                                 // 8 nibbles of each source row
    float bs[TILE2D ? 2 : 32];                       // E4M3 block scales, decoded
#pragma unroll
    for (int r = 0; r < 32; ++r)
        cw[r] = *reinterpret_cast<const uint32_t *>(p.codes + (r0 + r) * (p.C / 2) + c0 / 2);
#pragma unroll
    for (int i = 0; i < (TILE2D ? 2 : 32); ++i) {
        const int64_t srow = TILE2D ? r0 / 16 + i : r0 + i;
        bs[i] = __builtin_amdgcn_cvt_scalef32_f32_fp8((int)p.scales[srow * nsb + c0 / 16], 1.0f, 0);
    }

    auto emit = [&](const float (&x)[32], int64_t c) {
        float a = 0.0f;
#pragma unroll
        for (int r = 0; r < 32; ++r) a = fmaxf(a, fabsf(x[r]));
        const int k = e8m0_k(a);
        uint32_t out[8];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = ldexpf(x[8 * g + i], -k);   // exact
            if (SR) {
                uint32_t wd[4];
                sr_block(p.seed, p.stream, (uint64_t)(c * p.R + r0) / 8 + g, wd);
                out[2 * g] = e4m3_sr4(y[0], y[1], y[2], y[3], sr_word_lo(wd[0]), sr_word_hi(wd[0]),
                                      sr_word_lo(wd[1]), sr_word_hi(wd[1]));
                out[2 * g + 1] = e4m3_sr4(y[4], y[5], y[6], y[7], sr_word_lo(wd[2]),
                                          sr_word_hi(wd[2]), sr_word_lo(wd[3]), sr_word_hi(wd[3]));
            } else {
                out[2 * g] = e4m3_rne4(y[0], y[1], y[2], y[3]);
                out[2 * g + 1] = e4m3_rne4(y[4], y[5], y[6], y[7]);
            }
        }
        uint4 *dst = reinterpret_cast<uint4 *>(p.out_codes + c * p.R + r0);
        dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
        dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
        p.out_scales[c * (p.R / 32) + r0 / 32] = (uint8_t)(k + 127);
    };

    auto pair = [&](auto jp_tag) {                   // source columns 2jp, 2jp + 1
        constexpr int jp = decltype(jp_tag)::value;
        float xe[32], xo[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const f32x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[r], 1.0f, jp);
            const float b = bs[TILE2D ? r / 16 : r];
            // (E2M1 x E4M3) is exact; the multiply by s_dec is one FP32 rounding.
            xe[r] = (e[0] * b) * s_dec;
            xo[r] = (e[1] * b) * s_dec;
        }
        emit(xe, c0 + 2 * jp);
        emit(xo, c0 + 2 * jp + 1);
    };
    pair(std::integral_constant<int, 0>{});
    pair(std::integral_constant<int, 1>{});
    pair(std::integral_constant<int, 2>{});
    pair(std::integral_constant<int, 3>{});
}

// ---------------------------------------------------------------------------
// MXFP4 copy (FP4 Training on Blackwell, 'The scaling math, worked'): blocks
// of 32 along a row; scale 2^k with k the smallest integer such that
// amax <= 6 * 2^k (with amax = m * 2^E, m in [0.5, 1): k = E - 3 if
// m <= 0.75, else E - 2; clamped to [-127, 127]); elements x * 2^-k (exact)
// rounded onto the E2M1 grid.  One block per lane.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mx4_k(float amax) {
    if (amax == 0.0f) return -127;
    int E;
    const float m = frexpf(amax, &E);
    const int k = (m <= 0.75f) ? E - 3 : E - 2;
    return k < -127 ? -127 : (k > 127 ? 127 : k);
}

template <bool SR>
__global__ __launch_bounds__(kQT) void mx4_quant_kernel(const uint16_t *__restrict__ x, int64_t R,
                                                        int64_t C, int64_t ld,
                                                        uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ scales,
                                                        uint64_t seed, uint32_t stream) {
    const int64_t nb = C / 32;
    const int64_t b = (int64_t)blockIdx.x * kQT + threadIdx.x;
    if (b >= R * nb) return;
    const int64_t r = b / nb, cb = b - r * nb;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + r * ld + cb * 32);
    float y[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[8 * i + j] = elem(v, j);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[i]));
    const int k = mx4_k(amax);
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = ldexpf(y[i], -k);
    uint32_t word[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (SR) {
            uint32_t w[4];
            sr_block(seed, stream, (uint64_t)(r * C + cb * 32) / 8 + i, w);
            word[i] = e2m1_sr8(y + 8 * i, 1.0f, w);
        } else {
            word[i] = e2m1_rne8(y + 8 * i, 1.0f);
        }
    }
    *reinterpret_cast<uint4 *>(codes + r * (C / 2) + cb * 16) =
        make_uint4(word[0], word[1], word[2], word[3]);
    scales[b] = (uint8_t)(k + 127);
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after argument checks).
// ---------------------------------------------------------------------------

hipError_t launch_amax(const uint16_t *x, int64_t R, int64_t C, int64_t ld, bool plain, bool rht,
                       uint32_t signs, float *part, float *part_rht, int *n_part,
                       hipStream_t s, float *gelu_tab) {
    const int64_t T = ((R + kTileR - 1) / kTileR) * ((C + kTileC - 1) / kTileC);
    const int grid = (int)(T < kAmaxGrid ? T : kAmaxGrid);
    *n_part = grid;
    if (gelu_tab) {
        if (rht || !plain) return hipErrorInvalidValue;
        hipLaunchKernelGGL((amax_kernel<false, false, true>), dim3(grid), dim3(kQT), 0, s, x, R, C,
                           ld, signs, part, part_rht, gelu_tab);
    } else if (plain && rht)
        hipLaunchKernelGGL((amax_kernel<true, true, false>), dim3(grid), dim3(kQT), 0, s, x, R, C,
                           ld, signs, part, part_rht, nullptr);
    else if (plain)
        hipLaunchKernelGGL((amax_kernel<true, false, false>), dim3(grid), dim3(kQT), 0, s, x, R, C,
                           ld, signs, part, part_rht, nullptr);
    else if (rht)
        hipLaunchKernelGGL((amax_kernel<false, true, false>), dim3(grid), dim3(kQT), 0, s, x, R, C,
                           ld, signs, part, part_rht, nullptr);
    return hipGetLastError();
}

__global__ __launch_bounds__(kQT) void gelu_table_kernel(float *__restrict__ gelu_tab) {
    const int i = blockIdx.x * kQT + threadIdx.x;
    if (i < kGeluTabSize) gelu_tab[i] = gelu_table_entry(i);
}

hipError_t launch_gelu_table(float *gelu_tab, hipStream_t s) {
    hipLaunchKernelGGL(gelu_table_kernel, dim3((kGeluTabSize + kQT - 1) / kQT), dim3(kQT), 0, s,
                       gelu_tab);
    return hipGetLastError();
}

template <bool R_, bool C_, bool M_, bool T_, bool H_, bool G_ = false>
static void launch_q(const QuantParams &p, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((quant_kernel<R_, C_, M_, T_, H_, G_>), grid, dim3(kQT), 0, s, p);
}

hipError_t launch_quant_tile(const QuantParams &p, bool has_row, bool has_col, bool has_mx,
                             bool tile2d, bool rht, hipStream_t s, bool gelu) {
    const int64_t T = ((p.R + kTileR - 1) / kTileR) * ((p.C + kTileC - 1) / kTileC);
    const dim3 grid((unsigned)T);
    if (gelu) {
        if (has_col || tile2d || rht) return hipErrorInvalidValue;
        if (has_row && has_mx) launch_q<1, 0, 1, 0, 0, 1>(p, grid, s);
        else if (has_row) launch_q<1, 0, 0, 0, 0, 1>(p, grid, s);
        else if (has_mx) launch_q<0, 0, 1, 0, 0, 1>(p, grid, s);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    // The combinations the quantizer supports (RHT only on a 1x16 column copy).
    const int key = (has_row << 4) | (has_col << 3) | (has_mx << 2) | (tile2d << 1) | rht;
    switch (key) {
        case 0b10000: launch_q<1, 0, 0, 0, 0>(p, grid, s); break;
        case 0b10010: launch_q<1, 0, 0, 1, 0>(p, grid, s); break;
        case 0b11000: launch_q<1, 1, 0, 0, 0>(p, grid, s); break;
        case 0b11010: launch_q<1, 1, 0, 1, 0>(p, grid, s); break;
        case 0b11001: launch_q<1, 1, 0, 0, 1>(p, grid, s); break;
        case 0b01000: launch_q<0, 1, 0, 0, 0>(p, grid, s); break;
        case 0b01010: launch_q<0, 1, 0, 1, 0>(p, grid, s); break;
        case 0b01001: launch_q<0, 1, 0, 0, 1>(p, grid, s); break;
        case 0b00100: launch_q<0, 0, 1, 0, 0>(p, grid, s); break;
        case 0b10100: launch_q<1, 0, 1, 0, 0>(p, grid, s); break;
        case 0b10110: launch_q<1, 0, 1, 1, 0>(p, grid, s); break;
        case 0b01100: launch_q<0, 1, 1, 0, 0>(p, grid, s); break;
        case 0b01101: launch_q<0, 1, 1, 0, 1>(p, grid, s); break;
        case 0b11100: launch_q<1, 1, 1, 0, 0>(p, grid, s); break;
        case 0b11101: launch_q<1, 1, 1, 0, 1>(p, grid, s); break;
        case 0b01110: launch_q<0, 1, 1, 1, 0>(p, grid, s); break;
        case 0b11110: launch_q<1, 1, 1, 1, 0>(p, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool P_, bool F_, bool G_>
static void launch_act(const QuantParams &p, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((quant_act_kernel<P_, F_, G_>), grid, dim3(kQT), 0, s, p);
}

hipError_t launch_quant_act(const QuantParams &p, bool per_token, bool four_six, bool gelu,
                            hipStream_t s) {
    const dim3 grid((unsigned)((p.R + kQT / 64 - 1) / (kQT / 64)));
    switch ((per_token << 2) | (four_six << 1) | gelu) {
        case 0b110: launch_act<1, 1, 0>(p, grid, s); break;
        case 0b100: launch_act<1, 0, 0>(p, grid, s); break;
        case 0b010: launch_act<0, 1, 0>(p, grid, s); break;
        case 0b111: launch_act<1, 1, 1>(p, grid, s); break;
        case 0b101: launch_act<1, 0, 1>(p, grid, s); break;
        case 0b011: launch_act<0, 1, 1>(p, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_requant(const RequantParams &p, bool sr, hipStream_t s) {
    const int64_t T = ((p.R + kReqR - 1) / kReqR) * ((p.C + kReqC - 1) / kReqC);
    const dim3 grid((unsigned)T);
    if (sr && p.tile2d) hipLaunchKernelGGL((requant_kernel<true, true>), grid, dim3(kQT), 0, s, p);
    else if (sr) hipLaunchKernelGGL((requant_kernel<true, false>), grid, dim3(kQT), 0, s, p);
    else if (p.tile2d) hipLaunchKernelGGL((requant_kernel<false, true>), grid, dim3(kQT), 0, s, p);
    else hipLaunchKernelGGL((requant_kernel<false, false>), grid, dim3(kQT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_mxfp4_quant(const uint16_t *x, int64_t R, int64_t C, int64_t ld, uint8_t *codes,
                              uint8_t *scales, bool sr, uint64_t seed, uint32_t stream,
                              hipStream_t s) {
    const int64_t n = R * (C / 32);
    const dim3 grid((unsigned)((n + kQT - 1) / kQT));
    if (sr)
        hipLaunchKernelGGL(mx4_quant_kernel<true>, grid, dim3(kQT), 0, s, x, R, C, ld, codes,
                           scales, seed, stream);
    else
        hipLaunchKernelGGL(mx4_quant_kernel<false>, grid, dim3(kQT), 0, s, x, R, C, ld, codes,
                           scales, seed, stream);
    return hipGetLastError();
}

}  // namespace bbs

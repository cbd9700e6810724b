// NVFP4 quantizer and MXFP8 requantizer kernels (gfx950).
//
// Quantize (Pretraining LLMs with NVFP4, "NVFP4 Format and Quantization
// Procedure", steps 1-4; 4bit.vizuara.ai sections 5-6, 13):
//   pass 1  amax_kernel: per-workgroup maxima of |x| and / or of the RHT'd
//           16-row column chunks, from one read of x; no atomics, no zeroing.
//           A wave reads 16 rows x 256 columns per step (each load two
//           512-byte runs of two rows) and loads its next step while
//           reducing this one.
//   pass 2  quant_kernel: every workgroup folds the partials into the tensor
//           amax (bit-identical everywhere) and walks a run of 256-row x
//           128-column tiles of x, loading the next tile while it encodes
//           this one.  A workgroup has 512 threads and a thread owns an
//           8 x 8 piece of a tile, loaded as 8 rows of 16 bytes.  From that
//           one read it writes any of: the row-wise NVFP4 copy (a 1x16 block
//           is two neighbouring lanes), the column-wise NVFP4 copy of x^T
//           (lanes l and l ^ 16 hold the two halves of a 16 x 8 block and
//           trade halves, after which each encodes four full column blocks,
//           optional RHT; without row-wise copies a thread loads a 16 x 4
//           piece instead and needs no exchange), and the row-wise MXFP8
//           copy (a block of 32 is four lanes).  The column copy's codes and
//           every copy's block scales are gathered in LDS and written as
//           whole runs: each transposed row's 128 code bytes of a tile are
//           one store of eight lanes.  Block encode scales 1 / (E4M3 x
//           s_dec) come from a table of the 127 E4M3 codes built once per
//           workgroup.
// Requantize (4bit.vizuara.ai sections 9-10): requant_kernel dequantizes a
// 16-row x 8-column piece of an NVFP4 matrix in FP32 per lane and encodes
// its half of 8 transposed rows of 32 as MXFP8 (E8M0 per 32 shared by a lane
// pair, E4M3 elements, RTN or SR); a workgroup's 256 destination rows x 128
// bytes are gathered in LDS and stored as whole rows.
//
// Workgroups are mapped to tiles so that each of the 8 XCDs works through a
// contiguous run of tiles (neighbouring tiles share output lines in L2).
#include <type_traits>

#include "bbs_device.hpp"
#include "bbs_kernels.hpp"

namespace bbs {

constexpr int kQT = 256;                       // threads per workgroup
constexpr int kET = 512;                       // threads of the tile encode kernel
constexpr int kTileR = 256, kTileC = 128;      // quantizer tile of x
constexpr int kReqR = 128, kReqC = 256;        // requantizer tile of the source
static_assert(kReqC == kQT, "one scale row per thread");

static_assert(kGeluTabOffset + kGeluTabSize <= kWorkspaceFloats, "GELU table exceeds the workspace");
static_assert(kQT == 256, "the partial fold assumes four waves");
static_assert(kGeluTabOffset % 4 == 0, "GELU table must stay 16-byte aligned");

// Tile t of T when workgroup b runs on XCD b % 8: XCD x takes a contiguous
// run of tiles.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t T) {
    const int64_t x = b % 8, j = b / 8, per = T / 8, rem = T % 8;
    return x * per + (x < rem ? x : rem) + j;
}

// The tiles a workgroup of a persistent grid walks: the workgroups of XCD
// b % 8 share that XCD's contiguous eighth of the tiles, taking every
// (workgroups on the XCD)-th one.  Grids of fewer than 8 workgroups stride
// over all tiles.
struct TileWalk {
    int64_t first, end, step;
};
__device__ __forceinline__ TileWalk xcd_walk(int64_t T) {
    const int64_t G = gridDim.x, b = blockIdx.x;
    if (G < 8) return {b, T, G};
    const int64_t x = b % 8, j = b / 8, per = T / 8, rem = T % 8;
    const int64_t lo = x * per + (x < rem ? x : rem);
    const int64_t hi = lo + per + (x < rem ? 1 : 0);
    const int64_t gx = G / 8 + (x < G % 8 ? 1 : 0);
    return {lo + j, hi, gx};
}

// A thread's piece of a quantizer tile; wave w holds the 16-row bands 2w
// and 2w + 1 (lanes 0-31 and 32-63).
//   with row-wise copies: the 8 x 8 piece half `half` of band `band`,
//     columns 8 cg .. 8 cg + 7 (v[i] = row i); the two halves of a band's
//     16 x 8 block are lanes l and l ^ 16.
//   column copy only (CO): the 16 x 4 piece of band `band`, columns
//     4 cg .. 4 cg + 3 (words 0-1 of v[i] = row i, words 2-3 = row i + 8).
// col0 is the first of the four columns whose 16-row blocks the lane
// encodes for the column copy.
struct Piece {
    int64_t R0, C0;   // the tile's first row / column
    int64_t r0, c0;   // the piece's first row / column
    int band, half, cg, col0;
    bool in;          // the piece lies inside x (R, C are multiples of 16)
};

template <bool CO>
__device__ __forceinline__ Piece piece_of(int64_t tile, int64_t R, int64_t C) {
    const int64_t tiles_c = (C + kTileC - 1) / kTileC;
    const int64_t tr = tile / tiles_c;
    Piece q;
    q.R0 = tr * kTileR;
    q.C0 = (tile - tr * tiles_c) * kTileC;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    q.band = w * 2 + (lane >> 5);
    if (CO) {
        q.half = 0;
        q.cg = lane & 31;
        q.r0 = q.R0 + q.band * 16;
        q.c0 = q.C0 + q.cg * 4;
        q.col0 = q.cg * 4;
    } else {
        q.half = (lane >> 4) & 1;
        q.cg = lane & 15;
        q.r0 = q.R0 + q.band * 16 + q.half * 8;
        q.c0 = q.C0 + q.cg * 8;
        q.col0 = q.cg * 8 + q.half * 4;
    }
    q.in = q.R0 + q.band * 16 < R && q.c0 < C;
    return q;
}

// 8 rows of 16 bytes, or (CO) 16 rows of 8 bytes.  A piece outside x reads a
// valid piece instead (its results are never stored), so the loads need no
// branches.
template <bool CO>
__device__ __forceinline__ void load_piece(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                           const Piece &q, uint4 v[8]) {
    if (CO) {
        const int64_t r = q.r0 < R ? q.r0 : R - 16;
        const int64_t c = q.c0 < C ? q.c0 : C - 4;
        const uint16_t *src = x + r * ld + c;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint2 a = *reinterpret_cast<const uint2 *>(src + i * ld);
            const uint2 b = *reinterpret_cast<const uint2 *>(src + (i + 8) * ld);
            v[i] = make_uint4(a.x, a.y, b.x, b.y);
        }
    } else {
        const int64_t r = q.r0 < R ? q.r0 : R - 8;
        const int64_t c = q.c0 < C ? q.c0 : C - 8;
        const uint16_t *src = x + r * ld + c;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const uint4 *>(src + i * ld);
    }
}

// v_permlane16_swap: in each 32-lane group, lanes 16-31 of a trade places
// with lanes 0-15 of b.  Lanes l and l ^ 16 hold the two halves of a 16-row
// block, so this is how they exchange data.
__device__ __forceinline__ void swap_halves(uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// max(v of lane l, v of lane l ^ 16)
__device__ __forceinline__ float max_half_pair(float v) {
    uint32_t a = __float_as_uint(v), b = a;
    swap_halves(a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// Element j (compile-time) of a row of 8 BF16 values, as FP32.
__device__ __forceinline__ float elem(const uint4 &row, int j) {
    const uint32_t w = j < 2 ? row.x : (j < 4 ? row.y : (j < 6 ? row.z : row.w));
    return (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}

// The same with the sign flipped when sg (0 or 0x80000000) is set, as one
// integer operation (for an even j, adding sg to w << 16 flips bit 31 alone).
// The RHT's sign flips are applied here, and its butterflies then called
// with no signs.
__device__ __forceinline__ float elem_flip(const uint4 &row, int j, uint32_t sg) {
    const uint32_t w = j < 2 ? row.x : (j < 4 ? row.y : (j < 6 ? row.z : row.w));
    return __uint_as_float((j & 1) ? ((w & 0xFFFF0000u) ^ sg) : ((w << 16) + sg));
}
__device__ __forceinline__ uint32_t sign_bit(uint32_t signs, int i) {
    return ((signs >> i) & 1u) << 31;
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
// A wave step covers 16 rows x 512 columns: lane l reads columns
// 8l .. 8l + 7 of each row (one 16-byte load per row), so a load of the wave
// is a 1 KB run of one row and the lane holds eight full 16-row column
// chunks for the RHT.  Steps past the last column (C % 512 != 0) read a
// valid piece and are not counted.
// ---------------------------------------------------------------------------
// GELU: the partials are maxima of |GELU(x)|, found without evaluating GELU
// on most elements.  GELU is non-decreasing for x >= 0, so the largest value
// over the non-negative elements is GELU of their maximum; every negative
// element has |GELU| < kGeluNegBound, so the negative elements of a wave's
// pieces are evaluated only when GELU of the wave's largest element is below
// that bound (wave-uniform branch).  The result is the exact maximum.
constexpr int kAmaxStepC = 512;

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
    // a wave step is 16 rows x 256 columns: lane l holds 8 columns of rows
    // 8 (l >> 5) .. + 7; for the RHT maxima lanes l and l ^ 32 trade halves.
    // (GELU: 16 rows x 512 columns, lane l all 16 rows of its 8 columns.)
    constexpr int SC = GELU ? kAmaxStepC : kAmaxStepC / 2, PR = GELU ? 16 : 8;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int hf = GELU ? 0 : lane >> 5, cl = GELU ? lane : lane & 31;
    const int64_t steps_c = (C + SC - 1) / SC;
    const int64_t T = (R / 16) * steps_c;
    const int64_t stride = (int64_t)gridDim.x * (kQT / 64);
    float m = 0.0f, mr = 0.0f;
    float mx = 0.0f;     // GELU: largest element seen (0 if none is positive)
    auto load = [&](int64_t t, uint4 d[PR]) -> bool __attribute__((always_inline)) {
        const int64_t tr = t / steps_c;
        int64_t c = (t - tr * steps_c) * SC + cl * 8;
        const bool ok = c < C;
        if (!ok) c = C - 8;
        const uint16_t *src = x + (tr * 16 + hf * 8) * ld + c;
#pragma unroll
        for (int i = 0; i < PR; ++i) d[i] = *reinterpret_cast<const uint4 *>(src + i * ld);
        return ok;
    };
    int64_t t = (int64_t)blockIdx.x * (kQT / 64) + w;
    uint4 v[PR];
    bool ok = t < T ? load(t, v) : false;
    while (t < T) {                                   // wave-uniform
        const int64_t tn = t + stride;
        uint4 vn[PR];
        const bool okn = tn < T ? load(tn, vn) : false;
        if (ok) {
        if (PLAIN) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem(v[r], j)));
        }
        if (RHT) {
            // (the partner lane has the same columns, so the same ok):
            // words 0-1 of v[i] then hold row i, words 2-3 row i + 8, of the
            // lane's four columns 4 hf .. + 3
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const auto a = __builtin_amdgcn_permlane32_swap(v[i].x, v[i].z, false, false);
                const auto b = __builtin_amdgcn_permlane32_swap(v[i].y, v[i].w, false, false);
                v[i] = make_uint4(a[0], b[0], a[1], b[1]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float y[16];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    y[r] = elem_flip(v[r], j, sign_bit(signs, r));
                    y[r + 8] = elem_flip(v[r], 4 + j, sign_bit(signs, r + 8));
                }
                rht16_butterflies(y, 0u);
#pragma unroll
                for (int r = 0; r < 16; ++r) mr = fmaxf(mr, fabsf(y[r]));
            }
        }
        }
        if (GELU) {
            float pm = 0.0f;
            if (ok) {
#pragma unroll
                for (int r = 0; r < PR; ++r)
#pragma unroll
                    for (int j = 0; j < 8; ++j) pm = fmaxf(pm, elem(v[r], j));
            }
            mx = fmaxf(mx, pm);
            if (gelu_tanh(wave_max(pm)) < kGeluNegBound && ok) {
#pragma unroll
                for (int r = 0; r < PR; ++r)
#pragma unroll
                    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(gelu_tanh(elem(v[r], j))));
            }
        }
        t = tn;
        ok = okn;
#pragma unroll
        for (int i = 0; i < PR; ++i) v[i] = vn[i];
    }
    // The transform's final multiply by 1/4 is monotonic, so the maximum of
    // the scaled values is the scaled maximum (bit for bit).
    mr = mr * 0.25f;
    if (GELU) m = fmaxf(m, gelu_tanh(mx));
    m = wave_max(m);
    mr = wave_max(mr);
    if (lane == 0) {
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

// A thread's share of n <= kAmaxPartials amax partials, NT threads taking
// every NT-th: all its loads are issued before any value is used, so they
// cost one memory round trip, and, issued ahead of a tile's loads, they are
// waited on without waiting for the tile (the memory counter drains in
// order of issue).
template <int NT>
struct PartShare {
    static constexpr int K = kAmaxPartials / NT;
    float v[K];
    __device__ __forceinline__ void load(const float *part, int n) {
        const int t = (int)threadIdx.x % NT;
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = t + k * NT < n ? part[t + k * NT] : 0.0f;
    }
    __device__ __forceinline__ float max() const {
        float m = v[0];
#pragma unroll
        for (int k = 1; k < K; ++k) m = fmaxf(m, v[k]);
        return m;
    }
};

// The GELU table, workspace -> LDS, by asynchronous LDS copies (no
// registers, no wait per load): wave w of the NT threads copies the 1 KB
// chunks w, w + NT / 64, ...  The caller waits for the vector memory counter
// to drain, then synchronises, before the first lookup.
template <int NT>
__device__ __forceinline__ void gelu_table_copy(float *lds, const float *tab) {
    constexpr int kChunks = kGeluTabSize * 4 / 1024, kWaves = NT / 64;
    static_assert(kGeluTabSize % 256 == 0, "whole 1 KB chunks");
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < (kChunks + kWaves - 1) / kWaves; ++k) {
        const int c = w + k * kWaves;
        if (c < kChunks) copy_lds16(tab + c * 256 + lane * 4, lds + c * 256);
    }
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// The tensor amax: the maximum of n <= kAmaxPartials partials, in every lane
// (the first 256 in one round trip, any others in a loop).
__device__ __forceinline__ float fold_partials(const float *part, int n) {
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = (threadIdx.x & 63) + 64 * k;
        v[k] = i < n ? part[i] : 0.0f;
    }
    float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    for (int i = (threadIdx.x & 63) + 256; i < n; i += 64) m = fmaxf(m, part[i]);
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

// LDS of the encode kernel.  The column copy's codes: 128 transposed rows of
// 128 bytes, 16-byte groups swizzled by (row >> 3) & 7 so that the eight
// lanes writing one group index hit different banks.
template <bool GELU>
struct QuantLds {
    uint8_t row[kTileR * 8];           // row copy scales (1x16; 16x16 uses 16 x 8)
    uint8_t col[kTileC * 16];          // column copy scales
    uint8_t mx[kTileR * 4];            // MXFP8 scales
    uint8_t colc[kTileC * 128];        // column copy codes
    float tab[2][128];                 // encode scale per E4M3 code: row, column copy
    float fold[2][kET / 64];           // per-wave maxima of the amax partials
    float gelu[GELU ? kGeluTabSize : 1];
};
__device__ __forceinline__ int colc_off(int row, int group) {
    return row * 128 + ((group ^ ((row >> 3) & 7)) << 4);
}

// Encode one tile (piece q, values v) into every requested copy.  Every
// thread of the workgroup calls it (two barriers inside).  The column copy
// rearranges v.
// SR: some copy rounds stochastically (else every copy rounds to nearest and
// the stochastic paths are not compiled).
template <bool HAS_ROW, bool HAS_COL, bool HAS_MX, bool TILE2D, bool RHT, bool GELU, bool SR>
__device__ __forceinline__ void encode_tile(const QuantParams &p, const Piece &q,
                                            uint4 (&v)[8], float s_enc_row,
                                            float s_enc_col, QuantLds<GELU> &L) {
    const int lane = threadIdx.x & 63;
    constexpr bool CO = !HAS_ROW && !HAS_MX;
    // Element j of row r of the piece, as the row-wise copies see it (GELU:
    // looked up where it is used, so the piece stays in its BF16 registers).
    auto val = [&](int r, int j) -> float {
        if constexpr (GELU) return gelu_bf16(elem_bits(v[r], j), L.gelu);
        else return elem(v[r], j);
    };

    // 16x16 tile amax (lanes l, l ^ 1, l ^ 16, l ^ 17 hold one tile; CO: four
    // neighbouring lanes; TILE2D excludes RHT).
    float tile_amax = 0.0f;
    if (TILE2D) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) tile_amax = fmaxf(tile_amax, fabsf(elem(v[r], j)));
        tile_amax = CO ? max_lane_quad(tile_amax) : max_half_pair(max_lane_pair(tile_amax));
    }
    const int prow = q.band * 16 + q.half * 8;       // the piece's first row in the tile

    // ---- row-wise copies (NVFP4 and MXFP8), one row of the piece at a time ----
    uint32_t tsc = 0;
    float ts = 0.0f;
    if (HAS_ROW && TILE2D) {
        tsc = block_scale_code(tile_amax, s_enc_row);
        ts = L.tab[0][tsc];
    }
    // counters of the first row's Philox blocks; each further row adds C / 8
    const uint64_t n_row0 = (uint64_t)(q.r0 * p.C + q.c0) / 8;
    const uint64_t n_step = (uint64_t)p.C / 8;
    // NVFP4 copy of row r of the piece (values f)
    auto row_copy = [&](auto sr_tag, int r, const float f[8]) {
        constexpr bool RSR = decltype(sr_tag)::value;
        uint32_t sc = tsc;
        float s = ts;
        if (!TILE2D) {
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
            sc = block_scale_code(max_lane_pair(a), s_enc_row);
            s = L.tab[0][sc];
            if ((lane & 1) == 0) L.row[(prow + r) * 8 + (q.cg >> 1)] = (uint8_t)sc;
        }
        uint32_t packed;
        if constexpr (RSR) {
            uint32_t w[4];
            sr_block(p.row_seed, p.row_stream, n_row0 + (uint64_t)r * n_step, w);
            packed = e2m1_sr8(f, s, w);
        } else {
            packed = e2m1_rne8(f, s);
        }
        if (q.in) *reinterpret_cast<uint32_t *>(p.row_codes + (q.r0 + r) * (p.C / 2) + q.c0 / 2) =
            packed;
    };
    // MXFP8 copy of row r of the piece (values f): the block's power of two
    // rides in the conversion's scale operand
    auto mx_copy = [&](auto sr_tag, int r, const float (&f)[8]) {
        constexpr bool MSR = decltype(sr_tag)::value;
        float y[8];
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[j] = f[j];
            a = fmaxf(a, fabsf(f[j]));
        }
        const uint32_t kb = e8m0_byte(max_lane_quad(a));
        if (__builtin_amdgcn_ballot_w64(kb == 0)) {   // rare, wave-uniform test
            if (kb == 0) {                             // 2^-127: convert 2y at 2^-126
#pragma unroll
                for (int j = 0; j < 8; ++j) y[j] = y[j] * 2.0f;
            }
        }
        const float cs = e8m0_cvt_scale(kb);
        uint32_t lo, hi;
        if constexpr (MSR) {
            uint32_t w[4];
            sr_block(p.mx_seed, p.mx_stream, n_row0 + (uint64_t)r * n_step, w);
            lo = e4m3_sr4_scaled(y[0], y[1], y[2], y[3], sr_word_lo(w[0]), sr_word_hi(w[0]),
                                 sr_word_lo(w[1]), sr_word_hi(w[1]), cs);
            hi = e4m3_sr4_scaled(y[4], y[5], y[6], y[7], sr_word_lo(w[2]), sr_word_hi(w[2]),
                                 sr_word_lo(w[3]), sr_word_hi(w[3]), cs);
        } else {
            lo = e4m3_rne4_scaled(y[0], y[1], y[2], y[3], cs);
            hi = e4m3_rne4_scaled(y[4], y[5], y[6], y[7], cs);
        }
        if (q.in) *reinterpret_cast<uint2 *>(p.mx_codes + (q.r0 + r) * p.C + q.c0) = make_uint2(lo, hi);
        if ((lane & 3) == 0) L.mx[(prow + r) * 4 + (q.cg >> 2)] = (uint8_t)kb;
    };
    auto rows = [&](auto row_sr, auto mx_sr) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            float f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = val(r, j);
            if (HAS_ROW) row_copy(row_sr, r, f);
            if (HAS_MX) mx_copy(mx_sr, r, f);
        }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (HAS_ROW || HAS_MX) {
        if constexpr (SR) {
            const bool row_sr = HAS_ROW && p.row_round == 1, mx_sr = HAS_MX && p.mx_round == 1;
            if (row_sr && mx_sr) rows(T_{}, T_{});
            else if (row_sr) rows(T_{}, F_{});
            else if (mx_sr) rows(F_{}, T_{});
            else rows(F_{}, F_{});
        } else {
            rows(F_{}, F_{});
        }
    }
    if (HAS_ROW && TILE2D && (lane & 17) == 0) L.row[q.band * 8 + (q.cg >> 1)] = (uint8_t)tsc;

    // ---- column-wise NVFP4 copy (of x^T) ---------------------------------------
    if (HAS_COL) {
        uint32_t csc = 0;
        float cts = 0.0f;
        if (TILE2D) {
            csc = block_scale_code(tile_amax, s_enc_col);
            cts = L.tab[1][csc];
        }
        // Lanes l and l ^ 16 hold rows 0-7 and 8-15 of one 16 x 8 block; after
        // one exchange lane l (half 0) holds columns 0-3 of all 16 rows and
        // lane l ^ 16 columns 4-7: words 0-1 of v[i] are row i, words 2-3 row
        // i + 8, of the lane's four columns (the layout CO pieces load).
        if (!CO) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                swap_halves(v[i].x, v[i].z);
                swap_halves(v[i].y, v[i].w);
            }
        }
        const int col0 = q.col0;
        // FUSE: the RHT's 1/4 rides in the block's encode scale.  The block
        // amax is max |y| / 4 either way (rounding is monotonic), and
        // (y / 4) s = y (s / 4) is one rounding of the same product while y / 4
        // and s / 4 are exact; the caller takes the separate multiply unless
        // the tensor scale bounds every s to [2^-109, 2^89], where an inexact
        // y / 4 (|y| < 2^-124) gives a product far below any code's threshold.
        auto cols = [&](auto sr_tag, auto fuse_tag) {
            constexpr bool CSR = decltype(sr_tag)::value;
            constexpr bool FUSE = decltype(fuse_tag)::value;
            // counter of the first block of the lane's first column in this
            // band; each further column adds R / 8
            const uint64_t n0 = (uint64_t)((q.C0 + col0) * p.R + q.R0 + q.band * 16) / 8;
            const uint64_t nstep = (uint64_t)p.R / 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // column copy alone (registers to spare): the column's random
                // words first, which do not depend on the values, so they
                // overlap the transform and the scale (which ends in a rarely
                // taken branch)
                constexpr bool EARLY = CSR && !HAS_ROW && !HAS_MX;
                uint32_t wr0[4], wr1[4];
                const uint64_t n = n0 + (uint64_t)j * nstep;
                if constexpr (EARLY) {
                    sr_block(p.col_seed, p.col_stream, n, wr0);
                    sr_block(p.col_seed, p.col_stream, n + 1, wr1);
                }
                float y[16];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    if (RHT) {
                        y[r] = elem_flip(v[r], j, sign_bit(p.rht_signs, r));
                        y[r + 8] = elem_flip(v[r], 4 + j, sign_bit(p.rht_signs, r + 8));
                    } else {
                        y[r] = elem(v[r], j);
                        y[r + 8] = elem(v[r], 4 + j);
                    }
                }
                if (RHT) {
                    rht16_butterflies(y, 0u);
                    if (!FUSE) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) y[r] = y[r] * 0.25f;
                    }
                }
                uint32_t sc = csc;
                float s = cts;
                if (!TILE2D) {
                    float a = 0.0f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(y[r]));
                    if (FUSE) a = a * 0.25f;
                    sc = block_scale_code(a, s_enc_col);
                    s = L.tab[1][sc];
                    L.col[(col0 + j) * 16 + q.band] = (uint8_t)sc;
                }
                if (FUSE) s = s * 0.25f;
                uint32_t w0, w1;
                if constexpr (CSR) {
                    if constexpr (!EARLY) sr_block(p.col_seed, p.col_stream, n, wr0);
                    w0 = e2m1_sr8(y, s, wr0);
                    if constexpr (!EARLY) sr_block(p.col_seed, p.col_stream, n + 1, wr1);
                    w1 = e2m1_sr8(y + 8, s, wr1);
                } else {
                    w0 = e2m1_rne8(y, s);
                    w1 = e2m1_rne8(y + 8, s);
                }
                // transposed row col0 + j of the tile, bytes band * 8 .. + 7
                const int trow = col0 + j;
                *reinterpret_cast<uint2 *>(L.colc + colc_off(trow, q.band >> 1) + (q.band & 1) * 8) =
                    make_uint2(w0, w1);
            }
        };
        const bool fuse = RHT && !TILE2D && s_enc_col >= 0x1p-100f && s_enc_col <= 0x1p80f;
        auto cols_r = [&](auto sr_tag) {
            if constexpr (RHT && !TILE2D) {
                if (fuse) cols(sr_tag, T_{});
                else cols(sr_tag, F_{});
            } else {
                cols(sr_tag, F_{});
            }
        };
        if constexpr (SR) {
            if (p.col_round == 1) cols_r(T_{});
            else cols_r(F_{});
        } else {
            cols_r(F_{});
        }
        if (TILE2D && (CO ? (lane & 3) == 0 : (lane & 17) == 0))
            L.col[(col0 >> 4) * 16 + q.band] = (uint8_t)csc;
    }

    // ---- column codes and block scales, as whole runs -------------------------
    __syncthreads();
    const int t = threadIdx.x;
    const int64_t nb_row = (p.C - q.C0) / 16, nb_col = (p.R - q.R0) / 16;
    if (HAS_COL) {
        // 128 transposed rows x 16 halves of 8 bytes (16 source rows each):
        // 4 passes of 512 threads, 16 lanes per 128-byte row
        const int64_t rows_in = p.C - q.C0 < kTileC ? p.C - q.C0 : kTileC;
        const int64_t halves_in = (p.R - q.R0) / 16;              // bands inside x
#pragma unroll
        for (int i = 0; i < kTileC * 16 / kET; ++i) {
            const int idx = i * kET + t, trow = idx >> 4, h = idx & 15;
            if (trow < rows_in && h < halves_in)
                *reinterpret_cast<uint2 *>(p.col_codes + (q.C0 + trow) * (p.R / 2) + q.R0 / 2 + h * 8) =
                    *reinterpret_cast<const uint2 *>(L.colc + colc_off(trow, h >> 1) + (h & 1) * 8);
        }
    }
    if (HAS_ROW) {
        if (!TILE2D) {
            if (t < kTileR && q.R0 + t < p.R)
                put_run<8>(p.row_scales + (q.R0 + t) * (p.C / 16) + q.C0 / 16, L.row + t * 8,
                           nb_row < 8 ? nb_row : 8);
        } else if (t < 16 && q.R0 / 16 + t < p.R / 16) {
            put_run<8>(p.row_scales + (q.R0 / 16 + t) * (p.C / 16) + q.C0 / 16, L.row + t * 8,
                       nb_row < 8 ? nb_row : 8);
        }
    }
    if (HAS_MX && t < kTileR && q.R0 + t < p.R) {
        const int64_t nb = (p.C - q.C0) / 32;
        put_run<4>(p.mx_scales + (q.R0 + t) * (p.C / 32) + q.C0 / 32, L.mx + t * 4,
                   nb < 4 ? nb : 4);
    }
    if (HAS_COL) {
        if (!TILE2D) {
            if (t < kTileC && q.C0 + t < p.C)
                put_run<16>(p.col_scales + (q.C0 + t) * (p.R / 16) + q.R0 / 16, L.col + t * 16,
                            nb_col < 16 ? nb_col : 16);
        } else if (t < kTileC / 16 && q.C0 / 16 + t < p.C / 16) {
            put_run<16>(p.col_scales + (q.C0 / 16 + t) * (p.R / 16) + q.R0 / 16, L.col + t * 16,
                        nb_col < 16 ? nb_col : 16);
        }
    }
    __syncthreads();                       // LDS is rewritten by the next tile
}

// GELU: the row-wise copies are of GELU(x), evaluated once per element in
// FP32 (the pages' fused activation + quantize); the amax partials are those
// of |GELU(x)|.
// WALK = false: one tile per workgroup (XCD-contiguous mapping), registers
// capped for MINW waves per SIMD.  WALK = true: a resident grid walks runs
// of tiles, loading the next tile while it encodes the current one.
template <bool HAS_ROW, bool HAS_COL, bool HAS_MX, bool TILE2D, bool RHT, bool GELU, bool SR,
          bool WALK, int MINW>
__global__ __launch_bounds__(kET, MINW) void quant_kernel(QuantParams p) {
    static_assert(!GELU || (!HAS_COL && !TILE2D && !RHT), "GELU feeds the row-wise copies");
    __shared__ __align__(16) QuantLds<GELU> L;
    const int64_t T = ((p.R + kTileR - 1) / kTileR) * ((p.C + kTileC - 1) / kTileC);
    const TileWalk walk = WALK ? xcd_walk(T) : TileWalk{xcd_tile(blockIdx.x, T), 0, 1};
    // Tensor scales, identical in every wave: the partials are folded once
    // per workgroup (each thread a strided share, then the eight waves),
    // while the first tile's piece, loaded after them, is in flight.
    constexpr bool plain_amax = HAS_ROW || (HAS_COL && !RHT);
    // (the tile's arguments are read with the partials', not a round trip
    // after them)
    asm volatile("" ::"s"(p.x), "s"(p.R), "s"(p.C), "s"(p.ld), "s"(p.part), "s"(p.n_part));
    PartShare<kET> pa, pb;
    if (plain_amax) pa.load(p.part, p.n_part);
    if (HAS_COL && RHT) pb.load(p.part_rht, p.n_part_rht);
    uint4 v[8];
    constexpr bool CO = !HAS_ROW && !HAS_MX;
    Piece q = piece_of<CO>(!WALK || walk.first < walk.end ? walk.first : 0, p.R, p.C);
    // (unconditional, so that the fold's wait can leave these loads in flight
    // on every path: a workgroup without tiles loads tile 0, which always
    // exists, and never uses it)
    load_piece<CO>(p.x, p.R, p.C, p.ld, q, v);
    __builtin_amdgcn_sched_barrier(0);      // every load issued before the fold waits
    {
        float a = plain_amax ? pa.max() : 0.0f, b = HAS_COL && RHT ? pb.max() : 0.0f;
        a = wave_max(a);
        b = wave_max(b);
        if ((threadIdx.x & 63) == 0) {
            L.fold[0][threadIdx.x >> 6] = a;
            L.fold[1][threadIdx.x >> 6] = b;
        }
    }
    __syncthreads();
    float fa = L.fold[0][0], fb = L.fold[1][0];
#pragma unroll
    for (int i = 1; i < kET / 64; ++i) {
        fa = fmaxf(fa, L.fold[0][i]);
        fb = fmaxf(fb, L.fold[1][i]);
    }
    float s_enc_row = 1.0f, s_enc_col = 1.0f;
    if (plain_amax) s_enc_row = tensor_s_enc(fa);
    if (HAS_COL) s_enc_col = RHT ? tensor_s_enc(fb) : s_enc_row;
    const float s_dec_row = 1.0f / s_enc_row;
    const float s_dec_col = 1.0f / s_enc_col;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (HAS_ROW) p.row_sdec[0] = s_dec_row;
        if (HAS_COL) p.col_sdec[0] = s_dec_col;
    }
    if (HAS_ROW) enc_scale_table(L.tab[0], s_dec_row);
    if (HAS_COL) enc_scale_table(L.tab[1], s_dec_col);
    if constexpr (GELU) {
        gelu_table_copy<kET>(L.gelu, p.gelu_tab);
        wait_vmem();
    }
    __syncthreads();

    if constexpr (!WALK) {
        encode_tile<HAS_ROW, HAS_COL, HAS_MX, TILE2D, RHT, GELU, SR>(p, q, v, s_enc_row, s_enc_col,
                                                                     L);
    } else {
        for (int64_t t = walk.first; t < walk.end; t += walk.step) {     // workgroup-uniform
            const int64_t tn = t + walk.step;
            uint4 vn[8];
            Piece qn = q;
            if (tn < walk.end) {
                qn = piece_of<CO>(tn, p.R, p.C);
                load_piece<CO>(p.x, p.R, p.C, p.ld, qn, vn);
            }
            encode_tile<HAS_ROW, HAS_COL, HAS_MX, TILE2D, RHT, GELU, SR>(p, q, v, s_enc_row,
                                                                         s_enc_col, L);
            q = qn;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = vn[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Row-wise copies only (no column copy): the NVFP4 row copy (1x16 or 16x16
// tiles) and / or the MXFP8 row copy.  A wave step covers 16 rows x 512
// columns, lane l holding columns 8l .. 8l + 7 of each row, so each row's
// codes go out as one 256-byte (NVFP4) or 512-byte (MXFP8) store of the wave
// and its block scales as 4-byte words gathered across lanes.  Waves walk
// the steps with a stride of the whole grid, loading the next step while
// they encode the current one.
// ---------------------------------------------------------------------------
struct RowsLds {
    float tab[128];
    float fold[kQT / 64];
};

// Scale bytes of lanes l, l + d, l + 2d, l + 3d as one little-endian word (in
// lane l).
__device__ __forceinline__ uint32_t gather4(uint32_t b, int d) {
    const uint32_t b1 = __shfl_down(b, d, 64), b2 = __shfl_down(b, 2 * d, 64),
                   b3 = __shfl_down(b, 3 * d, 64);
    return (b & 0xFFu) | ((b1 & 0xFFu) << 8) | ((b2 & 0xFFu) << 16) | ((b3 & 0xFFu) << 24);
}

// Store the scale bytes of `per` consecutive lanes' blocks (one byte per d
// lanes, starting at lane l0 of a group of 4d lanes) at dst[0..3]: one word
// when the group is inside the row and 4-byte aligned, else byte stores.
__device__ __forceinline__ void put_scales4(uint8_t *dst, uint32_t word, int64_t nvalid) {
    if (nvalid >= 4 && (reinterpret_cast<uintptr_t>(dst) & 3) == 0) {
        *reinterpret_cast<uint32_t *>(dst) = word;
    } else {
        for (int64_t i = 0; i < nvalid && i < 4; ++i) dst[i] = (uint8_t)(word >> (8 * i));
    }
}

// AP / AR: the kernel is also the amax pass of a quantize whose other copies
// need the tensor scale: it writes the MXFP8 copy (which needs none) and the
// per-workgroup partials of |x| (AP) and of |RHT(column chunks)| (AR), as
// amax_kernel does, from the same read.
// HALF (the amax pass variants): a wave step is 16 rows x 256 columns, lane
// l holding 8 columns of rows 8 (l >> 5) .. + 7, so the step takes half the
// registers; for the RHT partials lanes l and l ^ 32 trade halves
// (v_permlane32_swap) after the MXFP8 copy, each then holding four whole
// 16-row column blocks.
template <bool HAS_ROW, bool HAS_MX, bool TILE2D, bool GELU, bool SR, int MINW, bool AP = false,
          bool AR = false, bool HALF = false>
__global__ __launch_bounds__(kQT, MINW) void quant_rows_kernel(QuantParams p, float *amax_part,
                                                               float *amax_part_rht) {
    static_assert(!(AP || AR) || (!HAS_ROW && !GELU), "the amax pass feeds the later copies");
    static_assert(!HALF || (!HAS_ROW && !GELU), "half steps serve the amax pass variants");
    constexpr int PR = HALF ? 8 : 16;                        // rows per lane
    constexpr int SC = HALF ? kAmaxStepC / 2 : kAmaxStepC;   // columns per wave step
    __shared__ __align__(16) RowsLds L;
    __shared__ __align__(16) float s_gelu[GELU ? kGeluTabSize : 1];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int hf = HALF ? lane >> 5 : 0, cl = HALF ? lane & 31 : lane;
    const int64_t steps_c = (p.C + SC - 1) / SC;
    const int64_t T = (p.R / 16) * steps_c;
    const int64_t stride = (int64_t)gridDim.x * (kQT / 64);
    auto load = [&](int64_t t, uint4 d[PR], int64_t &r0, int64_t &c0) {
        const int64_t tr = t / steps_c;
        r0 = tr * 16 + hf * 8;
        c0 = (t - tr * steps_c) * SC + cl * 8;
        const uint16_t *src = p.x + r0 * p.ld + (c0 < p.C ? c0 : p.C - 8);
#pragma unroll
        for (int i = 0; i < PR; ++i) d[i] = *reinterpret_cast<const uint4 *>(src + i * p.ld);
    };
    // the tensor scale (row copy): partials folded once per workgroup while
    // the first step, loaded after them, is in flight
    asm volatile("" ::"s"(p.x), "s"(p.R), "s"(p.C), "s"(p.ld), "s"(p.part), "s"(p.n_part));
    PartShare<kQT> pa;
    if (HAS_ROW) pa.load(p.part, p.n_part);
    int64_t t = (int64_t)blockIdx.x * (kQT / 64) + w;
    uint4 v[PR];
    int64_t r0 = 0, c0 = 0;
    if (HAS_ROW) load(t < T ? t : 0, v, r0, c0);     // (step 0 always exists; see quant_kernel)
    else if (t < T) load(t, v, r0, c0);
    __builtin_amdgcn_sched_barrier(0);
    float s_enc = 1.0f;
    if (HAS_ROW) {
        float a = wave_max(pa.max());
        if (lane == 0) L.fold[w] = a;
    }
    if constexpr (GELU) {
        gelu_table_copy<kQT>(s_gelu, p.gelu_tab);
        wait_vmem();
    }
    __syncthreads();
    if (HAS_ROW) {
        s_enc = tensor_s_enc(fmaxf(fmaxf(L.fold[0], L.fold[1]), fmaxf(L.fold[2], L.fold[3])));
        if (blockIdx.x == 0 && threadIdx.x == 0) p.row_sdec[0] = 1.0f / s_enc;
        enc_scale_table(L.tab, 1.0f / s_enc);
    }
    __syncthreads();

    const int64_t n_step = p.C / 8;
    float am = 0.0f, amr = 0.0f;                      // amax partials (AP, AR)
    // The next step is loaded while this one is encoded, except in the amax
    // pass variants and the GELU copy: their RHT, stochastic MXFP8 or GELU
    // work needs the registers, and without the look-ahead they run three or
    // four waves per SIMD instead of two (measured faster).
    constexpr bool kAhead = !(AP || AR) && !GELU;
    while (t < T) {                                   // wave-uniform
        const int64_t tn = t + stride;
        uint4 vn[kAhead ? PR : 1];
        int64_t r0n = r0, c0n = c0;
        if constexpr (kAhead) {
            if (tn < T) load(tn, vn, r0n, c0n);
        }
        const bool in = c0 < p.C;
        if (AP && in) {
#pragma unroll
            for (int r = 0; r < PR; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(elem(v[r], j)));
        }
        if (AR && !HALF && in) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float y[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) y[r] = elem_flip(v[r], j, sign_bit(p.rht_signs, r));
                rht16_butterflies(y, 0u);
#pragma unroll
                for (int r = 0; r < 16; ++r) amr = fmaxf(amr, fabsf(y[r]));
            }
        }
        auto val = [&](int r, int j) -> float {
            if constexpr (GELU) return gelu_bf16(elem_bits(v[r], j), s_gelu);
            else return elem(v[r], j);
        };
        uint32_t tsc = 0;
        float ts = 0.0f;
        if (HAS_ROW && TILE2D) {
            float a = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(elem(v[r], j)));
            tsc = block_scale_code(max_lane_pair(a), s_enc);
            ts = L.tab[tsc];
            // one scale byte per 16x16 tile: 32 per wave step, as 8 words
            const uint32_t word = gather4(tsc, 2);
            if ((lane & 7) == 0 && in)
                put_scales4(p.row_scales + (r0 / 16) * (p.C / 16) + c0 / 16, word, (p.C - c0) / 16);
        }
        const uint64_t nr0 = (uint64_t)(r0 * p.C + c0) / 8;
        auto one = [&](auto row_sr, auto mx_sr, int r) {
            constexpr bool RSR = decltype(row_sr)::value, MSR = decltype(mx_sr)::value;
            float f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = val(r, j);
            const int64_t row = r0 + r;
            if (HAS_ROW) {
                uint32_t sc = tsc;
                float sv = ts;
                if (!TILE2D) {
                    float a = 0.0f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
                    sc = block_scale_code(max_lane_pair(a), s_enc);
                    sv = L.tab[sc];
                    const uint32_t word = gather4(sc, 2);
                    if ((lane & 7) == 0 && in)
                        put_scales4(p.row_scales + row * (p.C / 16) + c0 / 16, word, (p.C - c0) / 16);
                }
                uint32_t packed;
                if constexpr (RSR) {
                    uint32_t wd[4];
                    sr_block(p.row_seed, p.row_stream, nr0 + (uint64_t)r * n_step, wd);
                    packed = e2m1_sr8(f, sv, wd);
                } else {
                    packed = e2m1_rne8(f, sv);
                }
                if (in) *reinterpret_cast<uint32_t *>(p.row_codes + row * (p.C / 2) + c0 / 2) = packed;
            }
            if (HAS_MX) {
                float y[8];
                float a = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    y[j] = f[j];
                    a = fmaxf(a, fabsf(f[j]));
                }
                const uint32_t kb = e8m0_byte(max_lane_quad(a));
                if (__builtin_amdgcn_ballot_w64(kb == 0)) {   // rare, wave-uniform test
                    if (kb == 0) {                             // 2^-127: convert 2y at 2^-126
#pragma unroll
                        for (int j = 0; j < 8; ++j) y[j] = y[j] * 2.0f;
                    }
                }
                const float cs = e8m0_cvt_scale(kb);
                uint32_t lo, hi;
                if constexpr (MSR) {
                    uint32_t wd[4];
                    sr_block(p.mx_seed, p.mx_stream, nr0 + (uint64_t)r * n_step, wd);
                    lo = e4m3_sr4_scaled(y[0], y[1], y[2], y[3], sr_word_lo(wd[0]), sr_word_hi(wd[0]),
                                         sr_word_lo(wd[1]), sr_word_hi(wd[1]), cs);
                    hi = e4m3_sr4_scaled(y[4], y[5], y[6], y[7], sr_word_lo(wd[2]), sr_word_hi(wd[2]),
                                         sr_word_lo(wd[3]), sr_word_hi(wd[3]), cs);
                } else {
                    lo = e4m3_rne4_scaled(y[0], y[1], y[2], y[3], cs);
                    hi = e4m3_rne4_scaled(y[4], y[5], y[6], y[7], cs);
                }
                if (in) *reinterpret_cast<uint2 *>(p.mx_codes + row * p.C + c0) = make_uint2(lo, hi);
                const uint32_t word = gather4(kb, 4);
                if ((lane & 15) == 0 && in)
                    put_scales4(p.mx_scales + row * (p.C / 32) + c0 / 32, word, (p.C - c0) / 32);
            }
        };
        auto rows = [&](auto row_sr, auto mx_sr) {
            // (loops of 8 rows: each stays under the full-unroll limit)
#pragma unroll
            for (int r = 0; r < 8; ++r) one(row_sr, mx_sr, r);
#pragma unroll
            for (int r = 8; r < PR; ++r) one(row_sr, mx_sr, r);
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        if constexpr (SR) {
            const bool row_sr = HAS_ROW && p.row_round == 1, mx_sr = HAS_MX && p.mx_round == 1;
            if (row_sr && mx_sr) rows(T_{}, T_{});
            else if (row_sr) rows(T_{}, F_{});
            else if (mx_sr) rows(F_{}, T_{});
            else rows(F_{}, F_{});
        } else {
            rows(F_{}, F_{});
        }
        if (AR && HALF && in) {
            // lanes l and l ^ 32 (same columns, the same in-flag) trade
            // halves: words 0-1 of v[i] then hold row i, words 2-3 row
            // i + 8, of the lane's four columns 4 (l >> 5) .. + 3
#pragma unroll
            for (int i = 0; i < PR; ++i) {
                const auto a = __builtin_amdgcn_permlane32_swap(v[i].x, v[i].z, false, false);
                const auto b = __builtin_amdgcn_permlane32_swap(v[i].y, v[i].w, false, false);
                v[i] = make_uint4(a[0], b[0], a[1], b[1]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float y[16];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    y[r] = elem_flip(v[r], j, sign_bit(p.rht_signs, r));
                    y[r + 8] = elem_flip(v[r], 4 + j, sign_bit(p.rht_signs, r + 8));
                }
                rht16_butterflies(y, 0u);
#pragma unroll
                for (int r = 0; r < 16; ++r) amr = fmaxf(amr, fabsf(y[r]));
            }
        }
        t = tn;
        if constexpr (kAhead) {
            r0 = r0n;
            c0 = c0n;
#pragma unroll
            for (int i = 0; i < PR; ++i) v[i] = vn[i];
        } else if (t < T) {
            load(t, v, r0, c0);
        }
    }
    if constexpr (AP || AR) {
        // the workgroup's partials (the RHT's final multiply by 1/4 is
        // monotonic, so it is applied to the maximum)
        am = wave_max(am);
        amr = wave_max(amr * 0.25f);
        __shared__ float red[2][kQT / 64];
        if (lane == 0) {
            red[0][w] = am;
            red[1][w] = amr;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float a = red[0][0], b = red[1][0];
            for (int i = 1; i < kQT / 64; ++i) {
                a = fmaxf(a, red[0][i]);
                b = fmaxf(b, red[1][i]);
            }
            if (AP) amax_part[blockIdx.x] = a;
            if (AR) amax_part_rht[blockIdx.x] = b;
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
        gelu_table_copy<kQT>(s_gelu, p.gelu_tab);   // while the row is in flight
        wait_vmem();
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
// A tile is 128 source rows x 256 source columns.  Wave w holds the rows
// 32w .. 32w + 31 and lane l the 16 rows 32w + 16 (l & 1) .. + 15 of the
// columns 8 (l >> 1) .. + 7, so a destination row's block of 32 (one wave's
// rows) is two neighbouring lanes: they share the block maximum and each
// encodes its 16 values.  The tile's 256 destination rows x 128 code bytes
// are gathered in LDS (16-byte groups swizzled by (row >> 3) & 7) and stored
// as whole rows, its 256 x 4 scale bytes as 4-byte runs; the 33 KB of LDS
// and the 16-row pieces leave room for four workgroups per CU.
// ---------------------------------------------------------------------------
struct RequantLds {
    uint8_t codes[kReqC * 128];
    uint8_t scales[kReqC * 4];
};
__device__ __forceinline__ int req_off(int row, int group) {
    return row * 128 + ((group ^ ((row >> 3) & 7)) << 4);
}

// WALK = false: one tile per workgroup (XCD-contiguous mapping), registers
// capped for MINW waves per SIMD; WALK = true: a resident grid walks runs
// of tiles, loading the next tile's codes while it encodes the current one.
template <bool SR, bool TILE2D, bool WALK, int MINW>
__global__ __launch_bounds__(kQT, MINW) void requant_kernel(RequantParams p) {
    __shared__ __align__(16) RequantLds L;
    const int64_t tiles_c = (p.C + kReqC - 1) / kReqC;
    const int64_t T = ((p.R + kReqR - 1) / kReqR) * tiles_c;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane & 1, cg = lane >> 1;
    const float s_dec = p.s_dec[0];
    const int64_t nsb = p.C / 16;                    // scale bytes per scale row
    constexpr int NB = TILE2D ? 1 : 16;              // block scales per lane

    // Source of tile t for this lane: 16 rows x 8 columns (invalid pieces
    // read a valid piece and store nothing; R is a multiple of 32).
    struct Src {
        int64_t band, r0, c0;   // the wave's first row, the lane's first row and column
        bool in;
    };
    auto src_of = [&](int64_t tile) -> Src {
        const int64_t tr = tile / tiles_c, tc = tile - tr * tiles_c;
        Src s;
        s.band = tr * kReqR + w * 32;
        s.r0 = s.band + h * 16;
        s.c0 = tc * kReqC + cg * 8;
        s.in = s.band < p.R && s.c0 < p.C;
        return s;
    };
    auto load = [&](const Src &s, uint32_t (&cw)[16], uint32_t (&sb)[NB]) {
        const int64_t r0 = s.r0 < p.R ? s.r0 : p.R - 16;
        const int64_t c0 = s.c0 < p.C ? s.c0 : p.C - 8;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            cw[r] = *reinterpret_cast<const uint32_t *>(p.codes + (r0 + r) * (p.C / 2) + c0 / 2);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int64_t srow = TILE2D ? r0 / 16 : r0 + i;
            sb[i] = p.scales[srow * nsb + c0 / 16];
        }
    };

    const TileWalk walk = WALK ? xcd_walk(T) : TileWalk{xcd_tile(blockIdx.x, T), xcd_tile(blockIdx.x, T) + 1, 1};
    uint32_t cw[16], sb[NB];
    Src s = src_of(walk.first < walk.end ? walk.first : 0);
    if (walk.first < walk.end) load(s, cw, sb);
    for (int64_t t = walk.first; t < walk.end; t += walk.step) {    // workgroup-uniform
        const int64_t tn = t + walk.step;
        uint32_t cwn[WALK ? 16 : 1], sbn[WALK ? NB : 1];
        Src sn = s;
        if (WALK && tn < walk.end) {
            sn = src_of(tn);
            load(sn, *reinterpret_cast<uint32_t(*)[16]>(cwn), *reinterpret_cast<uint32_t(*)[NB]>(sbn));
        }
        float bs[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) bs[i] = __builtin_amdgcn_cvt_scalef32_f32_fp8((int)sb[i], 1.0f, 0);
        // destination row (in the tile) cg * 8 + j, bytes w * 32 + h * 16 .. + 15
        auto emit = [&](const float (&x)[16], int j) {
            float a = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(x[r]));
            const uint32_t kb = e8m0_byte(max_lane_pair(a));
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] = x[r];
            if (__builtin_amdgcn_ballot_w64(kb == 0)) {   // rare, wave-uniform test
                if (kb == 0) {                             // 2^-127: convert 2y at 2^-126
#pragma unroll
                    for (int r = 0; r < 16; ++r) y[r] = y[r] * 2.0f;
                }
            }
            const float cs = e8m0_cvt_scale(kb);
            const int64_t c = s.c0 + j;                  // destination row
            uint32_t out[4];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                if constexpr (SR) {
                    // Philox block 2h + g of the destination row's 32-block
                    uint32_t wd[4];
                    sr_block(p.seed, p.stream, (uint64_t)(c * p.R + s.band) / 8 + 2 * h + g, wd);
                    out[2 * g] = e4m3_sr4_scaled(y[8 * g], y[8 * g + 1], y[8 * g + 2], y[8 * g + 3],
                                                 sr_word_lo(wd[0]), sr_word_hi(wd[0]),
                                                 sr_word_lo(wd[1]), sr_word_hi(wd[1]), cs);
                    out[2 * g + 1] = e4m3_sr4_scaled(y[8 * g + 4], y[8 * g + 5], y[8 * g + 6],
                                                     y[8 * g + 7], sr_word_lo(wd[2]),
                                                     sr_word_hi(wd[2]), sr_word_lo(wd[3]),
                                                     sr_word_hi(wd[3]), cs);
                } else {
                    out[2 * g] = e4m3_rne4_scaled(y[8 * g], y[8 * g + 1], y[8 * g + 2], y[8 * g + 3], cs);
                    out[2 * g + 1] = e4m3_rne4_scaled(y[8 * g + 4], y[8 * g + 5], y[8 * g + 6],
                                                      y[8 * g + 7], cs);
                }
            }
            const int drow = cg * 8 + j;
            *reinterpret_cast<uint4 *>(L.codes + req_off(drow, 2 * w + h)) =
                make_uint4(out[0], out[1], out[2], out[3]);
            if (h == 0) L.scales[drow * 4 + w] = (uint8_t)kb;
        };
        auto pair = [&](auto jp_tag) {                   // source columns 2jp, 2jp + 1
            constexpr int jp = decltype(jp_tag)::value;
            float xe[16], xo[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const f32x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[r], 1.0f, jp);
                const float b = bs[TILE2D ? 0 : r];
                // (E2M1 x E4M3) is exact; the multiply by s_dec is one FP32 rounding.
                xe[r] = (e[0] * b) * s_dec;
                xo[r] = (e[1] * b) * s_dec;
            }
            emit(xe, 2 * jp);
            emit(xo, 2 * jp + 1);
        };
        pair(std::integral_constant<int, 0>{});
        pair(std::integral_constant<int, 1>{});
        pair(std::integral_constant<int, 2>{});
        pair(std::integral_constant<int, 3>{});
        __syncthreads();
        // 256 destination rows x 8 groups of 16 bytes: 8 passes of 256 threads;
        // then 256 x 4 scale bytes
        {
            const int64_t tr = t / tiles_c, tc = t - tr * tiles_c;
            const int64_t R0 = tr * kReqR, C0 = tc * kReqC;
            const int64_t drows = p.C - C0 < kReqC ? p.C - C0 : kReqC;
            const int64_t groups = (p.R - R0) / 16 < 8 ? (p.R - R0) / 16 : 8;   // R % 32 == 0
#pragma unroll 4
            for (int i = 0; i < kReqC * 8 / kQT; ++i) {
                const int idx = i * kQT + threadIdx.x, drow = idx >> 3, g = idx & 7;
                if (drow < drows && g < groups)
                    *reinterpret_cast<uint4 *>(p.out_codes + (C0 + drow) * p.R + R0 + g * 16) =
                        *reinterpret_cast<const uint4 *>(L.codes + req_off(drow, g));
            }
            const int64_t nsc = (p.R - R0) / 32 < 4 ? (p.R - R0) / 32 : 4;
            const int drow = threadIdx.x;               // kReqC == kQT
            if (drow < drows)
                put_run<4>(p.out_scales + (C0 + drow) * (p.R / 32) + R0 / 32, L.scales + drow * 4,
                           nsc);
        }
        __syncthreads();
        if constexpr (WALK) {
            s = sn;
#pragma unroll
            for (int r = 0; r < 16; ++r) cw[r] = cwn[r];
#pragma unroll
            for (int i = 0; i < NB; ++i) sb[i] = sbn[i];
        }
    }
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

// Workgroups of a persistent launch of `kernel` (THREADS each): as many as
// are resident on the stream's device at once, at most `tiles`, at least 1.
// The occupancy per CU is the kernel's and is looked up once (thread-safe
// static initialisation).
template <auto Kernel, int THREADS = kQT>
static int persistent_grid(int64_t tiles, hipStream_t s) {
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Kernel, THREADS, 0) != hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    const int64_t g = (int64_t)per_cu * device_cus(s);
    return (int)(tiles < g ? (tiles < 1 ? 1 : tiles) : g);
}

hipError_t launch_amax(const uint16_t *x, int64_t R, int64_t C, int64_t ld, bool plain, bool rht,
                       uint32_t signs, float *part, float *part_rht, int *n_part,
                       hipStream_t s, float *gelu_tab) {
    // one wave per 16 x 256 step (16 x 512 for GELU); up to 256 workgroups
    // (1024 for GELU, whose tanh makes the pass slower per byte)
    const int64_t sc = gelu_tab ? kAmaxStepC : kAmaxStepC / 2;
    const int64_t steps = (R / 16) * ((C + sc - 1) / sc);
    const int64_t cap = gelu_tab ? kAmaxPartials / 2 : kAmaxPartials / 8;
    const int64_t want = (steps + kQT / 64 - 1) / (kQT / 64);
    const int grid = (int)(want < cap ? want : cap);
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

// The encode kernel variants the library launches (timed per variant; a
// workgroup of 512 threads is two waves per SIMD): copies with 16x16 tiles
// (weights) run one workgroup per CU, those rounding to nearest walking runs
// of tiles and loading ahead; the others take one tile per workgroup with
// registers capped for four waves per SIMD, six for the row copy + RHT'd
// stochastic column copy (activations for wgrad), whose row copy keeps the
// VALU light enough for the extra waves to pay, and five for the RHT'd
// stochastic column copy alone (gradients; 4% faster than four, with a few
// spilled bytes).
template <bool T_, bool SR_>
constexpr bool quant_walk() { return T_ && !SR_; }
template <bool R_, bool C_, bool M_, bool T_, bool H_, bool SR_>
constexpr int quant_min_waves() {
    if (T_) return 2;
    if (R_ && C_ && H_ && SR_) return 6;
    if (!R_ && C_ && !M_ && H_ && SR_) return 5;
    return 4;
}

template <bool R_, bool C_, bool M_, bool T_, bool H_, bool G_, bool SR_, bool W_, int MW_>
static void launch_qk(const QuantParams &p, hipStream_t s) {
    const int64_t T = ((p.R + kTileR - 1) / kTileR) * ((p.C + kTileC - 1) / kTileC);
    constexpr auto k = quant_kernel<R_, C_, M_, T_, H_, G_, SR_, W_, MW_>;
    const int grid = W_ ? persistent_grid<k, kET>(T, s) : (int)T;
    hipLaunchKernelGGL(k, dim3(grid), dim3(kET), 0, s, p);
}

template <bool R_, bool C_, bool M_, bool T_, bool H_, bool G_ = false>
static void launch_q(const QuantParams &p, bool sr, hipStream_t s) {
    if (sr)
        launch_qk<R_, C_, M_, T_, H_, G_, true, quant_walk<T_, true>(),
                  quant_min_waves<R_, C_, M_, T_, H_, true>()>(p, s);
    else
        launch_qk<R_, C_, M_, T_, H_, G_, false, quant_walk<T_, false>(),
                  quant_min_waves<R_, C_, M_, T_, H_, false>()>(p, s);
}

// Row-wise copies only: a resident grid of 16 x 512 wave steps.
template <bool R_, bool M_, bool T_, bool G_, bool SR_>
static void launch_rows_k(const QuantParams &p, hipStream_t s) {
    // (GELU, no look-ahead: 104 VGPRs; the others keep two steps in
    // registers, and a cap of four spills with SR)
    constexpr int MW = G_ ? 4 : 2;
    constexpr auto k = quant_rows_kernel<R_, M_, T_, G_, SR_, MW>;
    const int64_t steps = (p.R / 16) * ((p.C + kAmaxStepC - 1) / kAmaxStepC);
    hipLaunchKernelGGL(k, dim3(persistent_grid<k>((steps + 3) / 4, s)), dim3(kQT), 0, s, p,
                       nullptr, nullptr);
}

// The amax pass of a quantize with an MXFP8 row copy (no GELU): the row-step
// kernel writes that copy, which needs no tensor scale, and the partials the
// encode of the other copies folds, from one read of x.
template <bool SR_, bool AP_, bool AR_>
static int launch_amax_mx_k(const QuantParams &p, float *part, float *part_rht, hipStream_t s) {
    // half steps (8 rows per lane): six waves per SIMD with the RHT partials
    // alone (at the cost of a few spilled bytes, 2% faster than four), four
    // with the plain partials, three with the plain partials and stochastic
    // rounding (where four would spill)
    constexpr int MW = AP_ ? (SR_ ? 3 : 4) : 6;
    constexpr auto k = quant_rows_kernel<false, true, false, false, SR_, MW, AP_, AR_, true>;
    const int64_t steps = (p.R / 16) * ((p.C + kAmaxStepC / 2 - 1) / (kAmaxStepC / 2));
    int64_t grid = persistent_grid<k>((steps + 3) / 4, s);
    if (grid > kAmaxPartials) grid = kAmaxPartials;
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kQT), 0, s, p, part, part_rht);
    return (int)grid;
}

hipError_t launch_amax_mx(const QuantParams &p, bool plain, bool rht, float *part, float *part_rht,
                          int *n_part, hipStream_t s) {
    const bool sr = p.mx_round == 1;
    int n = 0;
    if (plain && rht) n = sr ? launch_amax_mx_k<true, true, true>(p, part, part_rht, s)
                             : launch_amax_mx_k<false, true, true>(p, part, part_rht, s);
    else if (plain) n = sr ? launch_amax_mx_k<true, true, false>(p, part, part_rht, s)
                           : launch_amax_mx_k<false, true, false>(p, part, part_rht, s);
    else if (rht) n = sr ? launch_amax_mx_k<true, false, true>(p, part, part_rht, s)
                         : launch_amax_mx_k<false, false, true>(p, part, part_rht, s);
    else return hipErrorInvalidValue;
    *n_part = n;
    return hipGetLastError();
}
// nearest-rounding row copies
template <bool R_, bool M_, bool T_, bool G_>
static void launch_rows(const QuantParams &p, hipStream_t s) {
    launch_rows_k<R_, M_, T_, G_, false>(p, s);
}

hipError_t launch_quant_tile(const QuantParams &p, bool has_row, bool has_col, bool has_mx,
                             bool tile2d, bool rht, hipStream_t s, bool gelu) {
    // the stochastic paths are compiled only into the variant that needs them
    const bool sr = (has_row && p.row_round == 1) || (has_col && p.col_round == 1) ||
                    (has_mx && p.mx_round == 1);
    if (gelu) {
        if (has_col || tile2d || rht) return hipErrorInvalidValue;
        if (has_row && has_mx) launch_q<1, 0, 1, 0, 0, 1>(p, sr, s);
        else if (has_row && !sr) launch_rows_k<1, 0, 0, 1, false>(p, s);
        else if (has_row) launch_q<1, 0, 0, 0, 0, 1>(p, sr, s);
        else if (has_mx) launch_q<0, 0, 1, 0, 0, 1>(p, sr, s);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    // Row-wise copies only, all rounding to nearest: light ALU work, so the
    // resident row-step kernel (whole-row stores, next step loaded ahead)
    // is used; the stochastic ones keep the tile kernel's four waves per SIMD
    // (GELU rows to nearest take the row-step kernel above, without the
    // look-ahead).
    if (!has_col && !sr) {
        if (has_row && has_mx) {
            if (tile2d) launch_rows<1, 1, 1, 0>(p, s);
            else launch_rows<1, 1, 0, 0>(p, s);
        } else if (has_row) {
            if (tile2d) launch_rows<1, 0, 1, 0>(p, s);
            else launch_rows<1, 0, 0, 0>(p, s);
        } else if (has_mx) {
            launch_rows<0, 1, 0, 0>(p, s);
        } else {
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    // The combinations the quantizer supports (RHT only on a 1x16 column copy).
    const int key = (has_row << 4) | (has_col << 3) | (has_mx << 2) | (tile2d << 1) | rht;
    switch (key) {
        case 0b10000: launch_q<1, 0, 0, 0, 0>(p, sr, s); break;
        case 0b10010: launch_q<1, 0, 0, 1, 0>(p, sr, s); break;
        case 0b00100: launch_q<0, 0, 1, 0, 0>(p, sr, s); break;
        case 0b10100: launch_q<1, 0, 1, 0, 0>(p, sr, s); break;
        case 0b10110: launch_q<1, 0, 1, 1, 0>(p, sr, s); break;
        case 0b11000: launch_q<1, 1, 0, 0, 0>(p, sr, s); break;
        case 0b11010: launch_q<1, 1, 0, 1, 0>(p, sr, s); break;
        case 0b11001: launch_q<1, 1, 0, 0, 1>(p, sr, s); break;
        case 0b01000: launch_q<0, 1, 0, 0, 0>(p, sr, s); break;
        case 0b01010: launch_q<0, 1, 0, 1, 0>(p, sr, s); break;
        case 0b01001: launch_q<0, 1, 0, 0, 1>(p, sr, s); break;
        case 0b01100: launch_q<0, 1, 1, 0, 0>(p, sr, s); break;
        case 0b01101: launch_q<0, 1, 1, 0, 1>(p, sr, s); break;
        case 0b11100: launch_q<1, 1, 1, 0, 0>(p, sr, s); break;
        case 0b11101: launch_q<1, 1, 1, 0, 1>(p, sr, s); break;
        case 0b01110: launch_q<0, 1, 1, 1, 0>(p, sr, s); break;
        case 0b11110: launch_q<1, 1, 1, 1, 0>(p, sr, s); break;
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

template <bool SR, bool TILE2D, bool WALK, int MINW>
static void launch_rqk(const RequantParams &p, hipStream_t s) {
    const int64_t T = ((p.R + kReqR - 1) / kReqR) * ((p.C + kReqC - 1) / kReqC);
    constexpr auto k = requant_kernel<SR, TILE2D, WALK, MINW>;
    hipLaunchKernelGGL(k, dim3(WALK ? persistent_grid<k>(T, s) : (int)T), dim3(kQT), 0, s, p);
}

// The requantizer variant the library launches: one tile per workgroup,
// registers capped for four waves per SIMD (walking runs of tiles at two
// waves per SIMD measured 36% slower).
constexpr bool kReqWalk = false;
constexpr int kReqMinW = 4;

hipError_t launch_requant(const RequantParams &p, bool sr, hipStream_t s) {
    if (sr && p.tile2d) launch_rqk<true, true, kReqWalk, kReqMinW>(p, s);
    else if (sr) launch_rqk<true, false, kReqWalk, kReqMinW>(p, s);
    else if (p.tile2d) launch_rqk<false, true, kReqWalk, kReqMinW>(p, s);
    else launch_rqk<false, false, kReqWalk, kReqMinW>(p, s);
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

// Kernel parameter blocks and host-side launchers shared by the C ABI layer
// and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bbs {

// Upper bound on the workgroups of an amax pass (= partial maxima written).
constexpr int kAmaxPartials = 2048;
// Workspace layout (floats): plain partials, RHT partials, GELU table.
constexpr int kGeluTabOffset = 2 * kAmaxPartials;
constexpr int kWorkspaceFloats = kGeluTabOffset + 7168;

struct QuantParams {
    const uint16_t *x;
    int64_t R, C, ld;
    // row-wise NVFP4 copy
    uint8_t *row_codes, *row_scales;
    float *row_sdec;
    int row_round;
    uint32_t row_stream;
    uint64_t row_seed;
    // column-wise NVFP4 copy (of x^T)
    uint8_t *col_codes, *col_scales;
    float *col_sdec;
    int col_round;
    uint32_t col_stream;
    uint64_t col_seed;
    uint32_t rht_signs;
    // row-wise MXFP8 copy
    uint8_t *mx_codes, *mx_scales;
    int mx_round;
    uint32_t mx_stream;
    uint64_t mx_seed;
    // amax partials
    const float *part;
    const float *part_rht;
    int n_part, n_part_rht;
    // GELU table (kGeluTabSize floats, 16-byte aligned) when the copies are
    // of GELU(x)
    const float *gelu_tab;
};

struct RequantParams {
    const uint8_t *codes, *scales;
    const float *s_dec;
    int64_t R, C;
    int tile2d;
    uint8_t *out_codes, *out_scales;
    uint64_t seed;
    uint32_t stream;
};

// NVFP4 GEMM operand view: rows x K, codes rows x K/2, scales per tile2d.
struct Fp4View {
    const uint8_t *codes, *scales;
    const float *s_dec;
    int64_t rows;
    int tile2d;
    int sdec_rows;      // s_dec holds one decode scale per row
};

// NVFP4 output of a GEMM quantized in its epilogue: 1x16 rows, nearest,
// with a given encode scale (optionally of GELU of the product).
struct QuantOut {
    uint8_t *codes, *scales;
    float *s_dec;            // receives 1 / s_enc
    const float *s_enc;      // one FP32 encode scale (device)
    unsigned *amax;          // max |y| of the quantized values as FP32 bits, or nullptr
    const float *gelu_tab;   // the GELU table (GELU modes)
    uint32_t signs;          // combine wire format (S2F6 mode): RHT sign flips
    int rht;                 //   and whether to rotate
};

struct GemmParams {
    Fp4View a, b;
    QuantOut q;                    // the quantizing kernels only
    int64_t M, N, K;
    void *c;
    int64_t ldc;
    // grouped mode
    const int32_t *row_index;      // A row gather (nullptr = identity)
    const int64_t *group_offsets;  // G + 1 entries
    int G;
    int64_t max_rows;
    int64_t a_src_rows;            // rows of A addressable through row_index
};

struct Mx8GemmParams {
    const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
    int64_t M, N, K;
    void *c;
    int64_t ldc;
};

struct S2F6CombineParams {
    const int8_t *codes;
    const uint8_t *scales;
    int64_t C;                 // values per row (C % 32 == 0)
    const int32_t *src;        // T x K rows of codes (negative or >= src_rows: skipped)
    int64_t src_rows;
    const float *w;            // T x K weights, or nullptr (weight 1)
    int64_t T;
    int K;
    uint32_t signs;
    void *out;
    int64_t ldo;
};

// Compute units of the device that runs stream s (the current device for
// the NULL stream); cached per device, safe to call from several threads.
int device_cus(hipStream_t s);

// Combine wire format: S2F6 encode (optionally rotated) and the receiver's
// weighted sum + inverse rotation.
hipError_t launch_s2f6_encode(const uint16_t *x, int64_t R, int64_t C, int64_t ld, bool rht,
                              uint32_t signs, int8_t *codes, uint8_t *scales, hipStream_t s);
hipError_t launch_s2f6_combine(const S2F6CombineParams &p, bool rht, bool bf16_out,
                               hipStream_t s);

// One read of x: partial maxima of |x| (plain) into part and of the RHT'd
// column chunks (rht) into part_rht; *n_part partials each.  With gelu (and
// plain, without rht) the partials are maxima of |GELU(x)|, and the pass
// also writes the GELU table.
hipError_t launch_amax(const uint16_t *x, int64_t R, int64_t C, int64_t ld, bool plain, bool rht,
                       uint32_t signs, float *part, float *part_rht, int *n_part, hipStream_t s,
                       float *gelu_tab = nullptr);
// The GELU table alone (for the activation copy with a per-token scale).
hipError_t launch_gelu_table(float *gelu_tab, hipStream_t s);
// gelu: the row-wise copies (NVFP4 and / or MXFP8, no column copy, 1x16) are
// of GELU(x).
// The amax pass (plain and / or RHT partials) fused with the MXFP8 row copy
// described by p (p.rht_signs for the RHT); *n_part = the partials written.
hipError_t launch_amax_mx(const QuantParams &p, bool plain, bool rht, float *part, float *part_rht,
                          int *n_part, hipStream_t s);
hipError_t launch_quant_tile(const QuantParams &p, bool has_row, bool has_col, bool has_mx,
                             bool tile2d, bool rht, hipStream_t s, bool gelu = false);
hipError_t launch_requant(const RequantParams &p, bool sr, hipStream_t s);
// Row copy of an activation with a per-token outer scale and / or Four Over
// Six (RTN, 1x16), optionally of GELU(x); without per_token, p.part holds
// the tensor amax partials.
hipError_t launch_quant_act(const QuantParams &p, bool per_token, bool four_six, bool gelu,
                            hipStream_t s);
// The large-tile NVFP4 kernels apply (K % 128 == 0, aligned operands and C);
// they are the ones that support a per-row A decode scale.
bool big_ok(const GemmParams &p, bool bf16_out);
hipError_t launch_nvfp4_gemm(const GemmParams &p, bool bf16_out, hipStream_t s);
hipError_t launch_grouped_nvfp4_gemm(const GemmParams &p, bool bf16_out, hipStream_t s);
// The same GEMMs (large-tile kernels only: big_ok must hold) writing p.q
// instead of C; p.q.amax, when given, is cleared first; with gelu the GELU
// table is written to p.q.gelu_tab first.
hipError_t launch_nvfp4_gemm_quant(const GemmParams &p, bool gelu, hipStream_t s);
hipError_t launch_grouped_nvfp4_gemm_quant(const GemmParams &p, bool gelu, hipStream_t s);
// The same GEMMs with the combine wire format encode (32-point RHT + S2F6)
// of the BF16 output in the epilogue; q.codes / q.scales receive it.
hipError_t launch_nvfp4_gemm_s2f6(const GemmParams &p, hipStream_t s);
hipError_t launch_grouped_nvfp4_gemm_s2f6(const GemmParams &p, hipStream_t s);
hipError_t launch_mxfp8_gemm(const Mx8GemmParams &p, bool bf16_out, hipStream_t s);
// MXFP4 x MXFP4 (codes rows x K/2): K % 256 == 0, 16-byte aligned codes,
// 4-byte aligned scales, N % 4 == 0, 16-byte aligned C with ldc % 4 == 0.
hipError_t launch_mxfp4_gemm(const Mx8GemmParams &p, bool bf16_out, hipStream_t s);
// MXFP4 copy of a BF16 matrix (blocks of 32 along its rows).
hipError_t launch_mxfp4_quant(const uint16_t *x, int64_t R, int64_t C, int64_t ld, uint8_t *codes,
                              uint8_t *scales, bool sr, uint64_t seed, uint32_t stream,
                              hipStream_t s);

}  // namespace bbs

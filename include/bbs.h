/*
 * bbs.h - C ABI of the MI355X (gfx950) NVFP4 quantized-linear library.
 *
 * The library implements the data-parallel hot path of an NVFP4 quantized
 * linear layer: the fused NVFP4 quantizer, the dequantize-transpose-
 * requantize to MXFP8 of a saved NVFP4 tensor, and the block-scaled GEMMs.
 * Every arithmetic step runs in HIP kernels on the GPU.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, allocated and owned by the
 *    caller.  The library never allocates, frees or retains them.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *    enqueued; no call synchronises the host.
 *  - Matrices are row-major.  BF16 values are passed as their 16-bit
 *    patterns.  An NVFP4 matrix of shape rows x cols stores its E2M1 codes
 *    as rows x cols/2 bytes: element 2j of a row is the low nibble of byte j,
 *    element 2j+1 the high nibble.  Its E4M3 block scales are row-major,
 *    rows x cols/16 (1x16 blocks) or rows/16 x cols/16 (16x16 tiles).  An
 *    MXFP8 matrix stores rows x cols E4M3 bytes and rows x cols/32 E8M0
 *    bytes (scale 2^(byte-127)).
 *  - Return value: BBS_OK (0) or a negative status.  Arguments are checked
 *    before anything is enqueued; on error nothing is launched.  Faults of
 *    a running kernel surface at the caller's next synchronisation.
 *  - Calls are thread-safe.  Calls on one stream run in order.
 *  - Precondition of the quantizers: finite inputs, and a tensor amax that
 *    is either 0 or at least 2^-100 (smaller non-zero maxima overflow the
 *    FP32 encode scales; the result is then unspecified).  With the RHT the
 *    transformed values must be finite too (|x| < 2^126 suffices: a 16-point
 *    transform grows a magnitude by at most 4x).
 */
#ifndef BBS_H
#define BBS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BBS_OK 0
#define BBS_EINVAL (-1)  /* null pointer, bad shape, misalignment, short workspace */
#define BBS_ENOTSUP (-2) /* a valid but unsupported combination of options        */
#define BBS_EHIP (-3)    /* the HIP runtime rejected a launch; see bbs_last_error  */

enum bbs_round { BBS_RTN = 0, BBS_SR = 1 };
enum bbs_out_dtype { BBS_OUT_F32 = 0, BBS_OUT_BF16 = 1 };
enum bbs_fmt { BBS_FMT_NVFP4 = 0, BBS_FMT_MXFP8 = 1, BBS_FMT_MXFP4 = 2 };

/* Words of device workspace nvfp4_quantize needs for its amax partials. */
#define BBS_AMAX_WS_FLOATS 11264

/* One NVFP4 tensor: value = E2M1(code) x E4M3(block scale) x s_dec
 * ("value = FP4 code x FP8 block scale x FP32 outer scale"; Pretraining LLMs
 * with NVFP4, "NVFP4 Format and Quantization Procedure", steps 1-5).
 * Blocks run along cols, the GEMM contraction dimension.  s_dec points to one
 * FP32 decode scale (G scales for the stacked weights of grouped_nvfp4_gemm),
 * or, with sdec_per_row = 1, to one per row (an activation copy with a
 * per-token outer scale, 4bit.vizuara.ai section 11; 1x16 blocks only).
 * codes must be 16-byte aligned; rows and cols must be positive multiples of
 * 16 (an empty tensor is BBS_EINVAL). */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    float *s_dec;
    int64_t rows, cols;
    int32_t tile2d;       /* 0: 1x16 blocks, 1: 16x16 tiles */
    int32_t sdec_per_row; /* 0: s_dec per tensor (per expert), 1: s_dec[row] */
} bbs_fp4;

/* One MXFP8 tensor: value = E4M3(code) x 2^(scale-127), one scale per 32
 * consecutive values of a row.  codes 16-byte aligned; cols % 32 == 0. */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    int64_t rows, cols;
} bbs_mx8;

/* One MXFP4 tensor (FP4 Training on Blackwell, 'The scaling math, worked';
 * the OCP microscaling format): value = E2M1(code) x 2^(scale-127), codes
 * rows x cols/2 bytes (element 2j of a row in the low nibble of byte j),
 * one E8M0 scale per 32 consecutive values of a row (rows x cols/32 bytes).
 * codes 16-byte aligned; cols % 32 == 0. */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    int64_t rows, cols;
} bbs_mx4;

/* Key of the stochastic-rounding draws: element idx of an output copy
 * (its row-major index in that copy's own layout) uses 16-bit lane idx % 8
 * of Philox4x32-10(counter = (idx/8 low, idx/8 high, stream, 0), key = seed),
 * as u = (lane + 1/2) / 65536, and rounds to floor(t + u) grid steps on the
 * exact sum, t being the magnitude in units of the local grid step
 * (4bit.vizuara.ai, section 6).  The same (seed, stream) reproduces the same
 * bits for any launch geometry. */
typedef struct {
    uint64_t seed;
    uint32_t stream;
} bbs_rng;

/* Arguments of nvfp4_quantize.  Any of row / col / row_mx8 may be NULL
 * (that copy is skipped); at least one must be given. */
typedef struct {
    const uint16_t *x; /* BF16 source, rows x cols, row stride ld elements   */
    int64_t rows, cols, ld; /* rows, cols > 0 and % 16 == 0; ld % 8 == 0;
                               x 16B aligned */

    bbs_fp4 *row;      /* NVFP4 copy of x (blocks along cols), shape rows x cols */
    int32_t row_round; /* BBS_RTN or BBS_SR */
    bbs_rng row_rng;

    bbs_fp4 *col;      /* NVFP4 copy of x^T (blocks along rows), shape cols x rows */
    int32_t col_round;
    bbs_rng col_rng;
    int32_t col_rht;    /* 1: 16-point random Hadamard transform of each 16-chunk
                           of the copy's rows before the amax and the encode */
    uint32_t rht_signs; /* bit i set: flip the sign of chunk element i first */

    bbs_mx8 *row_mx8;  /* MXFP8 copy of x (blocks of 32 along cols); cols % 32 == 0 */
    int32_t mx8_round;
    bbs_rng mx8_rng;

    int32_t tile2d; /* 1: 16x16 tile scales for row and col copies (col is then
                       the bit-identical transpose of row when both round RTN) */
    float *amax_ws; /* device workspace, >= BBS_AMAX_WS_FLOATS floats, 16-byte
                       aligned, not kept (amax partials; with gelu, also the
                       GELU table the encode pass reads) */

    /* Activation options of the row copy (4bit.vizuara.ai, section 11;
     * End-to-End 4-Bit Training, recipe details); both need row_round ==
     * BBS_RTN, tile2d == 0 and no col / row_mx8 copy in the same call.
     * row_per_token = 1: each row gets its own outer scale, s_enc_i = 2688 /
     *   amax(row i), and row->s_dec receives rows values (row->sdec_per_row
     *   must be 1); no tensor amax pass and no workspace are needed.
     * row_four_six = 1: each block is encoded with the scale that puts its
     *   largest magnitude on 6 and with the one that puts it on 4, and keeps
     *   the encoding with the smaller squared error (FP32: first eight
     *   values' sum plus last eight values' sum, each in element order; ties
     *   keep the first). */
    int32_t row_per_token;
    int32_t row_four_six;

    /* gelu = 1: the copies are of GELU(x) instead of x, with GELU applied
     * in FP32 inside the quantizer (4bit.vizuara.ai, section 13: the
     * activation rides along with the quantize), in the tanh form of
     * Hendrycks and Gimpel: 0.5 x (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3))),
     * tanh(u) = 1 - 2 / (exp(2u) + 1), each step one FP32 operation rounded
     * to nearest even, exp by Cody-Waite reduction (k = rint(v log2 e),
     * ln2 split into 0x3F317200 + 0x35BFBE8E) and the degree-7 Taylor
     * polynomial by Horner's rule, exp(v >= 88.5) = inf, exp(v <= -87) = 0.
     * The amax (tensor or per token) is that of |GELU(x)|.  Applies to the
     * row and row_mx8 copies (1x16, RTN or SR) and to the activation
     * options; a col copy or tile2d with gelu is BBS_ENOTSUP.  gelu always
     * needs amax_ws (per token too).  x finite. */
    int32_t gelu;
} bbs_quant_args;

/* NVFP4 quantizer (Pretraining LLMs with NVFP4, "NVFP4 Format and
 * Quantization Procedure", steps 1-4; 4bit.vizuara.ai, sections 5-6 and 13).
 * For each requested copy: tensor amax a (over the RHT'd values for an RHT
 * copy), s_enc = 2688 / a (1 if a == 0), s_dec = 1 / s_enc written to
 * copy->s_dec[0]; per block: E4M3 code of (amax_b / 6) * s_enc, round to
 * nearest even, saturating, never below code 1; s_enc_b = 1 / (E4M3 * s_dec);
 * elements x * s_enc_b rounded to E2M1 (nearest even, or stochastic).
 * The MXFP8 copy uses, per 32-block, the smallest power of two 2^k with
 * amax_b <= 448 * 2^k and rounds x * 2^-k to E4M3.
 * Errors: BBS_EINVAL (null x / workspace, no copy, bad shape or alignment,
 * output shapes not matching x), BBS_ENOTSUP (RHT on a tile2d copy). */
int nvfp4_quantize(const bbs_quant_args *a, void *stream);

/* nvfp4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same arguments, checks and results, except that a->amax_ws must be
 * NULL (else BBS_EINVAL): the amax partials and the GELU table go to a
 * scratch array of BBS_AMAX_WS_FLOATS floats (45056 bytes) that the library
 * holds in each GPU's memory until the process ends.  Its size does not
 * depend on the input: the amax pass writes at most 2048 partials for any
 * shape, so no shape is rejected for size.  The call allocates nothing (no
 * hipMalloc, no library allocation); its first call on a device looks up
 * that device's scratch address once.  Every call on one GPU shares that
 * GPU's scratch and nothing in it needs clearing (each call writes what it
 * reads), but calls that overlap in time on one GPU (two streams, or two
 * threads) race on it: order them on one stream.  Errors: as nvfp4_quantize;
 * BBS_EHIP if the scratch address cannot be found. */
int nvfp4_quantize_noalloc(const bbs_quant_args *a, void *stream);

/* MXFP4 copy of the BF16 matrix x (rows x cols, row stride ld elements,
 * x 16-byte aligned, ld % 8 == 0, cols % 32 == 0): per block of 32 values
 * of a row, scale 2^k with k = ceil(log2(amax / 6)) (the smallest k with
 * amax <= 6 * 2^k, clamped to [-127, 127]; amax 0 gives k = -127), and the
 * elements x * 2^-k rounded onto the E2M1 grid (nearest even, or stochastic
 * with the draws of rng as for the other copies).  out must be rows x cols.
 * Errors: BBS_EINVAL. */
int mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                   const bbs_mx4 *out, int32_t round, bbs_rng rng, void *stream);

/* Dequantize -> transpose -> requantize to MXFP8 (4bit.vizuara.ai, sections
 * 9-10; End-to-End 4-Bit Training, "requantization with stochastic
 * rounding").  src is an NVFP4 matrix R x C; dst receives the MXFP8 matrix of
 * src^T, shape C x R, blocks of 32 along R (R % 32 == 0).  Each value is
 * dequantized in FP32 as (E2M1 x E4M3) x s_dec, then encoded as in the MXFP8
 * copy of nvfp4_quantize with the given rounding and key.
 * Errors: BBS_EINVAL on null pointers or mismatched / unaligned shapes. */
int mxfp8_requantize_t(const bbs_fp4 *src, const bbs_mx8 *dst, int32_t round, bbs_rng rng,
                       void *stream);

/* Block-scaled GEMM C = A * B^T with FP32 accumulation (Pretraining LLMs
 * with NVFP4, "NVFP4 Format and Quantization Procedure", step 5;
 * 4bit.vizuara.ai, section 7).  Both operands carry their blocks along the
 * shared contraction dimension K = A.cols = B.cols; M = A.rows, N = B.rows.
 *   fmt == BBS_FMT_NVFP4: A, B are const bbs_fp4 *; C = s_dec,A * s_dec,B *
 *      sum over blocks of (E4M3_A * E4M3_B * sum of E2M1 products).
 *   fmt == BBS_FMT_MXFP8: A, B are const bbs_mx8 *; K % 32 == 0.
 *   fmt == BBS_FMT_MXFP4: A, B are const bbs_mx4 *; C = sum over 32-blocks
 *      of 2^(sa-127) * 2^(sb-127) * (sum of E2M1 products); K % 256 == 0,
 *      N % 4 == 0, 16-byte aligned C with ldc % 4 == 0 (else BBS_ENOTSUP).
 * C is M x N with row stride ldc (>= N) elements of c_dtype (BBS_OUT_F32 or
 * BBS_OUT_BF16, round to nearest even).  Output row i is scaled by
 * s_dec,A[i] * s_dec,B when A has a decode scale per row (then K % 128 == 0
 * and 16-byte aligned C, ldc * size % 16 == 0).
 * Errors: BBS_EINVAL; BBS_ENOTSUP for a per-row B scale or a per-row A
 * scale outside those conditions. */
int nvfp4_gemm(int32_t fmt, const void *A, const void *B, void *C, int32_t c_dtype,
               int64_t ldc, void *stream);

/* Grouped NVFP4 GEMM for mixture-of-experts layers (4bit.vizuara.ai,
 * section 11; End-to-End 4-Bit Training, "quantized communication"): for each
 * expert g, rows [group_offsets[g], group_offsets[g+1]) of the routed
 * activations times expert g's weights:
 *   C[i, :] = A_row(i) * B_g^T,   B_g = rows [g*N, (g+1)*N) of B, s_dec = B.s_dec[g]
 * A_row(i) is row row_index[i] of A, or row i when row_index is NULL.  A
 * dropped slot, i.e. a row_index entry that is negative or >= A.rows (or,
 * with row_index NULL, a routed row i >= A.rows), gives an output row of +0
 * (in the quantizing and encoding variants: the encode of a zero row, which
 * also leaves the reported amax unchanged).
 * group_offsets: device array of G+1 non-decreasing int64 (offsets[0] = 0);
 * empty groups are allowed.  max_rows bounds the routed rows C can hold
 * (rows beyond it are not computed).  B.rows == G * N, N % 16 == 0.
 * Tiles are scheduled on the device from group_offsets; the host never
 * reads them.  A per-row A decode scale is taken at A_row(i) (same
 * conditions as nvfp4_gemm).  Errors: BBS_EINVAL, BBS_ENOTSUP. */
int grouped_nvfp4_gemm(const bbs_fp4 *A, const int32_t *row_index,
                       const int64_t *group_offsets, int32_t G, int64_t max_rows,
                       const bbs_fp4 *B, int64_t N, void *C, int32_t c_dtype, int64_t ldc,
                       void *stream);

/* One S2F6 tensor (combine wire format; 4bit.vizuara.ai, section 11;
 * End-to-End 4-Bit Training, "quantized communication"): value =
 * code / 64 * 2^(scale - 127), int8 codes rows x cols, one E8M0 scale per
 * 32 consecutive values of a row (rows x cols/32 bytes): 8.25 bits per
 * value.  codes 16-byte aligned, cols % 32 == 0. */
typedef struct {
    int8_t *codes;
    uint8_t *scales;
    int64_t rows, cols;
} bbs_s2f6;

/* Encode of the combine wire format.  For each 32-value chunk of each row of
 * the BF16 matrix x (rows x cols, row stride ld elements, x 16-byte aligned,
 * ld % 8 == 0): with rht = 1, flip the sign of element i where bit i of
 * signs is set, apply the natural-order Sylvester Hadamard matrix as five
 * FP32 sum/difference stages (pair distance 1, 2, 4, 8, 16) and multiply by
 * 1/sqrt(32) rounded to FP32; then k = the smallest integer in [-127, 127]
 * with amax <= (127/64) 2^k, scale byte k + 127, codes rint(y 2^(6-k))
 * (nearest, ties to even; no value saturates).  out->rows/cols must equal
 * rows/cols.  Errors: BBS_EINVAL. */
int s2f6_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int32_t rht,
                  uint32_t signs, const bbs_s2f6 *out, void *stream);

/* Receiver side of the combine: for each token t < tokens and each 32-value
 * chunk, acc = sum over j = 0 .. k-1 (in order, FP32) of
 * weights[t*k + j] * decode(row src_index[t*k + j] of in), where decode is
 * exact and rows with a negative index are skipped (weights NULL: weight 1,
 * no multiply); with rht = 1 the inverse rotation follows (the same stages
 * and multiply, then the sign flips).  out is tokens x in->cols with row
 * stride ldo elements of out_dtype (BBS_OUT_F32, or BBS_OUT_BF16 rounded to
 * nearest even), 16-byte aligned with ldo * size % 16 == 0.  src_index
 * entries outside [0, in->rows) are skipped like negative ones.
 * Errors: BBS_EINVAL. */
int s2f6_combine(const bbs_s2f6 *in, const int32_t *src_index, const float *weights,
                 int64_t tokens, int32_t k, int32_t rht, uint32_t signs, void *out,
                 int32_t out_dtype, int64_t ldo, void *stream);

/* NVFP4 GEMM whose epilogue quantizes the product (4bit.vizuara.ai,
 * section 13; End-to-End 4-Bit Training, kernels for low-precision
 * training): the output never makes a round trip through memory.  With y =
 * the BF16 value nvfp4_gemm with BBS_OUT_BF16 would store, and with gelu = 1
 * y = GELU(y) (the tanh form of bbs_quant_args.gelu), Y receives the 1x16
 * NVFP4 copy of y encoded with the given tensor encode scale *s_enc (device,
 * one FP32; e.g. 2688 / a previous amax): per block, E4M3 code of
 * (amax_b / 6) * s_enc (nearest even, saturating at 448, never below code
 * 1), s_enc_b = 1 / (E4M3 * (1 / s_enc)), E2M1 codes of y * s_enc_b to
 * nearest even; Y->s_dec[0] = 1 / s_enc.  This is bit for bit the BF16 GEMM
 * followed by nvfp4_quantize with that encode scale.  Values beyond
 * 2688 / s_enc saturate.  amax (device, optional) receives max |y| over the
 * whole output (cleared by the call), e.g. the next call's scale.  ws
 * (BBS_AMAX_WS_FLOATS floats, 16-byte aligned) is needed with gelu (it
 * receives the GELU table).  Y must be rows x N (tile2d 0, one decode
 * scale); K % 128 == 0 and 16-byte aligned codes, 8-byte aligned scales
 * (else BBS_ENOTSUP).  Errors: BBS_EINVAL. */
int nvfp4_gemm_quant(const bbs_fp4 *A, const bbs_fp4 *B, const float *s_enc, int32_t gelu,
                     const bbs_fp4 *Y, float *amax, float *ws, void *stream);

/* The grouped GEMM (as grouped_nvfp4_gemm) with the same quantizing
 * epilogue: Y is max_rows x N. */
int grouped_nvfp4_gemm_quant(const bbs_fp4 *A, const int32_t *row_index,
                             const int64_t *group_offsets, int32_t G, int64_t max_rows,
                             const bbs_fp4 *B, int64_t N, const float *s_enc, int32_t gelu,
                             const bbs_fp4 *Y, float *amax, float *ws, void *stream);

/* NVFP4 GEMM whose epilogue encodes the product in the combine wire format
 * (4bit.vizuara.ai, section 11; End-to-End 4-Bit Training, "quantized
 * communication"): with y = the BF16 value nvfp4_gemm with BBS_OUT_BF16
 * would store, Y receives exactly what s2f6_quantize(y, rht, signs) writes,
 * without the BF16 output going to memory.  Y is rows x N (N % 32 == 0,
 * codes 16-byte aligned); K % 128 == 0 and 16-byte aligned codes, 8-byte
 * aligned scales (else BBS_ENOTSUP).  Errors: BBS_EINVAL. */
int nvfp4_gemm_s2f6(const bbs_fp4 *A, const bbs_fp4 *B, int32_t rht, uint32_t signs,
                    const bbs_s2f6 *Y, void *stream);

/* The grouped GEMM (as grouped_nvfp4_gemm) with the same encoding epilogue,
 * e.g. the experts' down projection feeding the combine: Y is
 * max_rows x N. */
int grouped_nvfp4_gemm_s2f6(const bbs_fp4 *A, const int32_t *row_index,
                            const int64_t *group_offsets, int32_t G, int64_t max_rows,
                            const bbs_fp4 *B, int64_t N, int32_t rht, uint32_t signs,
                            const bbs_s2f6 *Y, void *stream);

/* Name of a status code. */
const char *bbs_strerror(int status);

/* Text of the last error raised on the calling thread ("" if none). */
const char *bbs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BBS_H */

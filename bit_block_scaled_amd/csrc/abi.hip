// C ABI of the library (declared in include/bbs.h): argument checks, then
// kernel launches on the caller's stream.  Nothing here allocates device
// memory or synchronises the host.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>

#include "../../include/bbs.h"
#include "bbs_kernels.hpp"

static_assert(bbs::kWorkspaceFloats == BBS_AMAX_WS_FLOATS, "workspace size mismatch");

// The fixed device scratch of nvfp4_quantize_noalloc: the amax partials and
// the GELU table, BBS_AMAX_WS_FLOATS floats (45056 bytes) per GPU, held until
// the process ends.  Host code never uses the array's name as an address: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current, and is what the kernels receive.
static __device__ __align__(256) float scratch[BBS_AMAX_WS_FLOATS];

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return BBS_OK;
    return fail(BBS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape and pointer checks of one NVFP4 descriptor.
int check_fp4(const bbs_fp4 *d, const char *name, bool need_sdec) {
    if (!d) return fail(BBS_EINVAL, "%s: null descriptor", name);
    if (!d->codes || !d->scales || (need_sdec && !d->s_dec))
        return fail(BBS_EINVAL, "%s: null codes/scales/s_dec", name);
    if (d->rows <= 0 || d->cols <= 0 || d->rows % 16 || d->cols % 16)
        return fail(BBS_EINVAL, "%s: rows=%lld cols=%lld must be positive multiples of 16", name,
                    (long long)d->rows, (long long)d->cols);
    if (!aligned(d->codes, 16)) return fail(BBS_EINVAL, "%s: codes not 16-byte aligned", name);
    if (d->tile2d != 0 && d->tile2d != 1) return fail(BBS_EINVAL, "%s: tile2d must be 0 or 1", name);
    if (d->sdec_per_row != 0 && d->sdec_per_row != 1)
        return fail(BBS_EINVAL, "%s: sdec_per_row must be 0 or 1", name);
    if (d->sdec_per_row && d->tile2d)
        return fail(BBS_EINVAL, "%s: a per-row decode scale needs 1x16 blocks", name);
    return BBS_OK;
}

int check_mx8(const bbs_mx8 *d, const char *name) {
    if (!d) return fail(BBS_EINVAL, "%s: null descriptor", name);
    if (!d->codes || !d->scales) return fail(BBS_EINVAL, "%s: null codes/scales", name);
    if (d->rows <= 0 || d->cols <= 0 || d->cols % 32)
        return fail(BBS_EINVAL, "%s: rows=%lld cols=%lld (cols must be a multiple of 32)", name,
                    (long long)d->rows, (long long)d->cols);
    if (!aligned(d->codes, 16)) return fail(BBS_EINVAL, "%s: codes not 16-byte aligned", name);
    return BBS_OK;
}

bool round_ok(int32_t r) { return r == BBS_RTN || r == BBS_SR; }

int check_mx4(const bbs_mx4 *d, const char *name) {
    if (!d) return fail(BBS_EINVAL, "%s: null descriptor", name);
    if (!d->codes || !d->scales) return fail(BBS_EINVAL, "%s: null codes/scales", name);
    if (d->rows <= 0 || d->cols <= 0 || d->cols % 32)
        return fail(BBS_EINVAL, "%s: rows=%lld cols=%lld (cols must be a multiple of 32)", name,
                    (long long)d->rows, (long long)d->cols);
    if (!aligned(d->codes, 16)) return fail(BBS_EINVAL, "%s: codes not 16-byte aligned", name);
    return BBS_OK;
}

int check_s2f6(const bbs_s2f6 *d, const char *name) {
    if (!d) return fail(BBS_EINVAL, "%s: null descriptor", name);
    if (!d->codes || !d->scales) return fail(BBS_EINVAL, "%s: null codes/scales", name);
    if (d->rows <= 0 || d->cols <= 0 || d->cols % 32)
        return fail(BBS_EINVAL, "%s: rows=%lld cols=%lld (cols must be a multiple of 32)", name,
                    (long long)d->rows, (long long)d->cols);
    if (!aligned(d->codes, 16)) return fail(BBS_EINVAL, "%s: codes not 16-byte aligned", name);
    return BBS_OK;
}

}  // namespace

namespace bbs {

int device_cus(hipStream_t s) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (!s || hipStreamGetDevice(s, &dev) != hipSuccess)
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev < 0 || dev >= 64) dev = 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace bbs

extern "C" {

namespace {

// Shared checks of the quantizing GEMMs: the large-tile conditions and the
// NVFP4 output descriptor (rows x N, 1x16, one decode scale).
int check_quant_out(const bbs::GemmParams &p, const bbs_fp4 *Y, int64_t rows, const float *s_enc,
                    const float *amax, int32_t gelu, const float *ws) {
    int st;
    if ((st = check_fp4(Y, "Y", true))) return st;
    if (!s_enc) return fail(BBS_EINVAL, "null s_enc");
    if (gelu != 0 && gelu != 1) return fail(BBS_EINVAL, "gelu must be 0 or 1");
    if (gelu && (!ws || !aligned(ws, 16)))
        return fail(BBS_EINVAL, "gelu needs a 16-byte aligned workspace");
    if (Y->rows != rows || Y->cols != p.N) return fail(BBS_EINVAL, "Y must be rows x N");
    if (Y->tile2d || Y->sdec_per_row)
        return fail(BBS_EINVAL, "Y is a 1x16 copy with one decode scale");
    if (amax && !aligned(amax, 4)) return fail(BBS_EINVAL, "amax not 4-byte aligned");
    if (p.K % 128 || !aligned(p.a.codes, 16) || !aligned(p.b.codes, 16) || !aligned(p.a.scales, 8) ||
        !aligned(p.b.scales, 8))
        return fail(BBS_ENOTSUP, "quantizing GEMM needs K %% 128 == 0 and aligned operands");
    return BBS_OK;
}

bbs::QuantOut quant_out(const bbs_fp4 *Y, const float *s_enc, float *amax, float *ws) {
    return {Y->codes, Y->scales, Y->s_dec, s_enc, reinterpret_cast<unsigned *>(amax),
            ws ? ws + bbs::kGeluTabOffset : nullptr};
}

}  // namespace

int nvfp4_gemm_quant(const bbs_fp4 *A, const bbs_fp4 *B, const float *s_enc, int32_t gelu,
                     const bbs_fp4 *Y, float *amax, float *ws, void *stream) {
    g_err[0] = 0;
    int st;
    if ((st = check_fp4(A, "A", true))) return st;
    if ((st = check_fp4(B, "B", true))) return st;
    if (A->cols != B->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
    if (B->sdec_per_row) return fail(BBS_ENOTSUP, "B with a per-row decode scale");
    bbs::GemmParams p{};
    p.a = {A->codes, A->scales, A->s_dec, A->rows, A->tile2d, A->sdec_per_row};
    p.b = {B->codes, B->scales, B->s_dec, B->rows, B->tile2d, 0};
    p.M = A->rows;
    p.N = B->rows;
    p.K = A->cols;
    if ((st = check_quant_out(p, Y, p.M, s_enc, amax, gelu, ws))) return st;
    p.q = quant_out(Y, s_enc, amax, ws);
    return hip_status(bbs::launch_nvfp4_gemm_quant(p, gelu != 0,
                                                   reinterpret_cast<hipStream_t>(stream)),
                      "quantizing gemm launch");
}

int grouped_nvfp4_gemm_quant(const bbs_fp4 *A, const int32_t *row_index,
                             const int64_t *group_offsets, int32_t G, int64_t max_rows,
                             const bbs_fp4 *B, int64_t N, const float *s_enc, int32_t gelu,
                             const bbs_fp4 *Y, float *amax, float *ws, void *stream) {
    g_err[0] = 0;
    int st;
    if ((st = check_fp4(A, "A", true))) return st;
    if ((st = check_fp4(B, "B", true))) return st;
    if (!group_offsets) return fail(BBS_EINVAL, "null group_offsets");
    if (G <= 0 || G > 1024) return fail(BBS_EINVAL, "G must be in [1, 1024]");
    if (N <= 0 || N % 16 || B->rows != (int64_t)G * N)
        return fail(BBS_EINVAL, "B.rows must equal G * N with N %% 16 == 0");
    if (A->cols != B->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
    if (max_rows <= 0) return fail(BBS_EINVAL, "max_rows must be positive");
    if (B->sdec_per_row) return fail(BBS_ENOTSUP, "B with a per-row decode scale");
    bbs::GemmParams p{};
    p.a = {A->codes, A->scales, A->s_dec, A->rows, A->tile2d, A->sdec_per_row};
    p.b = {B->codes, B->scales, B->s_dec, N, B->tile2d, 0};
    p.M = max_rows;
    p.N = N;
    p.K = A->cols;
    p.row_index = row_index;
    p.group_offsets = group_offsets;
    p.G = G;
    p.max_rows = max_rows;
    p.a_src_rows = A->rows;
    if ((st = check_quant_out(p, Y, max_rows, s_enc, amax, gelu, ws))) return st;
    p.q = quant_out(Y, s_enc, amax, ws);
    return hip_status(bbs::launch_grouped_nvfp4_gemm_quant(p, gelu != 0,
                                                           reinterpret_cast<hipStream_t>(stream)),
                      "quantizing grouped gemm launch");
}

namespace {

// Shared checks of the GEMMs with the combine encode in the epilogue: the
// large-tile conditions and the S2F6 output (rows x N, N % 32 == 0).
int check_s2f6_out(const bbs::GemmParams &p, const bbs_s2f6 *Y, int64_t rows, int32_t rht) {
    int st;
    if ((st = check_s2f6(Y, "Y"))) return st;
    if (Y->rows != rows || Y->cols != p.N) return fail(BBS_EINVAL, "Y must be rows x N");
    if (rht != 0 && rht != 1) return fail(BBS_EINVAL, "rht must be 0 or 1");
    if (p.K % 128 || !aligned(p.a.codes, 16) || !aligned(p.b.codes, 16) || !aligned(p.a.scales, 8) ||
        !aligned(p.b.scales, 8))
        return fail(BBS_ENOTSUP, "encoding GEMM needs K %% 128 == 0 and aligned operands");
    return BBS_OK;
}

bbs::QuantOut s2f6_out(const bbs_s2f6 *Y, int32_t rht, uint32_t signs) {
    bbs::QuantOut q{};
    q.codes = reinterpret_cast<uint8_t *>(Y->codes);
    q.scales = Y->scales;
    q.signs = signs;
    q.rht = rht;
    return q;
}

}  // namespace

int nvfp4_gemm_s2f6(const bbs_fp4 *A, const bbs_fp4 *B, int32_t rht, uint32_t signs,
                    const bbs_s2f6 *Y, void *stream) {
    g_err[0] = 0;
    int st;
    if ((st = check_fp4(A, "A", true))) return st;
    if ((st = check_fp4(B, "B", true))) return st;
    if (A->cols != B->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
    if (B->sdec_per_row) return fail(BBS_ENOTSUP, "B with a per-row decode scale");
    bbs::GemmParams p{};
    p.a = {A->codes, A->scales, A->s_dec, A->rows, A->tile2d, A->sdec_per_row};
    p.b = {B->codes, B->scales, B->s_dec, B->rows, B->tile2d, 0};
    p.M = A->rows;
    p.N = B->rows;
    p.K = A->cols;
    if ((st = check_s2f6_out(p, Y, p.M, rht))) return st;
    p.q = s2f6_out(Y, rht, signs);
    return hip_status(bbs::launch_nvfp4_gemm_s2f6(p, reinterpret_cast<hipStream_t>(stream)),
                      "encoding gemm launch");
}

int grouped_nvfp4_gemm_s2f6(const bbs_fp4 *A, const int32_t *row_index,
                            const int64_t *group_offsets, int32_t G, int64_t max_rows,
                            const bbs_fp4 *B, int64_t N, int32_t rht, uint32_t signs,
                            const bbs_s2f6 *Y, void *stream) {
    g_err[0] = 0;
    int st;
    if ((st = check_fp4(A, "A", true))) return st;
    if ((st = check_fp4(B, "B", true))) return st;
    if (!group_offsets) return fail(BBS_EINVAL, "null group_offsets");
    if (G <= 0 || G > 1024) return fail(BBS_EINVAL, "G must be in [1, 1024]");
    if (N <= 0 || N % 16 || B->rows != (int64_t)G * N)
        return fail(BBS_EINVAL, "B.rows must equal G * N with N %% 16 == 0");
    if (A->cols != B->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
    if (max_rows <= 0) return fail(BBS_EINVAL, "max_rows must be positive");
    if (B->sdec_per_row) return fail(BBS_ENOTSUP, "B with a per-row decode scale");
    bbs::GemmParams p{};
    p.a = {A->codes, A->scales, A->s_dec, A->rows, A->tile2d, A->sdec_per_row};
    p.b = {B->codes, B->scales, B->s_dec, N, B->tile2d, 0};
    p.M = max_rows;
    p.N = N;
    p.K = A->cols;
    p.row_index = row_index;
    p.group_offsets = group_offsets;
    p.G = G;
    p.max_rows = max_rows;
    p.a_src_rows = A->rows;
    if ((st = check_s2f6_out(p, Y, max_rows, rht))) return st;
    p.q = s2f6_out(Y, rht, signs);
    return hip_status(bbs::launch_grouped_nvfp4_gemm_s2f6(p, reinterpret_cast<hipStream_t>(stream)),
                      "encoding grouped gemm launch");
}

int mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                   const bbs_mx4 *out, int32_t round, bbs_rng rng, void *stream) {
    g_err[0] = 0;
    int st;
    if (!x) return fail(BBS_EINVAL, "null x");
    if ((st = check_mx4(out, "out"))) return st;
    if (out->rows != rows || out->cols != cols) return fail(BBS_EINVAL, "out must be rows x cols");
    if (ld < cols || ld % 8) return fail(BBS_EINVAL, "ld must be >= cols and a multiple of 8");
    if (!aligned(x, 16)) return fail(BBS_EINVAL, "x not 16-byte aligned");
    if (!round_ok(round)) return fail(BBS_EINVAL, "bad round");
    return hip_status(bbs::launch_mxfp4_quant(x, rows, cols, ld, out->codes, out->scales,
                                              round == BBS_SR, rng.seed, rng.stream,
                                              reinterpret_cast<hipStream_t>(stream)),
                      "mxfp4 quantize launch");
}

int s2f6_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int32_t rht,
                  uint32_t signs, const bbs_s2f6 *out, void *stream) {
    g_err[0] = 0;
    int st;
    if (!x) return fail(BBS_EINVAL, "null x");
    if ((st = check_s2f6(out, "out"))) return st;
    if (out->rows != rows || out->cols != cols) return fail(BBS_EINVAL, "out must be rows x cols");
    if (ld < cols || ld % 8) return fail(BBS_EINVAL, "ld must be >= cols and a multiple of 8");
    if (!aligned(x, 16)) return fail(BBS_EINVAL, "x not 16-byte aligned");
    if (rht != 0 && rht != 1) return fail(BBS_EINVAL, "rht must be 0 or 1");
    return hip_status(bbs::launch_s2f6_encode(x, rows, cols, ld, rht != 0, signs, out->codes,
                                              out->scales, reinterpret_cast<hipStream_t>(stream)),
                      "s2f6 encode launch");
}

int s2f6_combine(const bbs_s2f6 *in, const int32_t *src_index, const float *weights,
                 int64_t tokens, int32_t k, int32_t rht, uint32_t signs, void *out,
                 int32_t out_dtype, int64_t ldo, void *stream) {
    g_err[0] = 0;
    int st;
    if ((st = check_s2f6(in, "in"))) return st;
    if (!src_index || !out) return fail(BBS_EINVAL, "null src_index / out");
    if (tokens <= 0 || k <= 0) return fail(BBS_EINVAL, "tokens and k must be positive");
    if (rht != 0 && rht != 1) return fail(BBS_EINVAL, "rht must be 0 or 1");
    if (out_dtype != BBS_OUT_F32 && out_dtype != BBS_OUT_BF16)
        return fail(BBS_EINVAL, "bad out_dtype");
    const int64_t esz = out_dtype == BBS_OUT_BF16 ? 2 : 4;
    if (ldo < in->cols || (ldo * esz) % 16 || !aligned(out, 16))
        return fail(BBS_EINVAL, "out must be 16-byte aligned with ldo >= cols, ldo * size %% 16 == 0");
    bbs::S2F6CombineParams p{};
    p.codes = in->codes;
    p.scales = in->scales;
    p.C = in->cols;
    p.src = src_index;
    p.src_rows = in->rows;
    p.w = weights;
    p.T = tokens;
    p.K = k;
    p.signs = signs;
    p.out = out;
    p.ldo = ldo;
    return hip_status(bbs::launch_s2f6_combine(p, rht != 0, out_dtype == BBS_OUT_BF16,
                                               reinterpret_cast<hipStream_t>(stream)),
                      "s2f6 combine launch");
}

const char *bbs_strerror(int status) {
    switch (status) {
        case BBS_OK: return "ok";
        case BBS_EINVAL: return "invalid argument";
        case BBS_ENOTSUP: return "unsupported combination";
        case BBS_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *bbs_last_error(void) { return g_err; }

namespace {

// The quantizer behind nvfp4_quantize and nvfp4_quantize_noalloc: ws is the
// amax workspace (BBS_AMAX_WS_FLOATS floats, 16-byte aligned) or nullptr.
// Validates every argument and, unless check_only, enqueues the passes.
// ws_in: the amax workspace (the caller's or the library's scratch).
int quantize_impl(const bbs_quant_args *a, float *ws_in, hipStream_t s, bool check_only = false) {
    if (!a) return fail(BBS_EINVAL, "null args");
    if (!a->x) return fail(BBS_EINVAL, "null x");
    if (!a->row && !a->col && !a->row_mx8) return fail(BBS_EINVAL, "no output copy requested");
    if (a->rows <= 0 || a->cols <= 0 || a->rows % 16 || a->cols % 16)
        return fail(BBS_EINVAL, "rows=%lld cols=%lld must be positive multiples of 16",
                    (long long)a->rows, (long long)a->cols);
    if (a->ld < a->cols || a->ld % 8) return fail(BBS_EINVAL, "ld must be >= cols and a multiple of 8");
    if (!aligned(a->x, 16)) return fail(BBS_EINVAL, "x not 16-byte aligned");
    if (a->tile2d != 0 && a->tile2d != 1) return fail(BBS_EINVAL, "tile2d must be 0 or 1");
    if ((a->row_per_token != 0 && a->row_per_token != 1) ||
        (a->row_four_six != 0 && a->row_four_six != 1))
        return fail(BBS_EINVAL, "row_per_token / row_four_six must be 0 or 1");
    if (a->gelu != 0 && a->gelu != 1) return fail(BBS_EINVAL, "gelu must be 0 or 1");
    const bool gelu = a->gelu != 0;
    if (gelu && (a->col || a->tile2d))
        return fail(BBS_ENOTSUP, "gelu applies to the row-wise 1x16 and MXFP8 copies");
    const bool act = a->row_per_token || a->row_four_six;
    if (act && (!a->row || a->col || a->row_mx8 || a->tile2d || a->row_round != BBS_RTN))
        return fail(BBS_ENOTSUP, "per-token / Four Over Six apply to a lone 1x16 RTN row copy");
    const bool need_ws = (a->row && !a->row_per_token) || a->col || gelu;
    if (need_ws && !ws_in) return fail(BBS_EINVAL, "null amax workspace");
    if (need_ws && !aligned(ws_in, 16))
        return fail(BBS_EINVAL, "amax workspace not 16-byte aligned");
    float *gelu_tab = gelu ? ws_in + bbs::kGeluTabOffset : nullptr;
    int st;
    if (a->row) {
        if ((st = check_fp4(a->row, "row", true))) return st;
        if (a->row->rows != a->rows || a->row->cols != a->cols)
            return fail(BBS_EINVAL, "row copy must be rows x cols");
        if (a->row->tile2d != a->tile2d) return fail(BBS_EINVAL, "row copy tile2d mismatch");
        if (a->row->sdec_per_row != a->row_per_token)
            return fail(BBS_EINVAL, "row copy sdec_per_row must equal row_per_token");
        if (!round_ok(a->row_round)) return fail(BBS_EINVAL, "bad row_round");
    }
    if (a->col) {
        if ((st = check_fp4(a->col, "col", true))) return st;
        if (a->col->rows != a->cols || a->col->cols != a->rows)
            return fail(BBS_EINVAL, "col copy must be cols x rows");
        if (a->col->tile2d != a->tile2d) return fail(BBS_EINVAL, "col copy tile2d mismatch");
        if (a->col->sdec_per_row) return fail(BBS_ENOTSUP, "col copy with a per-row decode scale");
        if (!round_ok(a->col_round)) return fail(BBS_EINVAL, "bad col_round");
        if (a->col_rht != 0 && a->col_rht != 1) return fail(BBS_EINVAL, "col_rht must be 0 or 1");
        if (a->col_rht && a->tile2d) return fail(BBS_ENOTSUP, "RHT on a 16x16-tiled copy");
        if (a->rht_signs > 0xFFFFu) return fail(BBS_EINVAL, "rht_signs has more than 16 bits");
    }
    if (a->row_mx8) {
        if ((st = check_mx8(a->row_mx8, "row_mx8"))) return st;
        if (a->row_mx8->rows != a->rows || a->row_mx8->cols != a->cols)
            return fail(BBS_EINVAL, "row_mx8 copy must be rows x cols");
        if (!round_ok(a->mx8_round)) return fail(BBS_EINVAL, "bad mx8_round");
    }
    if (check_only) return BBS_OK;

    bbs::QuantParams p{};
    p.x = a->x;
    p.R = a->rows;
    p.C = a->cols;
    p.ld = a->ld;
    p.gelu_tab = gelu_tab;
    if (act) {
        if (!a->row_per_token) {
            hipError_t e = bbs::launch_amax(a->x, a->rows, a->cols, a->ld, true, false, 0,
                                            ws_in, ws_in + bbs::kAmaxPartials,
                                            &p.n_part, s, gelu_tab);
            if ((st = hip_status(e, "amax launch"))) return st;
            p.part = ws_in;
        } else if (gelu) {
            if ((st = hip_status(bbs::launch_gelu_table(gelu_tab, s), "GELU table launch")))
                return st;
        }
        p.row_codes = a->row->codes;
        p.row_scales = a->row->scales;
        p.row_sdec = a->row->s_dec;
        return hip_status(bbs::launch_quant_act(p, a->row_per_token != 0, a->row_four_six != 0,
                                                gelu, s),
                          "activation quantize launch");
    }
    const bool rht = a->col && a->col_rht;
    const bool plain = a->row || (a->col && !rht);
    // An MXFP8 row copy needs no tensor scale: when an amax pass runs anyway
    // (and no GELU), that pass writes it from the same read.
    const bool mx_in_amax = a->row_mx8 && !gelu && (plain || rht);
    p.rht_signs = a->rht_signs;
    if (a->row_mx8) {
        p.mx_codes = a->row_mx8->codes;
        p.mx_scales = a->row_mx8->scales;
        p.mx_round = a->mx8_round;
        p.mx_seed = a->mx8_rng.seed;
        p.mx_stream = a->mx8_rng.stream;
    }
    if (plain || rht) {
        float *ws = ws_in;
        hipError_t e =
            mx_in_amax ? bbs::launch_amax_mx(p, plain, rht, ws, ws + bbs::kAmaxPartials, &p.n_part, s)
                       : bbs::launch_amax(a->x, a->rows, a->cols, a->ld, plain, rht, a->rht_signs,
                                          ws, ws + bbs::kAmaxPartials, &p.n_part, s, gelu_tab);
        if ((st = hip_status(e, "amax launch"))) return st;
        p.part = ws;
        p.part_rht = ws + bbs::kAmaxPartials;
        p.n_part_rht = p.n_part;
    } else if (gelu) {                  // an MXFP8 copy alone: no amax pass
        if ((st = hip_status(bbs::launch_gelu_table(gelu_tab, s), "GELU table launch"))) return st;
    }
    if (a->row) {
        p.row_codes = a->row->codes;
        p.row_scales = a->row->scales;
        p.row_sdec = a->row->s_dec;
        p.row_round = a->row_round;
        p.row_seed = a->row_rng.seed;
        p.row_stream = a->row_rng.stream;
    }
    if (a->col) {
        p.col_codes = a->col->codes;
        p.col_scales = a->col->scales;
        p.col_sdec = a->col->s_dec;
        p.col_round = a->col_round;
        p.col_seed = a->col_rng.seed;
        p.col_stream = a->col_rng.stream;
        p.rht_signs = a->rht_signs;
    }
    hipError_t e = bbs::launch_quant_tile(p, a->row != nullptr, a->col != nullptr,
                                          a->row_mx8 != nullptr && !mx_in_amax, a->tile2d != 0,
                                          rht, s, gelu);
    return hip_status(e, "quantize launch");
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that runs `s`.
int scratch_of(hipStream_t s, float **out) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "device of the stream");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BBS_ENOTSUP, "device %d is beyond the %d devices the scratch serves", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e, "hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (e2 != hipSuccess) return hip_status(e2, "hipSetDevice (restore)");
        if (!p || !aligned(p, 16)) return fail(BBS_EHIP, "scratch address unusable");
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return BBS_OK;
}

}  // namespace

int nvfp4_quantize(const bbs_quant_args *a, void *stream) {
    g_err[0] = 0;
    return quantize_impl(a, a ? a->amax_ws : nullptr, reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_quantize_noalloc(const bbs_quant_args *a, void *stream) {
    g_err[0] = 0;
    if (!a) return fail(BBS_EINVAL, "null args");
    if (a->amax_ws)
        return fail(BBS_EINVAL, "nvfp4_quantize_noalloc uses its own scratch: amax_ws must be NULL");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // arguments first (the scratch stands in by any aligned address), so a
    // bad call fails the same way with or without a device
    int st = quantize_impl(a, reinterpret_cast<float *>(static_cast<uintptr_t>(256)), s, true);
    if (st) return st;
    float *ws = nullptr;
    if ((st = scratch_of(s, &ws))) return st;
    return quantize_impl(a, ws, s);
}

int mxfp8_requantize_t(const bbs_fp4 *src, const bbs_mx8 *dst, int32_t round, bbs_rng rng,
                       void *stream) {
    g_err[0] = 0;
    int st;
    if ((st = check_fp4(src, "src", true))) return st;
    if ((st = check_mx8(dst, "dst"))) return st;
    if (dst->rows != src->cols || dst->cols != src->rows)
        return fail(BBS_EINVAL, "dst must be src.cols x src.rows");
    if (src->rows % 32) return fail(BBS_EINVAL, "src.rows must be a multiple of 32");
    if (src->sdec_per_row) return fail(BBS_ENOTSUP, "requantize of a per-row-scaled copy");
    if (!round_ok(round)) return fail(BBS_EINVAL, "bad round");
    if (!aligned(src->codes, 8)) return fail(BBS_EINVAL, "src codes not 8-byte aligned");
    bbs::RequantParams p{};
    p.codes = src->codes;
    p.scales = src->scales;
    p.s_dec = src->s_dec;
    p.R = src->rows;
    p.C = src->cols;
    p.tile2d = src->tile2d;
    p.out_codes = dst->codes;
    p.out_scales = dst->scales;
    p.seed = rng.seed;
    p.stream = rng.stream;
    return hip_status(bbs::launch_requant(p, round == BBS_SR, reinterpret_cast<hipStream_t>(stream)),
                      "requantize launch");
}

int nvfp4_gemm(int32_t fmt, const void *A, const void *B, void *C, int32_t c_dtype, int64_t ldc,
               void *stream) {
    g_err[0] = 0;
    if (!C) return fail(BBS_EINVAL, "null C");
    if (c_dtype != BBS_OUT_F32 && c_dtype != BBS_OUT_BF16) return fail(BBS_EINVAL, "bad c_dtype");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int st;
    if (fmt == BBS_FMT_NVFP4) {
        const bbs_fp4 *a = static_cast<const bbs_fp4 *>(A), *b = static_cast<const bbs_fp4 *>(B);
        if ((st = check_fp4(a, "A", true))) return st;
        if ((st = check_fp4(b, "B", true))) return st;
        if (a->cols != b->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
        if (ldc < b->rows) return fail(BBS_EINVAL, "ldc < N");
        bbs::GemmParams p{};
        if (b->sdec_per_row) return fail(BBS_ENOTSUP, "B with a per-row decode scale");
        p.a = {a->codes, a->scales, a->s_dec, a->rows, a->tile2d, a->sdec_per_row};
        p.b = {b->codes, b->scales, b->s_dec, b->rows, b->tile2d, 0};
        p.M = a->rows;
        p.N = b->rows;
        p.K = a->cols;
        p.c = C;
        p.ldc = ldc;
        if (a->sdec_per_row && !bbs::big_ok(p, c_dtype == BBS_OUT_BF16))
            return fail(BBS_ENOTSUP, "per-row A scale needs K %% 128 == 0 and aligned operands / C");
        return hip_status(bbs::launch_nvfp4_gemm(p, c_dtype == BBS_OUT_BF16, s), "gemm launch");
    }
    if (fmt == BBS_FMT_MXFP8) {
        const bbs_mx8 *a = static_cast<const bbs_mx8 *>(A), *b = static_cast<const bbs_mx8 *>(B);
        if ((st = check_mx8(a, "A"))) return st;
        if ((st = check_mx8(b, "B"))) return st;
        if (a->cols != b->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
        if (ldc < b->rows) return fail(BBS_EINVAL, "ldc < N");
        bbs::Mx8GemmParams p{};
        p.a_codes = a->codes;
        p.a_scales = a->scales;
        p.b_codes = b->codes;
        p.b_scales = b->scales;
        p.M = a->rows;
        p.N = b->rows;
        p.K = a->cols;
        p.c = C;
        p.ldc = ldc;
        return hip_status(bbs::launch_mxfp8_gemm(p, c_dtype == BBS_OUT_BF16, s), "mxfp8 gemm launch");
    }
    if (fmt == BBS_FMT_MXFP4) {
        const bbs_mx4 *a = static_cast<const bbs_mx4 *>(A), *b = static_cast<const bbs_mx4 *>(B);
        if ((st = check_mx4(a, "A"))) return st;
        if ((st = check_mx4(b, "B"))) return st;
        if (a->cols != b->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
        if (ldc < b->rows) return fail(BBS_EINVAL, "ldc < N");
        if (a->cols % 256) return fail(BBS_ENOTSUP, "MXFP4 GEMM needs K %% 256 == 0");
        if (!aligned(a->scales, 4) || !aligned(b->scales, 4))
            return fail(BBS_ENOTSUP, "MXFP4 GEMM needs 4-byte aligned scales");
        if (b->rows % 4 || !aligned(C, 16) || ldc % 4)
            return fail(BBS_ENOTSUP, "MXFP4 GEMM needs N %% 4 == 0, 16-byte aligned C, ldc %% 4 == 0");
        bbs::Mx8GemmParams p{};
        p.a_codes = a->codes;
        p.a_scales = a->scales;
        p.b_codes = b->codes;
        p.b_scales = b->scales;
        p.M = a->rows;
        p.N = b->rows;
        p.K = a->cols;
        p.c = C;
        p.ldc = ldc;
        return hip_status(bbs::launch_mxfp4_gemm(p, c_dtype == BBS_OUT_BF16, s), "mxfp4 gemm launch");
    }
    return fail(BBS_EINVAL, "unknown fmt %d", fmt);
}

int grouped_nvfp4_gemm(const bbs_fp4 *A, const int32_t *row_index, const int64_t *group_offsets,
                       int32_t G, int64_t max_rows, const bbs_fp4 *B, int64_t N, void *C,
                       int32_t c_dtype, int64_t ldc, void *stream) {
    g_err[0] = 0;
    int st;
    if ((st = check_fp4(A, "A", true))) return st;
    if ((st = check_fp4(B, "B", true))) return st;
    if (!group_offsets) return fail(BBS_EINVAL, "null group_offsets");
    if (!C) return fail(BBS_EINVAL, "null C");
    if (G <= 0 || G > 1024) return fail(BBS_EINVAL, "G must be in [1, 1024]");
    if (N <= 0 || N % 16 || B->rows != (int64_t)G * N)
        return fail(BBS_EINVAL, "B.rows must equal G * N with N %% 16 == 0");
    if (A->cols != B->cols) return fail(BBS_EINVAL, "A.cols != B.cols");
    if (max_rows < 0) return fail(BBS_EINVAL, "max_rows < 0");
    if (ldc < N) return fail(BBS_EINVAL, "ldc < N");
    if (c_dtype != BBS_OUT_F32 && c_dtype != BBS_OUT_BF16) return fail(BBS_EINVAL, "bad c_dtype");
    bbs::GemmParams p{};
    if (B->sdec_per_row) return fail(BBS_ENOTSUP, "B with a per-row decode scale");
    p.a = {A->codes, A->scales, A->s_dec, A->rows, A->tile2d, A->sdec_per_row};
    p.b = {B->codes, B->scales, B->s_dec, N, B->tile2d, 0};
    p.M = max_rows;
    p.N = N;
    p.K = A->cols;
    p.c = C;
    p.ldc = ldc;
    p.row_index = row_index;
    p.group_offsets = group_offsets;
    p.G = G;
    p.max_rows = max_rows;
    p.a_src_rows = A->rows;
    if (A->sdec_per_row && !bbs::big_ok(p, c_dtype == BBS_OUT_BF16))
        return fail(BBS_ENOTSUP, "per-row A scale needs K %% 128 == 0 and aligned operands / C");
    return hip_status(bbs::launch_grouped_nvfp4_gemm(p, c_dtype == BBS_OUT_BF16,
                                                     reinterpret_cast<hipStream_t>(stream)),
                      "grouped gemm launch");
}

}  // extern "C"

"""CPU-only checks of the C ABI library: it loads, it exports every entry
point the header declares, and argument errors come back as status codes
before any GPU work is attempted."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_block_scaled_amd", "libbbs.so")
HDR = os.path.join(ROOT, "include", "bbs.h")


def _declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_lists_the_entry_points():
    names = _declared()
    for n in ["nvfp4_quantize", "mxfp8_requantize_t", "nvfp4_gemm", "grouped_nvfp4_gemm",
              "bbs_strerror", "bbs_last_error"]:
        assert n in names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libbbs.so is not built (run __graft_entry__.build())")
    return C.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_error_paths_return_status(lib):
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    # null argument block / null x / no copy requested
    assert L.nvfp4_quantize(None, None) == bbs.BBS_EINVAL
    a = bbs.QuantArgs()
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"null x" in L.bbs_last_error()
    a.x = 0x1000
    a.rows, a.cols, a.ld = 32, 32, 32
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"no output copy" in L.bbs_last_error()
    # shapes that are not multiples of 16
    d = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 30, 32, 0)
    a.row = C.pointer(d)
    a.rows = 30
    a.amax_ws = 0x4000
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    # misaligned x
    a.rows, d.rows = 32, 32
    a.x = 0x1002
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"aligned" in L.bbs_last_error()
    # RHT on a 16x16-tiled copy is not supported
    a.x = 0x1000
    a.row = None
    cd = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 32, 1)
    a.col = C.pointer(cd)
    a.tile2d = 1
    a.col_rht = 1
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_ENOTSUP
    # bad rounding mode
    a.col_rht = 0
    a.col_round = 7
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    # GEMM: mismatched K, null C, bad dtype, bad fmt
    A = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 64, 0)
    B = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 48, 32, 0)
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), C.c_void_p(0x5000), 0, 48, None) == bbs.BBS_EINVAL
    B.cols = 64
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), None, 0, 48, None) == bbs.BBS_EINVAL
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), C.c_void_p(0x5000), 9, 48, None) == bbs.BBS_EINVAL
    assert L.nvfp4_gemm(5, C.byref(A), C.byref(B), C.c_void_p(0x5000), 0, 48, None) == bbs.BBS_EINVAL
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), C.c_void_p(0x5000), 0, 40, None) == bbs.BBS_EINVAL
    # MXFP8 operands need cols % 32 == 0
    MA = bbs.Mx8Desc(0x1000, 0x2000, 32, 48)
    MB = bbs.Mx8Desc(0x1000, 0x2000, 32, 48)
    assert L.nvfp4_gemm(1, C.byref(MA), C.byref(MB), C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_EINVAL
    # requantize: source rows must be a multiple of 32, dst the transpose
    src = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 48, 32, 0)
    dst = bbs.Mx8Desc(0x1000, 0x2000, 32, 48)
    assert L.mxfp8_requantize_t(C.byref(src), C.byref(dst), 1, bbs.Rng(0, 0), None) == bbs.BBS_EINVAL
    # grouped: B rows must be G * N, G in range
    gA = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 64, 64, 0)
    gB = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 96, 64, 1)
    assert L.grouped_nvfp4_gemm(C.byref(gA), None, C.c_void_p(0x6000), 4, 64, C.byref(gB), 32,
                                C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_EINVAL
    assert L.grouped_nvfp4_gemm(C.byref(gA), None, C.c_void_p(0x6000), 0, 64, C.byref(gB), 32,
                                C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_EINVAL
    assert L.grouped_nvfp4_gemm(C.byref(gA), None, None, 3, 64, C.byref(gB), 32,
                                C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_EINVAL
    assert L.bbs_strerror(bbs.BBS_EINVAL) == b"invalid argument"


def test_empty_tensors_are_rejected(lib):
    """Zero rows or columns are invalid shapes (BBS_EINVAL, nothing
    launched), for the quantizer, the requantizer and the GEMMs."""
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    for rows, cols in ((0, 32), (32, 0), (0, 0)):
        a = bbs.QuantArgs()
        a.x, a.rows, a.cols, a.ld, a.amax_ws = 0x1000, rows, cols, max(cols, 16), 0x4000
        d = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, rows, cols, 0)
        a.row = C.pointer(d)
        assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL, (rows, cols)
        a.amax_ws = None
        assert L.nvfp4_quantize_noalloc(C.byref(a), None) == bbs.BBS_EINVAL, (rows, cols)
        assert b"amax_ws" not in L.bbs_last_error()
        src = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, rows, cols, 0)
        dst = bbs.Mx8Desc(0x1000, 0x2000, cols, rows)
        assert L.mxfp8_requantize_t(C.byref(src), C.byref(dst), 0, bbs.Rng(0, 0), None) == \
            bbs.BBS_EINVAL
    A = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 0, 64, 0)
    B = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 48, 64, 0)
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), C.c_void_p(0x5000), 0, 48, None) == bbs.BBS_EINVAL
    A.rows, B.rows = 32, 0
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), C.c_void_p(0x5000), 0, 48, None) == bbs.BBS_EINVAL


def test_activation_option_errors(lib):
    """Per-token / Four Over Six: only on a lone 1x16 RTN row copy whose
    descriptor carries per-row decode scales exactly when per-token."""
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    a = bbs.QuantArgs()
    a.x, a.rows, a.cols, a.ld = 0x1000, 32, 64, 64
    row = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 64, 0, 1)
    a.row = C.pointer(row)
    a.row_per_token = 2
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    a.row_per_token = 1
    a.row_round = bbs.SR
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_ENOTSUP
    a.row_round = bbs.RTN
    col = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 64, 32, 0, 0)
    a.col = C.pointer(col)
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_ENOTSUP
    a.col = None
    row.sdec_per_row = 0                      # per-token output needs per-row s_dec
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    row.sdec_per_row, row.tile2d = 1, 1       # per-row decode scales need 1x16 blocks
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    # Four Over Six with a tensor scale still needs the amax workspace
    row.sdec_per_row, row.tile2d = 0, 0
    a.row_per_token, a.row_four_six = 0, 1
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"workspace" in L.bbs_last_error()
    # GEMM: a per-row B scale is not supported; a per-row A scale needs K % 128
    A = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 64, 0, 1)
    B = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 64, 0, 1)
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_ENOTSUP
    B.sdec_per_row = 0
    assert L.nvfp4_gemm(0, C.byref(A), C.byref(B), C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_ENOTSUP
    assert b"128" in L.bbs_last_error()
    # requantize of a per-row-scaled copy is not supported
    src = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 64, 32, 0, 1)
    dst = bbs.Mx8Desc(0x1000, 0x2000, 32, 64)
    assert L.mxfp8_requantize_t(C.byref(src), C.byref(dst), 1, bbs.Rng(0, 0), None) == bbs.BBS_ENOTSUP


def test_binding_has_no_cpu_fallback():
    import bit_block_scaled_amd as bbs
    src = open(bbs.__file__).read()
    assert "oracle" not in src.replace("no CPU fallback", "")


def test_gelu_option_errors(lib):
    """gelu: 0 or 1; with a column copy or 16x16 tiles it is unsupported."""
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    a = bbs.QuantArgs()
    a.x, a.rows, a.cols, a.ld = 0x1000, 32, 64, 64
    row = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 64, 0, 0)
    a.row = C.pointer(row)
    a.gelu = 2
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    a.gelu = 1
    col = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 64, 32, 0, 0)
    a.col = C.pointer(col)
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_ENOTSUP
    a.col = None
    a.tile2d, row.tile2d = 1, 1
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_ENOTSUP
    assert b"gelu" in L.bbs_last_error()
    # the GELU table lives in the workspace, also for a per-token copy
    a.tile2d, row.tile2d = 0, 0
    a.row_per_token, row.sdec_per_row = 1, 1
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"workspace" in L.bbs_last_error()
    a.amax_ws = 0x4004
    assert L.nvfp4_quantize(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"aligned" in L.bbs_last_error()


def test_s2f6_errors(lib):
    """Combine wire format: shapes, pointers and output layout are checked."""
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    d = bbs.S2F6Desc(0x1000, 0x2000, 8, 48)                 # cols not a multiple of 32
    assert L.s2f6_quantize(C.c_void_p(0x1000), 8, 48, 48, 1, 0, C.byref(d), None) == bbs.BBS_EINVAL
    d.cols = 64
    assert L.s2f6_quantize(None, 8, 64, 64, 1, 0, C.byref(d), None) == bbs.BBS_EINVAL
    assert L.s2f6_quantize(C.c_void_p(0x1000), 8, 64, 60, 1, 0, C.byref(d), None) == bbs.BBS_EINVAL
    assert L.s2f6_quantize(C.c_void_p(0x1000), 8, 64, 64, 2, 0, C.byref(d), None) == bbs.BBS_EINVAL
    assert L.s2f6_quantize(C.c_void_p(0x1000), 16, 64, 64, 1, 0, C.byref(d), None) == bbs.BBS_EINVAL
    src, out = C.c_void_p(0x3000), C.c_void_p(0x4000)
    assert L.s2f6_combine(C.byref(d), None, None, 4, 2, 1, 0, out, 1, 64, None) == bbs.BBS_EINVAL
    assert L.s2f6_combine(C.byref(d), src, None, 0, 2, 1, 0, out, 1, 64, None) == bbs.BBS_EINVAL
    assert L.s2f6_combine(C.byref(d), src, None, 4, 2, 1, 0, out, 7, 64, None) == bbs.BBS_EINVAL
    assert L.s2f6_combine(C.byref(d), src, None, 4, 2, 1, 0, out, 1, 60, None) == bbs.BBS_EINVAL
    assert L.s2f6_combine(C.byref(d), src, None, 4, 2, 1, 0, C.c_void_p(0x4004), 1, 64,
                          None) == bbs.BBS_EINVAL
    assert b"aligned" in L.bbs_last_error()


def test_mxfp4_errors(lib):
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    d = bbs.Mx4Desc(0x1000, 0x2000, 8, 48)                  # cols not a multiple of 32
    assert L.mxfp4_quantize(C.c_void_p(0x1000), 8, 48, 48, C.byref(d), 0, bbs.Rng(0, 0),
                            None) == bbs.BBS_EINVAL
    d.cols = 64
    assert L.mxfp4_quantize(C.c_void_p(0x1000), 8, 64, 64, C.byref(d), 5, bbs.Rng(0, 0),
                            None) == bbs.BBS_EINVAL
    a = bbs.Mx4Desc(0x1000, 0x2000, 32, 128)
    b = bbs.Mx4Desc(0x1000, 0x2000, 32, 128)
    assert L.nvfp4_gemm(2, C.byref(a), C.byref(b), C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_ENOTSUP
    assert b"256" in L.bbs_last_error()
    a.cols = b.cols = 256
    b.rows = 30
    assert L.nvfp4_gemm(2, C.byref(a), C.byref(b), C.c_void_p(0x5000), 0, 32, None) == bbs.BBS_ENOTSUP


def test_gemm_quant_errors(lib):
    """The quantizing GEMMs: Y must be a rows x N 1x16 copy, s_enc given,
    K % 128 (else unsupported)."""
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    A = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 128, 0, 0)
    B = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 48, 128, 1, 0)
    Y = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 48, 0, 0)
    s = C.c_void_p(0x4000)
    q = lambda s_, g, ws=None: L.nvfp4_gemm_quant(C.byref(A), C.byref(B), s_, g, C.byref(Y), None,
                                                  ws, None)
    assert q(None, 0) == bbs.BBS_EINVAL
    assert q(s, 2) == bbs.BBS_EINVAL
    assert q(s, 1) == bbs.BBS_EINVAL                      # GELU needs the workspace
    assert b"workspace" in L.bbs_last_error()
    Y.rows = 16
    assert q(s, 0) == bbs.BBS_EINVAL
    Y.rows, Y.tile2d = 32, 1
    assert q(s, 0) == bbs.BBS_EINVAL
    Y.tile2d = 0
    A.cols = B.cols = 64
    assert q(s, 0) == bbs.BBS_ENOTSUP
    assert L.grouped_nvfp4_gemm_quant(C.byref(A), None, None, 1, 32, C.byref(B), 48, s, 0,
                                      C.byref(Y), None, None, None) == bbs.BBS_EINVAL


def test_gemm_s2f6_errors(lib):
    """The GEMMs with the combine encode in the epilogue: Y must be an S2F6
    rows x N tensor with N % 32 == 0, rht 0 or 1, K % 128 (else unsupported)."""
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    A = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 128, 0, 0)
    B = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 64, 128, 1, 0)
    Y = bbs.S2F6Desc(0x1000, 0x2000, 32, 64)
    e = lambda r=1: L.nvfp4_gemm_s2f6(C.byref(A), C.byref(B), r, 0x1234, C.byref(Y), None)
    assert e(2) == bbs.BBS_EINVAL
    Y.rows = 16
    assert e() == bbs.BBS_EINVAL
    Y.rows, Y.cols = 32, 48
    assert e() == bbs.BBS_EINVAL                          # cols not a multiple of 32
    Y.cols = 64
    Y.codes = 0x1008
    assert e() == bbs.BBS_EINVAL                          # codes not 16-byte aligned
    Y.codes = 0x1000
    A.cols = B.cols = 64
    assert e() == bbs.BBS_ENOTSUP
    A.cols = B.cols = 128
    assert L.grouped_nvfp4_gemm_s2f6(C.byref(A), None, None, 1, 32, C.byref(B), 64, 1, 0,
                                     C.byref(Y), None) == bbs.BBS_EINVAL     # no offsets
    assert L.grouped_nvfp4_gemm_s2f6(C.byref(A), None, C.c_void_p(0x4000), 2, 32, C.byref(B), 64,
                                     1, 0, C.byref(Y), None) == bbs.BBS_EINVAL  # B.rows != G N


def test_noalloc_error_paths_need_no_gpu(lib):
    import bit_block_scaled_amd as bbs
    L = bbs.lib
    assert L.nvfp4_quantize_noalloc(None, None) == bbs.BBS_EINVAL
    d = bbs.Fp4Desc(0x1000, 0x2000, 0x3000, 32, 32, 0)
    a = bbs.QuantArgs()
    a.x, a.rows, a.cols, a.ld = 0x1000, 32, 32, 32
    a.row = C.pointer(d)
    a.amax_ws = 0x4000          # the variant brings its own scratch
    assert L.nvfp4_quantize_noalloc(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"amax_ws must be NULL" in L.bbs_last_error()

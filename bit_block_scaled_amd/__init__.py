"""Python binding of libbbs.so, the MI355X NVFP4 quantized-linear library.

Argument marshalling only: every step of the hot path runs in the HIP kernels
behind the C ABI declared in include/bbs.h.  PyTorch is used for device
memory and streams.  The functions have the names of the C entry points and
raise BbsError on a non-zero status.  There is no CPU fallback: importing
this module fails if the library has not been built.
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbbs.so")

BBS_OK, BBS_EINVAL, BBS_ENOTSUP, BBS_EHIP = 0, -1, -2, -3
RTN, SR = 0, 1
OUT_F32, OUT_BF16 = 0, 1
FMT_NVFP4, FMT_MXFP8, FMT_MXFP4 = 0, 1, 2
AMAX_WS_FLOATS = 11264


class Fp4Desc(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("s_dec", C.c_void_p),
                ("rows", C.c_int64), ("cols", C.c_int64), ("tile2d", C.c_int32),
                ("sdec_per_row", C.c_int32)]


class Mx8Desc(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("rows", C.c_int64),
                ("cols", C.c_int64)]


class Mx4Desc(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("rows", C.c_int64),
                ("cols", C.c_int64)]


class S2F6Desc(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("rows", C.c_int64),
                ("cols", C.c_int64)]


class Rng(C.Structure):
    _fields_ = [("seed", C.c_uint64), ("stream", C.c_uint32)]


class QuantArgs(C.Structure):
    _fields_ = [("x", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64), ("ld", C.c_int64),
                ("row", C.POINTER(Fp4Desc)), ("row_round", C.c_int32), ("row_rng", Rng),
                ("col", C.POINTER(Fp4Desc)), ("col_round", C.c_int32), ("col_rng", Rng),
                ("col_rht", C.c_int32), ("rht_signs", C.c_uint32),
                ("row_mx8", C.POINTER(Mx8Desc)), ("mx8_round", C.c_int32), ("mx8_rng", Rng),
                ("tile2d", C.c_int32), ("amax_ws", C.c_void_p),
                ("row_per_token", C.c_int32), ("row_four_six", C.c_int32),
                ("gelu", C.c_int32)]


class BbsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"bbs status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    lib.nvfp4_quantize.argtypes = [C.POINTER(QuantArgs), vp]
    lib.nvfp4_quantize_noalloc.argtypes = [C.POINTER(QuantArgs), vp]
    lib.mxfp8_requantize_t.argtypes = [C.POINTER(Fp4Desc), C.POINTER(Mx8Desc), i32, Rng, vp]
    lib.nvfp4_gemm.argtypes = [i32, vp, vp, vp, i32, i64, vp]
    lib.grouped_nvfp4_gemm.argtypes = [C.POINTER(Fp4Desc), vp, vp, i32, i64, C.POINTER(Fp4Desc),
                                       i64, vp, i32, i64, vp]
    lib.mxfp4_quantize.argtypes = [vp, i64, i64, i64, C.POINTER(Mx4Desc), i32, Rng, vp]
    lib.nvfp4_gemm_quant.argtypes = [C.POINTER(Fp4Desc), C.POINTER(Fp4Desc), vp, i32,
                                     C.POINTER(Fp4Desc), vp, vp, vp]
    lib.grouped_nvfp4_gemm_quant.argtypes = [C.POINTER(Fp4Desc), vp, vp, i32, i64,
                                             C.POINTER(Fp4Desc), i64, vp, i32, C.POINTER(Fp4Desc),
                                             vp, vp, vp]
    lib.nvfp4_gemm_s2f6.argtypes = [C.POINTER(Fp4Desc), C.POINTER(Fp4Desc), i32, C.c_uint32,
                                    C.POINTER(S2F6Desc), vp]
    lib.grouped_nvfp4_gemm_s2f6.argtypes = [C.POINTER(Fp4Desc), vp, vp, i32, i64,
                                            C.POINTER(Fp4Desc), i64, i32, C.c_uint32,
                                            C.POINTER(S2F6Desc), vp]
    lib.s2f6_quantize.argtypes = [vp, i64, i64, i64, i32, C.c_uint32, C.POINTER(S2F6Desc), vp]
    lib.s2f6_combine.argtypes = [C.POINTER(S2F6Desc), vp, vp, i64, i32, i32, C.c_uint32, vp, i32,
                                 i64, vp]
    for f in ("nvfp4_quantize", "nvfp4_quantize_noalloc", "mxfp8_requantize_t", "nvfp4_gemm", "grouped_nvfp4_gemm",
              "s2f6_quantize", "s2f6_combine", "mxfp4_quantize", "nvfp4_gemm_quant",
              "grouped_nvfp4_gemm_quant", "nvfp4_gemm_s2f6", "grouped_nvfp4_gemm_s2f6"):
        getattr(lib, f).restype = C.c_int
    lib.bbs_strerror.argtypes = [C.c_int]
    lib.bbs_strerror.restype = C.c_char_p
    lib.bbs_last_error.argtypes = []
    lib.bbs_last_error.restype = C.c_char_p
    return lib


lib = _load()


def _check(status):
    if status != BBS_OK:
        raise BbsError(status, lib.bbs_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# Tensor containers (device memory comes from PyTorch)
# ---------------------------------------------------------------------------

class NVFP4Tensor:
    """codes [rows, cols/2] u8, scales [rows(/16), cols/16] u8, s_dec [n] f32
    (n = 1, G stacked experts, or rows when sdec_per_row)."""

    def __init__(self, codes, scales, s_dec, rows, cols, tile2d, sdec_per_row=False):
        self.codes, self.scales, self.s_dec = codes, scales, s_dec
        self.rows, self.cols, self.tile2d = rows, cols, int(tile2d)
        self.sdec_per_row = int(sdec_per_row)

    @staticmethod
    def empty(rows, cols, tile2d=False, n_scales=1, device="cuda", sdec_per_row=False):
        srows = rows // 16 if tile2d else rows
        n = rows if sdec_per_row else n_scales
        return NVFP4Tensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                           torch.empty((srows, cols // 16), dtype=torch.uint8, device=device),
                           torch.empty((n,), dtype=torch.float32, device=device),
                           rows, cols, tile2d, sdec_per_row)

    def desc(self):
        return Fp4Desc(_ptr(self.codes), _ptr(self.scales), _ptr(self.s_dec), self.rows,
                       self.cols, self.tile2d, self.sdec_per_row)


class MXFP8Tensor:
    """codes [rows, cols] u8 (E4M3), scales [rows, cols/32] u8 (E8M0)."""

    def __init__(self, codes, scales, rows, cols):
        self.codes, self.scales, self.rows, self.cols = codes, scales, rows, cols

    @staticmethod
    def empty(rows, cols, device="cuda"):
        return MXFP8Tensor(torch.empty((rows, cols), dtype=torch.uint8, device=device),
                           torch.empty((rows, cols // 32), dtype=torch.uint8, device=device),
                           rows, cols)

    def desc(self):
        return Mx8Desc(_ptr(self.codes), _ptr(self.scales), self.rows, self.cols)


class MXFP4Tensor:
    """codes [rows, cols/2] u8 (E2M1 pairs, even column low), scales [rows, cols/32] u8 (E8M0)."""

    def __init__(self, codes, scales, rows, cols):
        self.codes, self.scales, self.rows, self.cols = codes, scales, rows, cols

    @staticmethod
    def empty(rows, cols, device="cuda"):
        return MXFP4Tensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                           torch.empty((rows, cols // 32), dtype=torch.uint8, device=device),
                           rows, cols)

    def desc(self):
        return Mx4Desc(_ptr(self.codes), _ptr(self.scales), self.rows, self.cols)


class S2F6Tensor:
    """codes [rows, cols] int8 (value code / 64), scales [rows, cols/32] u8 (E8M0)."""

    def __init__(self, codes, scales, rows, cols):
        self.codes, self.scales, self.rows, self.cols = codes, scales, rows, cols

    @staticmethod
    def empty(rows, cols, device="cuda"):
        return S2F6Tensor(torch.empty((rows, cols), dtype=torch.int8, device=device),
                          torch.empty((rows, cols // 32), dtype=torch.uint8, device=device),
                          rows, cols)

    def desc(self):
        return S2F6Desc(_ptr(self.codes), _ptr(self.scales), self.rows, self.cols)


def amax_workspace(device="cuda"):
    return torch.empty((AMAX_WS_FLOATS,), dtype=torch.float32, device=device)


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------

def nvfp4_quantize(x, row=None, col=None, row_mx8=None, *, row_round=RTN, row_rng=(0, 0),
                   col_round=RTN, col_rng=(0, 0), col_rht=False, rht_signs=0, mx8_round=RTN,
                   mx8_rng=(0, 0), tile2d=False, amax_ws=None, row_per_token=False,
                   row_four_six=False, gelu=False, stream=None):
    """x: BF16 bit patterns as a [rows, cols] int16/uint16/bfloat16 device tensor
    (row stride x.stride(0)).  row / col: NVFP4Tensor outputs; row_mx8: MXFP8Tensor.
    row_per_token / row_four_six: activation options of the row copy (a
    per-token row copy needs NVFP4Tensor.empty(..., sdec_per_row=True)).
    gelu: the row / row_mx8 copies are of GELU(x) (tanh form, FP32)."""
    rd = row.desc() if row is not None else None
    cd = col.desc() if col is not None else None
    md = row_mx8.desc() if row_mx8 is not None else None
    if amax_ws is None:
        amax_ws = amax_workspace(x.device)
    a = QuantArgs(_ptr(x), x.shape[0], x.shape[1], x.stride(0),
                  C.pointer(rd) if rd else None, row_round, Rng(*row_rng),
                  C.pointer(cd) if cd else None, col_round, Rng(*col_rng),
                  int(col_rht), rht_signs,
                  C.pointer(md) if md else None, mx8_round, Rng(*mx8_rng),
                  int(tile2d), _ptr(amax_ws), int(row_per_token), int(row_four_six),
                  int(gelu))
    _check(lib.nvfp4_quantize(C.byref(a), _stream(stream)))


def nvfp4_quantize_noalloc(x, row=None, col=None, row_mx8=None, *, row_round=RTN, row_rng=(0, 0),
                           col_round=RTN, col_rng=(0, 0), col_rht=False, rht_signs=0,
                           mx8_round=RTN, mx8_rng=(0, 0), tile2d=False, row_per_token=False,
                           row_four_six=False, gelu=False, stream=None):
    """nvfp4_quantize without a workspace argument: the library's own per-GPU
    scratch holds the amax partials (nothing is allocated by the call)."""
    rd = row.desc() if row is not None else None
    cd = col.desc() if col is not None else None
    md = row_mx8.desc() if row_mx8 is not None else None
    a = QuantArgs(_ptr(x), x.shape[0], x.shape[1], x.stride(0),
                  C.pointer(rd) if rd else None, row_round, Rng(*row_rng),
                  C.pointer(cd) if cd else None, col_round, Rng(*col_rng),
                  int(col_rht), rht_signs,
                  C.pointer(md) if md else None, mx8_round, Rng(*mx8_rng),
                  int(tile2d), None, int(row_per_token), int(row_four_six), int(gelu))
    _check(lib.nvfp4_quantize_noalloc(C.byref(a), _stream(stream)))


def mxfp8_requantize_t(src, dst, round=SR, rng=(0, 0), stream=None):
    sd, dd = src.desc(), dst.desc()
    _check(lib.mxfp8_requantize_t(C.byref(sd), C.byref(dd), round, Rng(*rng), _stream(stream)))


def nvfp4_gemm(fmt, A, B, C_out, c_dtype, ldc=None, stream=None):
    ad, bd = A.desc(), B.desc()
    ldc = C_out.stride(0) if ldc is None else ldc
    _check(lib.nvfp4_gemm(fmt, C.byref(ad), C.byref(bd), _ptr(C_out), c_dtype, ldc,
                          _stream(stream)))


def grouped_nvfp4_gemm(A, row_index, group_offsets, G, max_rows, B, N, C_out, c_dtype, ldc=None,
                       stream=None):
    ad, bd = A.desc(), B.desc()
    ldc = C_out.stride(0) if ldc is None else ldc
    _check(lib.grouped_nvfp4_gemm(C.byref(ad), _ptr(row_index), _ptr(group_offsets), G, max_rows,
                                  C.byref(bd), N, _ptr(C_out), c_dtype, ldc, _stream(stream)))


def s2f6_quantize(x, out, rht=True, signs=0, stream=None):
    """Combine wire format encode of x (BF16 patterns [rows, cols]) into the
    S2F6Tensor out, with the 32-point RHT when rht."""
    d = out.desc()
    _check(lib.s2f6_quantize(_ptr(x), x.shape[0], x.shape[1], x.stride(0), int(rht), signs,
                             C.byref(d), _stream(stream)))


def s2f6_combine(inp, src_index, out, weights=None, rht=True, signs=0, out_dtype=OUT_BF16,
                 ldo=None, stream=None):
    """out[t] = inverse RHT of sum_j weights[t, j] * decode(inp row src_index[t, j]);
    src_index: int32 [tokens, k] device tensor, weights: float32 [tokens, k] or None."""
    d = inp.desc()
    T, K = src_index.shape
    ldo = out.stride(0) if ldo is None else ldo
    _check(lib.s2f6_combine(C.byref(d), _ptr(src_index), _ptr(weights), T, K, int(rht), signs,
                            _ptr(out), out_dtype, ldo, _stream(stream)))


def mxfp4_quantize(x, out, round=RTN, rng=(0, 0), stream=None):
    """MXFP4 copy of x (BF16 patterns [rows, cols]) into the MXFP4Tensor out."""
    d = out.desc()
    _check(lib.mxfp4_quantize(_ptr(x), x.shape[0], x.shape[1], x.stride(0), C.byref(d), round,
                              Rng(*rng), _stream(stream)))


def nvfp4_gemm_quant(A, B, s_enc, Y, gelu=False, amax=None, ws=None, stream=None):
    """Y (NVFP4Tensor, 1x16) = NVFP4 copy of (GELU of) the BF16 product A * B^T
    with the encode scale s_enc (a one-element float32 device tensor); amax
    (optional one-element float32 device tensor) receives max |y|."""
    ad, bd, yd = A.desc(), B.desc(), Y.desc()
    if gelu and ws is None:
        ws = amax_workspace(s_enc.device)
    _check(lib.nvfp4_gemm_quant(C.byref(ad), C.byref(bd), _ptr(s_enc), int(gelu), C.byref(yd),
                                _ptr(amax), _ptr(ws), _stream(stream)))


def grouped_nvfp4_gemm_quant(A, row_index, group_offsets, G, max_rows, B, N, s_enc, Y,
                             gelu=False, amax=None, ws=None, stream=None):
    ad, bd, yd = A.desc(), B.desc(), Y.desc()
    if gelu and ws is None:
        ws = amax_workspace(s_enc.device)
    _check(lib.grouped_nvfp4_gemm_quant(C.byref(ad), _ptr(row_index), _ptr(group_offsets), G,
                                        max_rows, C.byref(bd), N, _ptr(s_enc), int(gelu),
                                        C.byref(yd), _ptr(amax), _ptr(ws), _stream(stream)))


def nvfp4_gemm_s2f6(A, B, Y, rht=True, signs=0, stream=None):
    """Y (S2F6Tensor) = combine wire format encode of the BF16 product A * B^T."""
    ad, bd, yd = A.desc(), B.desc(), Y.desc()
    _check(lib.nvfp4_gemm_s2f6(C.byref(ad), C.byref(bd), int(rht), signs, C.byref(yd),
                               _stream(stream)))


def grouped_nvfp4_gemm_s2f6(A, row_index, group_offsets, G, max_rows, B, N, Y, rht=True, signs=0,
                            stream=None):
    """The grouped GEMM with the combine wire format encode of its BF16 output."""
    ad, bd, yd = A.desc(), B.desc(), Y.desc()
    _check(lib.grouped_nvfp4_gemm_s2f6(C.byref(ad), _ptr(row_index), _ptr(group_offsets), G,
                                       max_rows, C.byref(bd), N, int(rht), signs, C.byref(yd),
                                       _stream(stream)))

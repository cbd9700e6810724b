"""Python face of the C oracle (TEST INFRASTRUCTURE; see oracle/nvfp4_oracle.c).

Thin ctypes marshalling over liboracle.so plus plain numpy bookkeeping
(allocation, reshapes).  The method's arithmetic happens in the C file, with
three small exceptions done here in numpy: the maximum of |GELU(x)| taken by
gelu_quantize (a max, so exact), the FP32 reciprocal 1 / s_enc that
nvfp4_encode_f32 stores as the decode scale (one IEEE division), and the
error norms (rel_fro) used by the checks.

Parity note: every function below is pinned by a CPU test in tests/ that
checks it against what the pages or the mathematics fix (worked examples,
closed forms, brute force, invariants).
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

RTN, SR = 0, 1
E2M1, E4M3 = 0, 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = C.CDLL(path)
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
        u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
        u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
        i64, u64, u32, i32, f32 = C.c_int64, C.c_uint64, C.c_uint32, C.c_int, C.c_float
        sig = {
            "orc_e2m1_value": (C.c_double, [u32]),
            "orc_e4m3_value": (C.c_double, [u32]),
            "orc_e8m0_value": (C.c_double, [u32]),
            "orc_round": (f32, [f32, i32, i32, f32]),
            "orc_e2m1_code": (u32, [f32]),
            "orc_e4m3_code": (u32, [f32]),
            "orc_philox4x32_10": (None, [u32p, u32p, u32p]),
            "orc_sr_uniform": (f32, [u64, u32, u64]),
            "orc_tensor_s_enc": (f32, [f32]),
            "orc_block_scale_code": (u32, [f32, f32]),
            "orc_e8m0_k": (i32, [f32]),
            "orc_e8m0_k_for": (i32, [f32, C.c_double]),
            "orc_nvfp4_encode": (None, [f32p, i64, i64, i32, f32, i32, u64, u32, u8p, u8p]),
            "orc_nvfp4_quantize": (f32, [u16p, i64, i64, i64, i32, i32, i32, u32, i32, u64,
                                         u32, u8p, u8p]),
            "orc_nvfp4_dequant_f32": (None, [u8p, u8p, f32, i64, i64, i32, f32p]),
            "orc_nvfp4_dequant_f64": (None, [u8p, u8p, f32, i64, i64, i32, f64p]),
            "orc_mxfp8_encode": (None, [f32p, i64, i64, i32, u64, u32, u8p, u8p]),
            "orc_mxfp8_requantize_t": (None, [u8p, u8p, f32, i64, i64, i32, i32, u64, u32,
                                              u8p, u8p]),
            "orc_mxfp8_quantize": (None, [u16p, i64, i64, i64, i32, u64, u32, u8p, u8p]),
            "orc_mxfp8_dequant_f64": (None, [u8p, u8p, i64, i64, f64p]),
            "orc_gemm_f64": (None, [f64p, f64p, i64, i64, i64, f64p]),
            "orc_gemm_f64_sampled": (None, [f64p, f64p, i64, i64p, i64p, i64, f64p]),
            "orc_num_threads": (i32, []),
            "orc_round_n": (None, [f32p, C.c_void_p, i64, i32, i32, f32p]),
            "orc_e2m1_code_n": (None, [f32p, i64, u8p]),
            "orc_e4m3_code_n": (None, [f32p, i64, u8p]),
            "orc_sr_uniform_n": (None, [u64, u32, u64p, i64, f32p]),
            "orc_rht16_n": (None, [f32p, i64, u32]),
            "orc_e8m0_k_n": (None, [f32p, i64, i32p]),
            "orc_amax": (f32, [f32p, i64]),
            "orc_nvfp4_quantize_act": (None, [u16p, i64, i64, i64, i32, i32, i32, u8p, u8p,
                                              f32p]),
            "orc_exp_n": (None, [f32p, i64, f32p]),
            "orc_gelu_n": (None, [f32p, i64, f32p]),
            "orc_nvfp4_dequant_rows_f64": (None, [u8p, u8p, f32p, i64, i64, f64p]),
            "orc_rht32_n": (None, [f32p, i64, u32, i32]),
            "orc_s2f6_encode": (None, [f32p, i64, i64, i32, u32, i8p, u8p]),
            "orc_s2f6_quantize": (None, [u16p, i64, i64, i64, i32, u32, i8p, u8p]),
            "orc_s2f6_combine": (None, [i8p, u8p, i64, i32p, C.c_void_p, i64, i32, i32, u32,
                                        f32p]),
            "orc_s2f6_dequant_f64": (None, [i8p, u8p, i64, i64, f64p]),
            "orc_mxfp4_encode": (None, [f32p, i64, i64, i32, u64, u32, u8p, u8p]),
            "orc_mxfp4_quantize": (None, [u16p, i64, i64, i64, i32, u64, u32, u8p, u8p]),
            "orc_mxfp4_dequant_f64": (None, [u8p, u8p, i64, i64, f64p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().orc_num_threads()


# --------------------------------------------------------------------------
# scalar / element-wise formats
# --------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(byte)


def e8m0_value(byte: int) -> float:
    return lib().orc_e8m0_value(byte)


def round_to(v, fmt: int, mode: int = RTN, u=None) -> np.ndarray:
    """The single rounding function, element-wise over a float32 array."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty_like(v)
    uu = None
    if u is not None:
        uu = np.ascontiguousarray(np.broadcast_to(np.asarray(u, np.float32), v.shape))
    lib().orc_round_n(v.reshape(-1), None if uu is None else uu.ctypes.data_as(C.c_void_p),
                      v.size, fmt, mode, out.reshape(-1))
    return out


def e2m1_code(g) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty(g.shape, np.uint8)
    lib().orc_e2m1_code_n(g.reshape(-1), g.size, out.reshape(-1))
    return out


def e4m3_code(g) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty(g.shape, np.uint8)
    lib().orc_e4m3_code_n(g.reshape(-1), g.size, out.reshape(-1))
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(c, k, out)
    return out


def sr_uniform(seed: int, stream: int, idx) -> np.ndarray:
    idx = np.ascontiguousarray(idx, np.uint64)
    out = np.empty(idx.shape, np.float32)
    lib().orc_sr_uniform_n(seed, stream, idx.reshape(-1), idx.size, out.reshape(-1))
    return out


def rht16(y, signs: int) -> np.ndarray:
    """RHT of each consecutive 16-chunk of a float32 array (last dim % 16 == 0)."""
    y = np.array(y, dtype=np.float32, copy=True, order="C")
    lib().orc_rht16_n(y.reshape(-1), y.size // 16, signs)
    return y


def tensor_s_enc(amax: float) -> np.float32:
    return np.float32(lib().orc_tensor_s_enc(amax))


def block_scale_code(amax_b: float, s_enc: float) -> int:
    return lib().orc_block_scale_code(amax_b, s_enc)


def e8m0_k_for(amax: float, elem_max: float) -> int:
    return lib().orc_e8m0_k_for(amax, elem_max)


def e8m0_k(amax) -> np.ndarray:
    a = np.ascontiguousarray(amax, np.float32)
    out = np.empty(a.shape, np.int32)
    lib().orc_e8m0_k_n(a.reshape(-1), a.size, out.reshape(-1))
    return out


# --------------------------------------------------------------------------
# tensor-level quantizers
# --------------------------------------------------------------------------

class NVFP4:
    """One NVFP4 copy: codes [r][c/2], scales, FP32 decode scale s_dec."""

    def __init__(self, codes, scales, s_dec, rows, cols, tile2d):
        self.codes, self.scales = codes, scales
        self.s_dec = np.float32(s_dec)
        self.rows, self.cols, self.tile2d = rows, cols, tile2d

    def dequant_f64(self) -> np.ndarray:
        out = np.empty((self.rows, self.cols), np.float64)
        lib().orc_nvfp4_dequant_f64(self.codes, self.scales, self.s_dec, self.rows,
                                    self.cols, int(self.tile2d), out)
        return out

    def dequant_f32(self) -> np.ndarray:
        out = np.empty((self.rows, self.cols), np.float32)
        lib().orc_nvfp4_dequant_f32(self.codes, self.scales, self.s_dec, self.rows,
                                    self.cols, int(self.tile2d), out)
        return out


class NVFP4Rows(NVFP4):
    """A 1x16 NVFP4 copy whose rows carry their own decode scale s_dec[i]
    (per-token outer scale)."""

    def __init__(self, codes, scales, s_dec_rows, rows, cols):
        super().__init__(codes, scales, 0.0, rows, cols, False)
        self.s_dec = np.ascontiguousarray(s_dec_rows, np.float32)

    def dequant_f64(self) -> np.ndarray:
        out = np.empty((self.rows, self.cols), np.float64)
        lib().orc_nvfp4_dequant_rows_f64(self.codes, self.scales, self.s_dec, self.rows,
                                         self.cols, out)
        return out

    def dequant_f32(self) -> np.ndarray:
        raise NotImplementedError("per-row copies dequantize in FP64 only")


class MXFP8:
    """One MXFP8 copy: E4M3 codes [r][c], E8M0 scales [r][c/32]."""

    def __init__(self, codes, scales, rows, cols):
        self.codes, self.scales, self.rows, self.cols = codes, scales, rows, cols

    def dequant_f64(self) -> np.ndarray:
        out = np.empty((self.rows, self.cols), np.float64)
        lib().orc_mxfp8_dequant_f64(self.codes, self.scales, self.rows, self.cols, out)
        return out


def _scales_shape(r, c, tile2d):
    return (r // 16, c // 16) if tile2d else (r, c // 16)


def nvfp4_quantize(x_bf16: np.ndarray, transpose=False, tile2d=False, rht=False,
                   signs=0, mode=RTN, seed=0, stream=0) -> NVFP4:
    """One NVFP4 copy of a BF16 matrix (given as uint16 bit patterns).

    transpose=True quantizes x^T (the column-wise copy); rht=True applies the
    16-point RHT to the 16-chunks of that copy's rows first."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    R, Cc = x.shape
    r, c = (Cc, R) if transpose else (R, Cc)
    codes = np.zeros((r, c // 2), np.uint8)
    scales = np.zeros(_scales_shape(r, c, tile2d), np.uint8)
    s_dec = lib().orc_nvfp4_quantize(x, R, Cc, Cc, int(transpose), int(tile2d), int(rht),
                                     signs, mode, seed, stream, codes, scales)
    return NVFP4(codes, scales, s_dec, r, c, tile2d)


def exp_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty_like(x)
    lib().orc_exp_n(x.reshape(-1), x.size, out.reshape(-1))
    return out


def gelu_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty_like(x)
    lib().orc_gelu_n(x.reshape(-1), x.size, out.reshape(-1))
    return out


def nvfp4_quantize_act(x_bf16: np.ndarray, per_token=True, four_six=True, gelu=False):
    """Row-wise 1x16 NVFP4 copy of an activation matrix, round to nearest,
    with a per-token outer scale (per_token) and / or Four Over Six block
    scales (four_six), optionally of GELU(x) (gelu).  Returns NVFP4Rows when
    per_token, else NVFP4."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    R, Cc = x.shape
    codes = np.zeros((R, Cc // 2), np.uint8)
    scales = np.zeros((R, Cc // 16), np.uint8)
    s_dec = np.zeros(R if per_token else 1, np.float32)
    lib().orc_nvfp4_quantize_act(x, R, Cc, Cc, int(per_token), int(four_six), int(gelu), codes,
                                 scales, s_dec)
    if per_token:
        return NVFP4Rows(codes, scales, s_dec, R, Cc)
    return NVFP4(codes, scales, s_dec[0], R, Cc, False)


def bf16_to_f32(x_bf16: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) to FP32 values (exact)."""
    return (np.asarray(x_bf16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def gelu_quantize(x_bf16: np.ndarray, mode=RTN, seed=0, stream=0, mx_mode=None, mx_seed=0,
                  mx_stream=0):
    """GELU(x) in FP32, then its row-wise 1x16 NVFP4 copy with the per-tensor
    outer scale of GELU(x), and (mx_mode not None) its row-wise MXFP8 copy
    (4bit.vizuara.ai, section 13: the activation is applied in the quantizer
    and its FP32 result is quantized).  Returns (NVFP4, MXFP8 or None)."""
    g = gelu_f32(bf16_to_f32(x_bf16))
    q = nvfp4_encode_f32(g, tensor_s_enc(float(np.abs(g).max())), mode=mode, seed=seed,
                         stream=stream)
    m = None if mx_mode is None else mxfp8_encode_f32(g, mx_mode, mx_seed, mx_stream)
    return q, m


def nvfp4_encode_f32(x: np.ndarray, s_enc: float, tile2d=False, mode=RTN, seed=0,
                     stream=0) -> NVFP4:
    """Encode an FP32 matrix with a given tensor encode scale."""
    x = np.ascontiguousarray(x, np.float32)
    r, c = x.shape
    codes = np.zeros((r, c // 2), np.uint8)
    scales = np.zeros(_scales_shape(r, c, tile2d), np.uint8)
    lib().orc_nvfp4_encode(x, r, c, int(tile2d), np.float32(s_enc), mode, seed, stream,
                           codes, scales)
    return NVFP4(codes, scales, np.float32(1.0) / np.float32(s_enc), r, c, tile2d)


def mxfp8_quantize(x_bf16: np.ndarray, mode=SR, seed=0, stream=0) -> MXFP8:
    x = np.ascontiguousarray(x_bf16, np.uint16)
    R, Cc = x.shape
    codes = np.zeros((R, Cc), np.uint8)
    scales = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_mxfp8_quantize(x, R, Cc, Cc, mode, seed, stream, codes, scales)
    return MXFP8(codes, scales, R, Cc)


def mxfp8_encode_f32(x: np.ndarray, mode=RTN, seed=0, stream=0) -> MXFP8:
    x = np.ascontiguousarray(x, np.float32)
    R, Cc = x.shape
    codes = np.zeros((R, Cc), np.uint8)
    scales = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_mxfp8_encode(x, R, Cc, mode, seed, stream, codes, scales)
    return MXFP8(codes, scales, R, Cc)


def mxfp8_requantize_t(q: NVFP4, mode=SR, seed=0, stream=0) -> MXFP8:
    R, Cc = q.rows, q.cols
    codes = np.zeros((Cc, R), np.uint8)
    scales = np.zeros((Cc, R // 32), np.uint8)
    lib().orc_mxfp8_requantize_t(np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales),
                                 q.s_dec, R, Cc, int(q.tile2d), mode, seed, stream, codes,
                                 scales)
    return MXFP8(codes, scales, Cc, R)


# --------------------------------------------------------------------------
# Combine wire format (32-point RHT + block-scaled S2F6) and MXFP4
# --------------------------------------------------------------------------

def rht32(y, signs: int, inverse=False) -> np.ndarray:
    """32-point RHT of each consecutive 32-chunk of y (FP32), or its inverse."""
    y = np.array(y, np.float32, copy=True).reshape(-1)
    assert y.size % 32 == 0
    lib().orc_rht32_n(y, y.size // 32, signs, int(inverse))
    return y


class S2F6:
    """One S2F6 copy: int8 codes [r][c], E8M0 scales [r][c/32]; value of a
    code = code / 64 * 2^(scale - 127)."""

    def __init__(self, codes, scales, rows, cols):
        self.codes, self.scales, self.rows, self.cols = codes, scales, rows, cols

    def dequant_f64(self) -> np.ndarray:
        out = np.empty((self.rows, self.cols), np.float64)
        lib().orc_s2f6_dequant_f64(self.codes, self.scales, self.rows, self.cols, out)
        return out


def s2f6_quantize(x_bf16: np.ndarray, rht=True, signs=0) -> S2F6:
    x = np.ascontiguousarray(x_bf16, np.uint16)
    R, Cc = x.shape
    codes = np.zeros((R, Cc), np.int8)
    scales = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_s2f6_quantize(x, R, Cc, Cc, int(rht), signs, codes, scales)
    return S2F6(codes, scales, R, Cc)


def s2f6_encode_f32(x: np.ndarray, rht=True, signs=0) -> S2F6:
    x = np.ascontiguousarray(x, np.float32)
    R, Cc = x.shape
    codes = np.zeros((R, Cc), np.int8)
    scales = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_s2f6_encode(x, R, Cc, int(rht), signs, codes, scales)
    return S2F6(codes, scales, R, Cc)


def s2f6_combine(q: S2F6, src, weights=None, rht=True, signs=0) -> np.ndarray:
    """out[t] = inverse RHT of sum_j weights[t, j] * dequant(q row src[t, j])
    (FP32; negative indices skipped; weights None = 1)."""
    src = np.ascontiguousarray(src, np.int32)
    T, K = src.shape
    out = np.empty((T, q.cols), np.float32)
    w = None
    if weights is not None:
        w = np.ascontiguousarray(weights, np.float32)
        assert w.shape == (T, K)
    lib().orc_s2f6_combine(np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales), q.cols,
                           src, None if w is None else w.ctypes.data, T, K, int(rht), signs,
                           out)
    return out


class MXFP4:
    """One MXFP4 copy: E2M1 codes [r][c/2] (even column in the low nibble),
    E8M0 scales [r][c/32]."""

    def __init__(self, codes, scales, rows, cols):
        self.codes, self.scales, self.rows, self.cols = codes, scales, rows, cols

    def dequant_f64(self) -> np.ndarray:
        out = np.empty((self.rows, self.cols), np.float64)
        lib().orc_mxfp4_dequant_f64(self.codes, self.scales, self.rows, self.cols, out)
        return out


def mxfp4_quantize(x_bf16: np.ndarray, mode=RTN, seed=0, stream=0) -> MXFP4:
    x = np.ascontiguousarray(x_bf16, np.uint16)
    R, Cc = x.shape
    codes = np.zeros((R, Cc // 2), np.uint8)
    scales = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_mxfp4_quantize(x, R, Cc, Cc, mode, seed, stream, codes, scales)
    return MXFP4(codes, scales, R, Cc)


def mxfp4_encode_f32(x: np.ndarray, mode=RTN, seed=0, stream=0) -> MXFP4:
    x = np.ascontiguousarray(x, np.float32)
    R, Cc = x.shape
    codes = np.zeros((R, Cc // 2), np.uint8)
    scales = np.zeros((R, Cc // 32), np.uint8)
    lib().orc_mxfp4_encode(x, R, Cc, mode, seed, stream, codes, scales)
    return MXFP4(codes, scales, R, Cc)


# --------------------------------------------------------------------------
# GEMM references (FP64 accumulation over the dequantized operands)
# --------------------------------------------------------------------------

def gemm_f64(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Y = A B^T, plain FP64 loop in k order."""
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    M, K = A.shape
    N = B.shape[0]
    Y = np.empty((M, N), np.float64)
    lib().orc_gemm_f64(A, B, M, N, K, Y)
    return Y


def gemm_f64_sampled(A: np.ndarray, B: np.ndarray, rows, cols) -> np.ndarray:
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    Y = np.empty(rows.shape, np.float64)
    lib().orc_gemm_f64_sampled(A, B, A.shape[1], rows, cols, rows.size, Y)
    return Y


def rel_fro(y, ref) -> float:
    """Relative Frobenius error ||y - ref|| / ||ref||."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / (den if den > 0 else 1.0))


def bf16_rne(y: np.ndarray) -> np.ndarray:
    """FP64 -> FP32 -> BF16 (round to nearest even), returned as float64 values."""
    f = np.asarray(y, np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


__all__ = [n for n in dir() if not n.startswith("_")]

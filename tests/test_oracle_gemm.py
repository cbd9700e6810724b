"""Pins of the oracle's GEMM references."""
import numpy as np

import oracle as O
from workloads import synth


def _random_nvfp4(R, C, seed, tile2d=False, s_dec=0.75):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    shape = (R // 16, C // 16) if tile2d else (R, C // 16)
    scales = rng.integers(1, 0x7F, size=shape, dtype=np.uint8)
    return O.NVFP4(codes, scales, np.float32(s_dec), R, C, tile2d)


def test_integer_special_case_exact():
    # All block scales 1.0 (0x38) and s_dec = 1: every product is a multiple of
    # 1/4 and the sums are exact, so the reference equals integer arithmetic.
    rng = np.random.default_rng(1)
    M, N, K = 40, 24, 256
    a = O.NVFP4(rng.integers(0, 256, (M, K // 2), dtype=np.uint8),
                np.full((M, K // 16), 0x38, np.uint8), 1.0, M, K, False)
    b = O.NVFP4(rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
                np.full((N, K // 16), 0x38, np.uint8), 1.0, N, K, False)
    dec2 = np.array([int(round(2 * O.e2m1_value(c))) for c in range(16)], np.int64)

    def ints(q):
        v = np.empty((q.rows, q.cols), np.int64)
        v[:, 0::2], v[:, 1::2] = dec2[q.codes & 0xF], dec2[q.codes >> 4]
        return v
    Y = O.gemm_f64(a.dequant_f64(), b.dequant_f64())
    assert np.array_equal(Y * 4, (ints(a) @ ints(b).T).astype(np.float64))


def test_block_scaled_form():
    # Y = sum_b s_a,b s_b,b sum_{k in b} a_k b_k, then the two tensor decode
    # scales: the block-scaled dot product written out from codes and scales.
    M, N, K = 16, 32, 64
    a = _random_nvfp4(M, K, 2, s_dec=0.5)
    b = _random_nvfp4(N, K, 3, tile2d=True, s_dec=0.25)
    dec = np.array([O.e2m1_value(c) for c in range(16)])
    e4 = np.array([O.e4m3_value(x) for x in range(256)])

    def vals(q):
        v = np.empty((q.rows, q.cols))
        v[:, 0::2], v[:, 1::2] = dec[q.codes & 0xF], dec[q.codes >> 4]
        return v
    av, bv = vals(a), vals(b)
    Y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            for kb in range(K // 16):
                sa = e4[a.scales[m, kb]]
                sb = e4[b.scales[n // 16, kb]]
                Y[m, n] += sa * sb * np.dot(av[m, kb * 16:kb * 16 + 16],
                                            bv[n, kb * 16:kb * 16 + 16])
    Y *= float(a.s_dec) * float(b.s_dec)
    got = O.gemm_f64(a.dequant_f64(), b.dequant_f64())
    assert np.allclose(got, Y, rtol=1e-12, atol=1e-12 * np.abs(Y).max())


def test_gemm_matches_library_matmul():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((33, 47))
    B = rng.standard_normal((29, 47))
    assert np.allclose(O.gemm_f64(A, B), A @ B.T, rtol=1e-12, atol=1e-12)
    rows = rng.integers(0, 33, 50)
    cols = rng.integers(0, 29, 50)
    assert np.allclose(O.gemm_f64_sampled(A, B, rows, cols), (A @ B.T)[rows, cols],
                       rtol=1e-12, atol=1e-12)


def test_single_block_k16():
    a = _random_nvfp4(1, 16, 5, s_dec=2.0)
    b = _random_nvfp4(1, 16, 6, s_dec=0.5)
    av, bv = a.dequant_f64()[0], b.dequant_f64()[0]
    assert O.gemm_f64(a.dequant_f64(), b.dequant_f64())[0, 0] == float(np.dot(av, bv))


def test_mxfp8_dequant_definition():
    m = O.mxfp8_quantize(synth.normal(8, 64, 7, 1.0), mode=O.RTN)
    ref = np.array([[O.e4m3_value(int(c)) for c in row] for row in m.codes])
    ref *= np.repeat(2.0 ** (m.scales.astype(np.float64) - 127), 32, axis=1)
    assert np.array_equal(ref, m.dequant_f64())


def test_bf16_reference_rounding():
    y = np.array([1.0, 1.00390625, 1.005859375, -3.14159, 65504.0])
    r = O.bf16_rne(y)
    assert r[0] == 1.0 and r[1] == 1.0            # tie -> even
    assert r[2] == 1.0078125
    assert abs(r[3] + 3.140625) < 1e-12

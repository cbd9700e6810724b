"""Pins of the oracle's tensor-level quantizers (NVFP4 and MXFP8)."""
import numpy as np

import oracle as O
from golden_data import golden
from workloads import synth


def _f64(x_bf16):
    return synth.bf16_to_f32(x_bf16).astype(np.float64)


def test_gaussian_errors_match_pages():
    g = golden("gaussian_errors")
    x = synth.normal(1024, 1024, 11, 1.0)
    xf = _f64(x)
    assert abs(O.rel_fro(O.nvfp4_quantize(x).dequant_f64(), xf) - g["nvfp4_rtn"]) < g["tol"]
    m = O.mxfp8_quantize(x, mode=O.RTN)
    assert abs(O.rel_fro(m.dequant_f64(), xf) - g["mxfp8_rtn"]) < g["tol"]
    m = O.mxfp8_quantize(x, mode=O.SR, seed=5)
    assert abs(O.rel_fro(m.dequant_f64(), xf) - g["mxfp8_sr"]) < g["tol"]


def test_sr_noise_averages_away():
    # The mean of n stochastic draws approaches the input like pure noise
    # (error / sqrt(n)); round-to-nearest keeps a fixed error.
    x = synth.normal(128, 256, 12, 1.0)
    xf = _f64(x)
    one = O.nvfp4_quantize(x, mode=O.SR, seed=1).dequant_f64()
    e1 = O.rel_fro(one, xf)
    acc = np.zeros_like(xf)
    n = 16
    for i in range(n):
        acc += O.nvfp4_quantize(x, mode=O.SR, seed=100 + i).dequant_f64()
    e16 = O.rel_fro(acc / n, xf)
    assert 3.3 < e1 / e16 < 4.7
    assert e16 < O.rel_fro(O.nvfp4_quantize(x).dequant_f64(), xf) / 2


def test_tile2d_copies_are_transposes():
    w = synth.normal(96, 160, 13, 0.02)
    row = O.nvfp4_quantize(w, tile2d=True)
    col = O.nvfp4_quantize(w, tile2d=True, transpose=True)
    assert row.s_dec == col.s_dec
    assert np.array_equal(row.scales.T, col.scales)
    assert np.array_equal(row.dequant_f64().T, col.dequant_f64())
    # and a 16x16 scale is the max over its tile
    wf = np.abs(synth.bf16_to_f32(w))
    s_enc = O.tensor_s_enc(wf.max())
    tmax = wf.reshape(6, 16, 10, 16).max(axis=(1, 3))
    ref = np.array([[O.block_scale_code(a, s_enc) for a in r] for r in tmax])
    assert np.array_equal(row.scales, ref)


def test_one_by_sixteen_scales_are_block_maxima():
    x = synth.normal_with_outliers(32, 64, 14)
    q = O.nvfp4_quantize(x)
    xf = np.abs(synth.bf16_to_f32(x))
    s_enc = O.tensor_s_enc(xf.max())
    bmax = xf.reshape(32, 4, 16).max(axis=2)
    ref = np.array([[O.block_scale_code(a, s_enc) for a in r] for r in bmax])
    assert np.array_equal(q.scales, ref)
    # element 2j in the low nibble: decode by hand and compare with dequant
    dec = np.array([O.e2m1_value(c) for c in range(16)])
    lo, hi = q.codes & 0xF, q.codes >> 4
    vals = np.empty((32, 64))
    vals[:, 0::2], vals[:, 1::2] = dec[lo], dec[hi]
    sc = np.array([O.e4m3_value(int(b)) for b in q.scales.reshape(-1)]).reshape(32, 4)
    ref_deq = vals * np.repeat(sc, 16, axis=1) * np.float64(q.s_dec)
    assert np.array_equal(ref_deq, q.dequant_f64())


def test_column_copy_is_copy_of_transpose():
    x = synth.student_t(48, 80, 15)
    col = O.nvfp4_quantize(x, transpose=True, mode=O.SR, seed=3, stream=1)
    ref = O.nvfp4_quantize(np.ascontiguousarray(x.T), mode=O.SR, seed=3, stream=1)
    assert np.array_equal(col.codes, ref.codes) and np.array_equal(col.scales, ref.scales)


def test_rht_column_copy_uses_transformed_amax():
    x = synth.normal_with_outliers(64, 48, 16)
    s = 0x3C5A
    q = O.nvfp4_quantize(x, transpose=True, rht=True, signs=s)
    xt = np.ascontiguousarray(synth.bf16_to_f32(x).T)
    y = O.rht16(xt, s)
    assert q.s_dec == np.float32(1.0) / O.tensor_s_enc(np.abs(y).max())
    ref = O.nvfp4_encode_f32(y, O.tensor_s_enc(np.abs(y).max()))
    assert np.array_equal(q.codes, ref.codes) and np.array_equal(q.scales, ref.scales)


def test_sr_reproducible_and_keyed():
    x = synth.student_t(64, 64, 17)
    a = O.nvfp4_quantize(x, mode=O.SR, seed=11, stream=0)
    b = O.nvfp4_quantize(x, mode=O.SR, seed=11, stream=0)
    c = O.nvfp4_quantize(x, mode=O.SR, seed=11, stream=1)
    assert np.array_equal(a.codes, b.codes)
    assert not np.array_equal(a.codes, c.codes)


def test_degenerate_tensors():
    z = np.zeros((16, 32), np.uint16)
    q = O.nvfp4_quantize(z)
    assert q.s_dec == 1.0 and np.all(q.codes == 0) and np.all(q.scales == 1)
    nz = np.full((16, 32), 0x8000, np.uint16)           # all -0.0
    q = O.nvfp4_quantize(nz)
    assert np.all(q.codes == 0x88)
    m = O.mxfp8_quantize(z)
    assert np.all(m.codes == 0) and np.all(m.scales == 0)
    # one non-zero element: it lands on +-6 with the largest scale
    one = np.zeros((16, 32), np.float32)
    one[3, 7] = -0.3
    q = O.nvfp4_quantize(synth.bf16_bits(one))
    assert q.scales[3, 0] == 0x7E and (q.codes[3, 3] >> 4) == 0xF


def test_mxfp8_scale_is_the_smallest_power():
    x = synth.laplace(64, 256, 18, 1e-3)
    m = O.mxfp8_quantize(x, mode=O.RTN)
    xf = np.abs(synth.bf16_to_f32(x)).astype(np.float64).reshape(64, 8, 32).max(axis=2)
    k = m.scales.astype(np.int64) - 127
    assert np.all(xf <= 448.0 * 2.0 ** k)
    assert np.all(xf > 448.0 * 2.0 ** (k - 1))


def _pow2_scaled_nvfp4(R, C, seed):
    """An NVFP4 tensor whose scales are powers of two (E4M3 mantissa 0):
    every dequantized value then has at most two significant bits."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    e = rng.integers(5, 9, size=(R, C // 16))          # exponent field 5..8
    scales = (e << 3).astype(np.uint8)
    return O.NVFP4(codes, scales, np.float32(0.125), R, C, False)


def test_requantize_exact_when_representable():
    q = _pow2_scaled_nvfp4(64, 96, 19)
    for mode in (O.RTN, O.SR):
        m = O.mxfp8_requantize_t(q, mode=mode, seed=4, stream=2)
        assert m.rows == 96 and m.cols == 64
        assert np.array_equal(m.dequant_f64(), q.dequant_f64().T)


def test_requantize_sr_is_unbiased():
    w = synth.normal(64, 64, 20, 0.02)
    q = O.nvfp4_quantize(w, tile2d=True)
    ref = q.dequant_f32().astype(np.float64).T
    e1 = O.rel_fro(O.mxfp8_requantize_t(q, seed=1).dequant_f64(), ref)
    acc = np.zeros_like(ref)
    n = 16
    for i in range(n):
        acc += O.mxfp8_requantize_t(q, seed=50 + i).dequant_f64()
    e16 = O.rel_fro(acc / n, ref)
    assert 3.0 < e1 / e16 < 5.0
    rtn = O.rel_fro(O.mxfp8_requantize_t(q, mode=O.RTN).dequant_f64(), ref)
    assert e16 < rtn

"""Pins of the activation quantizer variant: per-token outer scale and Four
Over Six (4bit.vizuara.ai, section 11; End-to-End 4-Bit Training, recipe
details).  Expected values are derived by hand from the definitions."""
import numpy as np

import oracle as O
from workloads import synth


def _bf(v):
    return synth.bf16_bits(np.asarray(v, np.float32))


def _row_with_tensor_scale_one(block):
    # a second block holding 2688 makes the tensor amax 2688, so s_enc = 1
    row = np.zeros((1, 32), np.float32)
    row[0, :16] = block
    row[0, 16] = 2688.0
    return row


def test_four_six_worked_block():
    """Block [6, 5 x 15] with s_enc = 1.  Top-6 scale: 6/6 = 1 (E4M3 0x38);
    6 -> 6 (code 7), 5 is the midpoint of 4 and 6 -> 4 (even code 6): squared
    error 15.  Top-4 scale: 6/4 = 1.5 (0x3C, exact); 6/1.5 = 4 (code 6),
    5/1.5 = 3.33 -> 3 (code 5), dequantized 4.5: squared error 15 * 0.25 =
    3.75 < 15, so Four Over Six keeps the top-4 encoding."""
    x = _bf(_row_with_tensor_scale_one([6.0] + [5.0] * 15))
    q = O.nvfp4_quantize_act(x, per_token=False, four_six=True)
    assert q.s_dec == 1.0
    assert q.scales[0, 0] == 0x3C
    assert q.codes[0, 0] == 0x56 and np.all(q.codes[0, 1:8] == 0x55)
    # the 2688 block: 2688/6 = 448 (0x7E) either way (the top-4 scale 672
    # saturates to 448): identical errors, the top-6 encoding is kept
    assert q.scales[0, 1] == 0x7E and q.codes[0, 8] == 0x07
    plain = O.nvfp4_quantize_act(x, per_token=False, four_six=False)
    assert plain.scales[0, 0] == 0x38
    assert plain.codes[0, 0] == 0x67 and np.all(plain.codes[0, 1:8] == 0x66)


def test_four_six_exact_top4_block():
    """Block [4, 2, 1, 0.5, 0 ...] with s_enc = 1: the top-4 scale 4/4 = 1 is
    exact and every value is on the grid (error 0); the top-6 scale 4/6 rounds
    to 0.6875 and leaves errors, so the top-4 encoding wins."""
    x = _bf(_row_with_tensor_scale_one([4.0, 2.0, 1.0, 0.5] + [0.0] * 12))
    q = O.nvfp4_quantize_act(x, per_token=False, four_six=True)
    assert q.scales[0, 0] == 0x38                     # 1.0
    assert list(q.codes[0, :2]) == [0x46, 0x12]       # 4, 2 | 1, 0.5
    plain = O.nvfp4_quantize_act(x, per_token=False, four_six=False)
    assert O.e4m3_value(int(plain.scales[0, 0])) == 0.6875


def test_per_token_scale_invariance_and_independence():
    """With a per-token outer scale, multiplying a row by 2^-20 changes only
    its decode scale, and a row's codes do not depend on the other rows."""
    a = synth.normal_with_outliers(4, 256, 31)
    af = (a.astype(np.uint32) << 16).view(np.float32)
    scaled = af.copy()
    scaled[1] = af[1] * np.float32(2.0 ** -20)
    q = O.nvfp4_quantize_act(_bf(af), per_token=True, four_six=True)
    qs = O.nvfp4_quantize_act(_bf(scaled), per_token=True, four_six=True)
    assert np.array_equal(q.codes, qs.codes) and np.array_equal(q.scales, qs.scales)
    assert qs.s_dec[1] == q.s_dec[1] * np.float32(2.0 ** -20)
    other = af.copy()
    other[2:] *= np.float32(1000.0)
    qo = O.nvfp4_quantize_act(_bf(other), per_token=True, four_six=True)
    assert np.array_equal(qo.codes[:2], q.codes[:2]) and np.array_equal(qo.s_dec[:2], q.s_dec[:2])
    # the per-tensor copy of the same matrix does depend on the other rows
    pt = O.nvfp4_quantize_act(_bf(other), per_token=False, four_six=True)
    assert not np.array_equal(pt.codes[:2], q.codes[:2])


def test_per_token_equals_tensor_scale_on_one_row():
    """On a single row the per-token and the per-tensor scales coincide, so
    the two paths give the same bytes (the tensor path is pinned elsewhere)."""
    x = synth.normal_with_outliers(1, 1024, 41)
    for fs in (False, True):
        a = O.nvfp4_quantize_act(x, per_token=True, four_six=fs)
        b = O.nvfp4_quantize_act(x, per_token=False, four_six=fs)
        assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
        assert a.s_dec[0] == b.s_dec
    # and without 4/6 the per-tensor path is the standard quantizer
    std = O.nvfp4_quantize(x)
    b = O.nvfp4_quantize_act(x, per_token=False, four_six=False)
    assert np.array_equal(std.codes, b.codes) and np.array_equal(std.scales, b.scales)


def test_four_six_lowers_gaussian_error():
    """On Gaussian activations Four Over Six lowers the relative error of the
    1x16 copy (the pages report 9.3% -> 8.9% on real activations); it can
    never raise a block's error."""
    x = synth.normal(512, 4096, 51, 1.0)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    e6 = O.rel_fro(O.nvfp4_quantize_act(x, True, False).dequant_f64(), xf)
    e46 = O.rel_fro(O.nvfp4_quantize_act(x, True, True).dequant_f64(), xf)
    assert 0.05 < e46 < e6 < 0.15
    assert e46 < 0.99 * e6
    # block by block the kept encoding is never worse than the top-6 one
    q6 = O.nvfp4_quantize_act(x, True, False).dequant_f64()
    q46 = O.nvfp4_quantize_act(x, True, True).dequant_f64()
    b6 = ((q6 - xf) ** 2).reshape(-1, 16).sum(1)
    b46 = ((q46 - xf) ** 2).reshape(-1, 16).sum(1)
    assert np.all(b46 <= b6 * (1 + 1e-6) + 1e-30)

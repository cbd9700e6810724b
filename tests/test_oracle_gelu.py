"""Pins of the oracle's GELU and of the fused GELU + quantize reading
(4bit.vizuara.ai, section 13: the activation is applied inside the quantizer
and its FP32 output is quantized).  GELU is the tanh form of Hendrycks and
Gimpel, "Gaussian Error Linear Units", with exp by Cody-Waite reduction and a
Taylor polynomial; the pins hold it to the mathematics, not to itself."""
import math

import numpy as np
import pytest
from scipy.special import erf

import oracle as O
from workloads import synth


def _ulps(got, ref64):
    ref32 = ref64.astype(np.float32)
    return np.abs(got.astype(np.float64) - ref64) / np.spacing(np.abs(ref32)).astype(np.float64)


def test_exp_within_two_ulp_of_libm():
    v = np.linspace(-86.5, 88.0, 400001).astype(np.float32)
    assert _ulps(O.exp_f32(v), np.exp(v.astype(np.float64))).max() < 1.5
    small = np.float32([0.0, 1e-8, -1e-8, 0.5, -0.5, 1.0, math.log(2.0)])
    assert _ulps(O.exp_f32(small), np.exp(small.astype(np.float64))).max() < 1.0
    assert O.exp_f32(np.float32([0.0]))[0] == 1.0


def test_exp_cutoffs():
    """Inputs <= -87 give 0 (the result would be within a factor of 1.5 of the
    smallest normal number), inputs >= 88.5 give +inf."""
    out = O.exp_f32(np.float32([-87.0, -1000.0, 88.5, 1000.0]))
    assert out[0] == 0.0 and out[1] == 0.0
    assert np.isinf(out[2]) and np.isinf(out[3])


def test_gelu_close_to_x_phi_x():
    """GELU(x) = x * Phi(x); the tanh form is within 4.8e-4 of it everywhere
    (its largest deviation is about 4.73e-4, near |x| = 2).  A wrong
    coefficient (0.8 for sqrt(2/pi), a cubic term off by 1%) or 1 - tanh for
    1 + tanh exceeds the bound."""
    x = np.linspace(-12.0, 12.0, 240001).astype(np.float32)
    xd = x.astype(np.float64)
    exact = 0.5 * xd * (1.0 + erf(xd / math.sqrt(2.0)))
    g = O.gelu_f32(x).astype(np.float64)
    dev = np.abs(g - exact)
    assert dev.max() < 4.8e-4
    assert dev.max() > 4.6e-4        # the approximation, not the exact function
    assert np.argmax(dev) != 0


def test_gelu_matches_fp64_tanh_form_on_every_bf16():
    """The oracle's FP32 GELU against the same tanh form evaluated in FP64
    with libm's tanh, on every finite BF16 input: within 2 x (ulp of the
    result + 2^-24 |x|) (the second term covers the cancellation in
    1 + tanh for large negative x; the largest ratio seen is 1.42).  A
    cubic coefficient off in its fourth digit (0.04472) is 26 times the
    unit away, a wrong sqrt(2/pi) or a dropped half further still."""
    b = np.arange(65536, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]
    x = (b << 16).view(np.float32)
    xd = x.astype(np.float64)
    a = math.sqrt(2.0 / math.pi) * (xd + 0.044715 * xd ** 3)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = 0.5 * xd * (1.0 + np.tanh(a))
    ok = np.isfinite(ref)
    g = O.gelu_f32(x).astype(np.float64)
    unit = np.spacing(np.abs(ref[ok]).astype(np.float32)).astype(np.float64) + \
        2.0 ** -24 * np.abs(xd[ok])
    ratio = np.abs(g[ok] - ref[ok]) / unit
    assert ratio.max() <= 2.0, (ratio.max(), xd[ok][np.argmax(ratio)])


def test_gelu_special_values():
    x = np.float32([0.0, 10.0, 37.5, 1e4, -6.0, -10.0, -1e4])
    g = O.gelu_f32(x)
    assert g[0] == 0.0
    # tanh saturates to 1 in FP32 for x >= 10: GELU(x) = x
    assert np.array_equal(g[1:4], x[1:4])
    # and to -1 for x <= -6: GELU(x) = -0
    assert np.all(g[4:] == 0.0)
    # the minimum of GELU: about -0.170 near x = -0.752
    t = np.linspace(-3, 0, 30001).astype(np.float32)
    gt = O.gelu_f32(t)
    i = int(np.argmin(gt))
    assert abs(float(t[i]) + 0.752) < 2e-3 and abs(float(gt[i]) + 0.1700) < 1e-3


def test_gelu_odd_part_is_identity():
    """0.5x(1 + tanh a(x)) - 0.5(-x)(1 + tanh a(-x)) = x for any odd a: a
    dropped or doubled 0.5 fails, up to FP32 rounding of the two terms."""
    x = np.linspace(-8.0, 8.0, 16001).astype(np.float32)
    d = O.gelu_f32(x).astype(np.float64) - O.gelu_f32(-x).astype(np.float64)
    assert np.abs(d - x.astype(np.float64)).max() < 4.0 * np.spacing(np.float32(8.0))


def test_gelu_quantize_reduces_to_plain_quantizer():
    """Where GELU is exact (x >= 10: GELU(x) = x; x <= -10: GELU(x) = -0) the
    fused copies equal the plain quantizer's copies of GELU(x)."""
    rng = np.random.default_rng(5)
    x = rng.uniform(10.0, 300.0, (64, 96)).astype(np.float32)
    neg = rng.random((64, 96)) < 0.3
    x[neg] = -rng.uniform(10.0, 300.0, neg.sum())
    xb = synth.bf16_bits(x)
    gx = np.where(neg, -0.0, O.bf16_to_f32(xb)).astype(np.float32)   # GELU(x < 0) = -0
    gb = synth.bf16_bits(gx)
    for mode in (O.RTN, O.SR):
        q, m = O.gelu_quantize(xb, mode=mode, seed=7, stream=3, mx_mode=mode, mx_seed=9,
                               mx_stream=4)
        ref = O.nvfp4_quantize(gb, mode=mode, seed=7, stream=3)
        assert np.array_equal(q.codes, ref.codes) and np.array_equal(q.scales, ref.scales)
        assert q.s_dec == ref.s_dec
        mref = O.mxfp8_quantize(gb, mode=mode, seed=9, stream=4)
        assert np.array_equal(m.codes, mref.codes) and np.array_equal(m.scales, mref.scales)
    for pt in (False, True):
        for fs in (False, True):
            a = O.nvfp4_quantize_act(xb, per_token=pt, four_six=fs, gelu=True)
            b = O.nvfp4_quantize_act(gb, per_token=pt, four_six=fs, gelu=False)
            assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
            assert np.array_equal(np.atleast_1d(a.s_dec), np.atleast_1d(b.s_dec))


@pytest.mark.parametrize("four_six", [False, True])
def test_gelu_quantize_error(four_six):
    """The dequantized copy of GELU(x) is within NVFP4's error of x * Phi(x)."""
    xb = synth.normal_with_outliers(128, 256, 11)
    xd = O.bf16_to_f32(xb).astype(np.float64)
    exact = 0.5 * xd * (1.0 + erf(xd / math.sqrt(2.0)))
    q, _ = O.gelu_quantize(xb)
    assert O.rel_fro(q.dequant_f64(), exact) < 0.12
    a = O.nvfp4_quantize_act(xb, per_token=True, four_six=four_six, gelu=True)
    assert O.rel_fro(a.dequant_f64(), exact) < 0.12

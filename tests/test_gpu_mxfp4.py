"""GPU parity of the MXFP4 format (FP4 Training on Blackwell, 'The scaling
math, worked'): the quantizer bit for bit against the oracle, and the MXFP4 x
MXFP4 GEMM (gfx950's block-scaled MFMA with E2M1 operands) against the FP64
sum over the oracle's dequantized operands (relative Frobenius error <=
1e-3; BF16 output against that sum rounded to BF16).
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import announce, bf16_bits_to_f64, dev, host, to_dev
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 1e-3


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _quant(bbs, x, mode=O.RTN, rng=(0, 0), ld=None):
    R, C = x.shape
    xd = to_dev(x)
    if ld is not None:
        pad = torch.zeros((R, ld), dtype=torch.int16, device=dev())
        pad[:, :C] = xd
        xd = pad[:, :C]
    q = bbs.MXFP4Tensor.empty(R, C, device=dev())
    bbs.mxfp4_quantize(xd, q, round=mode, rng=rng)
    torch.cuda.synchronize()
    return q


def _same(g, o, what):
    assert np.array_equal(host(g.scales), o.scales), f"{what}: scales differ"
    gc = host(g.codes)
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()}")


@pytest.mark.parametrize("shape", [(1, 32), (16, 64), (37, 96), (64, 4096), (300, 544)])
def test_quantize(bbs, shape):
    R, C = shape
    announce(f"MXFP4 quantize {R}x{C} RTN + SR")
    x = synth.normal_with_outliers(R, C, 1100 + R + C)
    _same(_quant(bbs, x), O.mxfp4_quantize(x), "RTN")
    _same(_quant(bbs, x, O.SR, (99, 4)), O.mxfp4_quantize(x, O.SR, 99, 4), "SR")


def test_quantize_edges(bbs):
    """Row stride; zero, tiny (subnormal), huge blocks; exact grid values and
    the worked example's block (amax 22)."""
    announce("MXFP4 quantize edge blocks")
    x = synth.bf16_to_f32(synth.student_t(8, 128, 45)).copy()
    x[0] = 0.0
    x[1, :32] = np.float32([6.0, 4.0, 3.0, -2.0, 1.5, 1.0, 0.5, -6.0] * 4)
    x[2] *= np.float32(2.0 ** -130)
    x[3] *= np.float32(2.0 ** 100)
    x[4, :3] = [22.0, 3.0, -11.0]
    xb = synth.bf16_bits(x)
    _same(_quant(bbs, xb, ld=160), O.mxfp4_quantize(xb), "edges RTN")
    _same(_quant(bbs, xb, O.SR, (3, 1), ld=160), O.mxfp4_quantize(xb, O.SR, 3, 1), "edges SR")


def _gemm(bbs, a, b, M, N, bf16):
    c = torch.empty((M, N), dtype=torch.int16 if bf16 else torch.float32, device=dev())
    bbs.nvfp4_gemm(bbs.FMT_MXFP4, a, b, c, bbs.OUT_BF16 if bf16 else bbs.OUT_F32)
    torch.cuda.synchronize()
    y = host(c)
    return bf16_bits_to_f64(y.view(np.uint16)) if bf16 else y.astype(np.float64)


def _upload(bbs, o):
    return bbs.MXFP4Tensor(to_dev(o.codes), to_dev(o.scales), o.rows, o.cols)


def _random_mx4(R, C, seed):
    rng = np.random.default_rng(seed)
    return O.MXFP4(rng.integers(0, 256, (R, C // 2), dtype=np.uint8),
                   rng.integers(117, 137, (R, C // 32), dtype=np.uint8), R, C)


def _check(y, ref, bf16, what):
    r = O.bf16_rne(ref) if bf16 else ref
    err = O.rel_fro(y, r)
    print(f"  {what}: rel err {err:.3e}", flush=True)
    assert err <= TOL, f"{what}: relative error {err}"


def test_gemm_integer_case_exact(bbs):
    """All scales 1.0: every product is a multiple of 1/4 and the sums stay
    below 2^22, so the FP32 result is exact."""
    announce("MXFP4 GEMM integer special case, exact")
    rng = np.random.default_rng(12)
    M, N, K = 64, 96, 512
    a = O.MXFP4(rng.integers(0, 256, (M, K // 2), dtype=np.uint8),
                np.full((M, K // 32), 127, np.uint8), M, K)
    b = O.MXFP4(rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
                np.full((N, K // 32), 127, np.uint8), N, K)
    y = _gemm(bbs, _upload(bbs, a), _upload(bbs, b), M, N, False)
    assert np.array_equal(y, O.gemm_f64(a.dequant_f64(), b.dequant_f64()))


@pytest.mark.parametrize("M,N,K,bf16", [
    (16, 16, 256, False),
    (272, 400, 1024, True),        # ragged M and N
    (528, 272, 512, False),
    (64, 4112, 256, True),
    (300, 260, 2048, False),
])
def test_gemm_random(bbs, M, N, K, bf16):
    announce(f"MXFP4 GEMM random operands M={M} N={N} K={K} bf16={bf16}")
    a, b = _random_mx4(M, K, M + K), _random_mx4(N, K, N + 3 * K)
    y = _gemm(bbs, _upload(bbs, a), _upload(bbs, b), M, N, bf16)
    _check(y, O.gemm_f64(a.dequant_f64(), b.dequant_f64()), bf16, "random")


def test_gemm_unsupported_shapes(bbs):
    a, b = _random_mx4(32, 128, 1), _random_mx4(32, 128, 2)
    c = torch.empty((32, 32), dtype=torch.float32, device=dev())
    with pytest.raises(bbs.BbsError) as e:
        bbs.nvfp4_gemm(bbs.FMT_MXFP4, _upload(bbs, a), _upload(bbs, b), c, bbs.OUT_F32)
    assert e.value.status == bbs.BBS_ENOTSUP


def test_full_forward_mxfp4(bbs):
    """X 8192 x 4096 and W 14336 x 4096 of the dense layer as MXFP4 (RTN),
    the forward GEMM in the configuration bench.py times (BF16 out, sampled
    outputs against the FP64 sum)."""
    announce("full MXFP4 forward 8192x14336x4096 (quantize on the GPU, sampled check)")
    d = synth.dense_forward()
    ox, ow = O.mxfp4_quantize(d["x"]), O.mxfp4_quantize(d["w"])
    gx, gw = _quant(bbs, d["x"]), _quant(bbs, d["w"])
    _same(gx, ox, "X")
    _same(gw, ow, "W")
    y = _gemm(bbs, gx, gw, 8192, 14336, True)
    rng = np.random.default_rng(0)
    rows = np.concatenate([rng.integers(0, 8192, 4096), np.full(256, 8191)])
    cols = np.concatenate([rng.integers(0, 14336, 4096), np.arange(256) * 56])
    ref = O.gemm_f64_sampled(ox.dequant_f64(), ow.dequant_f64(), rows, cols)
    _check(y[rows, cols], ref, True, "MXFP4 fprop")

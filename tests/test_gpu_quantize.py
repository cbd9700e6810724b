"""GPU parity of the quantizer and requantizer against the CPU oracle.

Every code byte, scale byte and FP32 decode scale must be identical.  Inputs
are seeded synthetic tensors; expected values come from oracle/ only.
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import announce, dev, host, to_dev, upload_nvfp4
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _gpu_quantize(bbs, x, *, row=False, col=False, mx=False, tile2d=False, rht=False,
                  signs=0, row_round=O.RTN, col_round=O.RTN, mx_round=O.RTN,
                  row_rng=(0, 0), col_rng=(0, 0), mx_rng=(0, 0)):
    R, C = x.shape
    xd = to_dev(x)
    rq = bbs.NVFP4Tensor.empty(R, C, tile2d, device=dev()) if row else None
    cq = bbs.NVFP4Tensor.empty(C, R, tile2d, device=dev()) if col else None
    mq = bbs.MXFP8Tensor.empty(R, C, device=dev()) if mx else None
    bbs.nvfp4_quantize(xd, rq, cq, mq, row_round=row_round, row_rng=row_rng,
                       col_round=col_round, col_rng=col_rng, col_rht=rht, rht_signs=signs,
                       mx8_round=mx_round, mx8_rng=mx_rng, tile2d=tile2d)
    torch.cuda.synchronize()
    return rq, cq, mq


def _same_fp4(gq, oq, what):
    assert np.array_equal(host(gq.scales), oq.scales), f"{what}: scales differ"
    gc = host(gq.codes)
    if not np.array_equal(gc, oq.codes):
        bad = np.argwhere(gc != oq.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()}")
    assert host(gq.s_dec)[0] == oq.s_dec, f"{what}: s_dec {host(gq.s_dec)[0]} vs {oq.s_dec}"


def _same_mx8(gm, om, what):
    assert np.array_equal(host(gm.scales), om.scales), f"{what}: E8M0 scales differ"
    gc = host(gm.codes)
    if not np.array_equal(gc, om.codes):
        bad = np.argwhere(gc != om.codes)
        raise AssertionError(f"{what}: {len(bad)} E4M3 bytes differ, first at {bad[0].tolist()}")


SHAPES = [(16, 16), (32, 48), (48, 80), (64, 1040), (256, 256), (80, 96), (144, 528)]


@pytest.mark.parametrize("shape", SHAPES)
def test_row_rtn_and_sr(bbs, shape):
    R, C = shape
    announce(f"row 1x16 RTN+SR {shape}")
    x = synth.normal_with_outliers(R, C, 1000 + R + C)
    rq, _, _ = _gpu_quantize(bbs, x, row=True)
    _same_fp4(rq, O.nvfp4_quantize(x), "row RTN")
    rq, _, _ = _gpu_quantize(bbs, x, row=True, row_round=O.SR, row_rng=(0x1234, 5))
    _same_fp4(rq, O.nvfp4_quantize(x, mode=O.SR, seed=0x1234, stream=5), "row SR")


@pytest.mark.parametrize("shape", SHAPES)
def test_row_and_col_sr(bbs, shape):
    R, C = shape
    announce(f"row+col SR {shape}")
    x = synth.student_t(R, C, 2000 + R + C)
    rq, cq, _ = _gpu_quantize(bbs, x, row=True, col=True, row_round=O.SR, col_round=O.SR,
                              row_rng=(77, 0), col_rng=(77, 1))
    _same_fp4(rq, O.nvfp4_quantize(x, mode=O.SR, seed=77, stream=0), "row SR")
    _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, mode=O.SR, seed=77, stream=1), "col SR")


@pytest.mark.parametrize("shape", SHAPES)
def test_col_rht(bbs, shape):
    R, C = shape
    announce(f"col RHT RTN/SR {shape}")
    x = synth.normal_with_outliers(R, C, 3000 + R + C)
    s = synth.rht_signs(7 + R)
    _, cq, _ = _gpu_quantize(bbs, x, col=True, rht=True, signs=s)
    _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, rht=True, signs=s), "col RHT RTN")
    _, cq, _ = _gpu_quantize(bbs, x, col=True, rht=True, signs=s, col_round=O.SR,
                             col_rng=(99, 2))
    _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, rht=True, signs=s, mode=O.SR, seed=99,
                                   stream=2), "col RHT SR")


@pytest.mark.parametrize("shape", SHAPES)
def test_col_copy_alone(bbs, shape):
    """The column copy without row-wise copies (a 16 x 4 piece per thread):
    1x16 without the RHT and 16x16 tiles, each to nearest and stochastic."""
    R, C = shape
    announce(f"col alone 1x16 / 16x16, RTN+SR {shape}")
    x = synth.student_t(R, C, 5000 + R + C)
    for tile2d in (False, True):
        tag = "16x16" if tile2d else "1x16"
        _, cq, _ = _gpu_quantize(bbs, x, col=True, tile2d=tile2d)
        _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, tile2d=tile2d), f"col {tag} RTN")
        _, cq, _ = _gpu_quantize(bbs, x, col=True, tile2d=tile2d, col_round=O.SR,
                                 col_rng=(31, 3))
        _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, tile2d=tile2d, mode=O.SR, seed=31,
                                       stream=3), f"col {tag} SR")


@pytest.mark.parametrize("shape", SHAPES)
def test_tile2d_row_and_col(bbs, shape):
    R, C = shape
    announce(f"16x16 row+col RTN {shape}")
    w = synth.normal(R, C, 4000 + R + C, 0.02)
    rq, cq, _ = _gpu_quantize(bbs, w, row=True, col=True, tile2d=True)
    orow = O.nvfp4_quantize(w, tile2d=True)
    _same_fp4(rq, orow, "16x16 row")
    _same_fp4(cq, O.nvfp4_quantize(w, tile2d=True, transpose=True), "16x16 col")
    assert np.array_equal(host(cq.scales), host(rq.scales).T)


@pytest.mark.parametrize("shape", [s for s in SHAPES if s[1] % 32 == 0])
def test_mxfp8_row_copy(bbs, shape):
    R, C = shape
    announce(f"row MXFP8 RTN/SR {shape}")
    x = synth.laplace(R, C, 5000 + R + C, 1e-3)
    _, _, mq = _gpu_quantize(bbs, x, mx=True)
    _same_mx8(mq, O.mxfp8_quantize(x, mode=O.RTN), "MXFP8 RTN")
    _, _, mq = _gpu_quantize(bbs, x, mx=True, mx_round=O.SR, mx_rng=(404, 9))
    _same_mx8(mq, O.mxfp8_quantize(x, mode=O.SR, seed=404, stream=9), "MXFP8 SR")


def test_backward_pass_combination(bbs):
    # one read of dY: column-wise NVFP4 (RHT, SR) and row-wise MXFP8 (SR)
    R, C = 96, 160
    announce("dY combination col RHT SR + MXFP8 SR")
    x = synth.laplace(R, C, 6001, 1e-3)
    s = synth.rht_signs(402)
    _, cq, mq = _gpu_quantize(bbs, x, col=True, mx=True, rht=True, signs=s, col_round=O.SR,
                              mx_round=O.SR, col_rng=(403, 0), mx_rng=(404, 0))
    _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, rht=True, signs=s, mode=O.SR, seed=403),
              "dY col")
    _same_mx8(mq, O.mxfp8_quantize(x, mode=O.SR, seed=404), "dY MXFP8")
    # every copy at once, 1x16
    rq, cq, mq = _gpu_quantize(bbs, x, row=True, col=True, mx=True, rht=True, signs=s,
                               row_round=O.SR, col_round=O.SR, mx_round=O.SR,
                               row_rng=(1, 1), col_rng=(1, 2), mx_rng=(1, 3))
    _same_fp4(rq, O.nvfp4_quantize(x, mode=O.SR, seed=1, stream=1), "all: row")
    _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, rht=True, signs=s, mode=O.SR, seed=1,
                                   stream=2), "all: col")
    _same_mx8(mq, O.mxfp8_quantize(x, mode=O.SR, seed=1, stream=3), "all: MXFP8")


MX_COMBOS = [
    # (row, col, tile2d, rht): the MXFP8 row copy beside copies that need the
    # tensor amax, which the amax pass then writes from its own read
    (False, True, False, True),     # dY: columns RHT + MXFP8
    (True, False, False, False),    # rows 1x16 + MXFP8
    (True, False, True, False),     # rows 16x16 + MXFP8
    (True, True, False, False),     # rows + columns + MXFP8
    (True, True, False, True),      # rows + RHT'd columns + MXFP8
]


@pytest.mark.parametrize("shape", [(32, 96), (64, 1056), (144, 544), (272, 1600)])
@pytest.mark.parametrize("combo", MX_COMBOS, ids=["colrht", "row", "row2d", "rowcol", "rowcolrht"])
@pytest.mark.parametrize("mode", [O.RTN, O.SR], ids=["rtn", "sr"])
def test_mxfp8_beside_amax_copies(bbs, shape, combo, mode):
    row, col, tile2d, rht = combo
    R, C = shape
    announce(f"MXFP8 + copies {combo} {shape} mode={mode}")
    x = synth.laplace(R, C, 7000 + R + 3 * C, 1e-3)
    s = synth.rht_signs(402) if rht else 0
    rq, cq, mq = _gpu_quantize(bbs, x, row=row, col=col, mx=True, tile2d=tile2d, rht=rht, signs=s,
                               row_round=mode, col_round=mode, mx_round=mode,
                               row_rng=(11, 1), col_rng=(11, 2), mx_rng=(11, 3))
    _same_mx8(mq, O.mxfp8_quantize(x, mode=mode, seed=11, stream=3), "MXFP8")
    if row:
        _same_fp4(rq, O.nvfp4_quantize(x, tile2d=tile2d, mode=mode, seed=11, stream=1), "row")
    if col:
        _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, tile2d=tile2d, rht=rht, signs=s,
                                       mode=mode, seed=11, stream=2), "col")


@pytest.mark.parametrize("combo", [MX_COMBOS[1], MX_COMBOS[4]], ids=["row", "rowcolrht"])
def test_mxfp8_beside_amax_copies_many_partials(bbs, combo):
    # 2048 x 4096: the amax pass with the MXFP8 copy runs 512 workgroups, so
    # the encode folds 512 partials (more than one per thread of its share)
    row, col, tile2d, rht = combo
    R, C = 2048, 4096
    announce(f"MXFP8 + copies {combo} {(R, C)} mode=SR, many partials")
    x = synth.laplace(R, C, 7100, 1e-3)
    s = synth.rht_signs(403) if rht else 0
    rq, cq, mq = _gpu_quantize(bbs, x, row=row, col=col, mx=True, tile2d=tile2d, rht=rht, signs=s,
                               row_round=O.SR, col_round=O.SR, mx_round=O.SR,
                               row_rng=(12, 1), col_rng=(12, 2), mx_rng=(12, 3))
    _same_mx8(mq, O.mxfp8_quantize(x, mode=O.SR, seed=12, stream=3), "MXFP8")
    _same_fp4(rq, O.nvfp4_quantize(x, tile2d=tile2d, mode=O.SR, seed=12, stream=1), "row")
    if col:
        _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, tile2d=tile2d, rht=rht, signs=s,
                                       mode=O.SR, seed=12, stream=2), "col")


def test_degenerate_inputs(bbs):
    announce("zero / negative-zero / single-outlier tensors")
    z = np.zeros((32, 64), np.uint16)
    rq, cq, mq = _gpu_quantize(bbs, z, row=True, col=True, mx=True)
    _same_fp4(rq, O.nvfp4_quantize(z), "zeros row")
    _same_fp4(cq, O.nvfp4_quantize(z, transpose=True), "zeros col")
    _same_mx8(mq, O.mxfp8_quantize(z, mode=O.RTN), "zeros MXFP8")
    nz = np.full((32, 64), 0x8000, np.uint16)
    rq, _, _ = _gpu_quantize(bbs, nz, row=True)
    _same_fp4(rq, O.nvfp4_quantize(nz), "negative zeros")
    one = np.zeros((32, 64), np.float32)
    one[5, 9] = -3.0e-3
    one[17, 40] = 1.0e-30          # far below every other value: scale floor of 1
    x = synth.bf16_bits(one)
    rq, cq, _ = _gpu_quantize(bbs, x, row=True, col=True)
    _same_fp4(rq, O.nvfp4_quantize(x), "outlier row")
    _same_fp4(cq, O.nvfp4_quantize(x, transpose=True), "outlier col")


def test_row_stride(bbs):
    announce("source with a row stride larger than cols")
    full = synth.normal(64, 160, 6100, 1.0)
    xd = to_dev(full)[:, 16:144]
    rq = bbs.NVFP4Tensor.empty(64, 128, device=dev())
    bbs.nvfp4_quantize(xd, rq)
    torch.cuda.synchronize()
    _same_fp4(rq, O.nvfp4_quantize(np.ascontiguousarray(full[:, 16:144])), "strided row")


def test_sr_deterministic(bbs):
    announce("SR repeat determinism")
    x = synth.student_t(128, 256, 6200)
    a, b, _ = _gpu_quantize(bbs, x, row=True, col=True, row_round=O.SR, col_round=O.SR,
                            row_rng=(5, 0), col_rng=(5, 1))
    a2, b2, _ = _gpu_quantize(bbs, x, row=True, col=True, row_round=O.SR, col_round=O.SR,
                              row_rng=(5, 0), col_rng=(5, 1))
    assert torch.equal(a.codes, a2.codes) and torch.equal(b.codes, b2.codes)


# ---------------------------------------------------------------------------
# Requantize
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,tile2d", [((32, 16), False), ((64, 48), True), ((96, 160), False),
                                          ((256, 256), True), ((160, 1040), True)])
def test_requantize(bbs, shape, tile2d):
    R, C = shape
    announce(f"requantize {shape} tile2d={tile2d}")
    w = synth.normal_with_outliers(R, C, 7000 + R + C)
    oq = O.nvfp4_quantize(w, tile2d=tile2d)
    src = upload_nvfp4(oq, bbs)
    for mode, seed, stream in [(O.RTN, 0, 0), (O.SR, 406, 3)]:
        dst = bbs.MXFP8Tensor.empty(C, R, device=dev())
        bbs.mxfp8_requantize_t(src, dst, mode, (seed, stream))
        torch.cuda.synchronize()
        _same_mx8(dst, O.mxfp8_requantize_t(oq, mode=mode, seed=seed, stream=stream),
                  f"requant mode={mode}")


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

def test_full_activation_sr(bbs):
    announce("activation SR 4096x4096 row+col")
    d = synth.activation_sr()
    rq, cq, _ = _gpu_quantize(bbs, d["x"], row=True, col=True, row_round=O.SR, col_round=O.SR,
                              row_rng=(d["seed"], d["row_stream"]),
                              col_rng=(d["seed"], d["col_stream"]))
    _same_fp4(rq, O.nvfp4_quantize(d["x"], mode=O.SR, seed=d["seed"], stream=d["row_stream"]),
              "4096^2 row")
    _same_fp4(cq, O.nvfp4_quantize(d["x"], transpose=True, mode=O.SR, seed=d["seed"],
                                   stream=d["col_stream"]), "4096^2 col")


def test_full_dense_forward_quantize(bbs):
    announce("dense forward X 8192x4096 row RTN, W 14336x4096 16x16 RTN")
    d = synth.dense_forward()
    rq, _, _ = _gpu_quantize(bbs, d["x"], row=True)
    _same_fp4(rq, O.nvfp4_quantize(d["x"]), "X")
    del rq
    wq, _, _ = _gpu_quantize(bbs, d["w"], row=True, tile2d=True)
    _same_fp4(wq, O.nvfp4_quantize(d["w"], tile2d=True), "W")


def test_full_backward_quantize(bbs):
    announce("backward dY 8192x14336 col RHT SR + MXFP8 SR; X col RHT SR; W requant SR")
    fw = synth.dense_forward()
    bw = synth.backward()
    s, seeds = bw["rht_signs"], bw["seeds"]
    _, cq, mq = _gpu_quantize(bbs, bw["dy"], col=True, mx=True, rht=True, signs=s,
                              col_round=O.SR, mx_round=O.SR, col_rng=(seeds["dy_col"], 0),
                              mx_rng=(seeds["dy_mx8"], 0))
    _same_fp4(cq, O.nvfp4_quantize(bw["dy"], transpose=True, rht=True, signs=s, mode=O.SR,
                                   seed=seeds["dy_col"]), "dY col")
    _same_mx8(mq, O.mxfp8_quantize(bw["dy"], mode=O.SR, seed=seeds["dy_mx8"]), "dY MXFP8")
    del cq, mq
    _, xc, _ = _gpu_quantize(bbs, fw["x"], col=True, rht=True, signs=s, col_round=O.SR,
                             col_rng=(seeds["x_col"], 0))
    _same_fp4(xc, O.nvfp4_quantize(fw["x"], transpose=True, rht=True, signs=s, mode=O.SR,
                                   seed=seeds["x_col"]), "X col")
    del xc
    ow = O.nvfp4_quantize(fw["w"], tile2d=True)
    src = upload_nvfp4(ow, bbs)
    dst = bbs.MXFP8Tensor.empty(ow.cols, ow.rows, device=dev())
    bbs.mxfp8_requantize_t(src, dst, bbs.SR, (seeds["w_req"], 0))
    torch.cuda.synchronize()
    _same_mx8(dst, O.mxfp8_requantize_t(ow, mode=O.SR, seed=seeds["w_req"]), "W requant")


# ---------------------------------------------------------------------------
# Activation copy: per-token outer scale and / or Four Over Six
# ---------------------------------------------------------------------------

ACT_SHAPES = [(16, 16), (48, 80), (64, 1040), (256, 4096), (32, 8192 + 528)]


def _gpu_quantize_act(bbs, x, per_token, four_six, gelu=False):
    R, C = x.shape
    q = bbs.NVFP4Tensor.empty(R, C, device=dev(), sdec_per_row=per_token)
    bbs.nvfp4_quantize(to_dev(x), q, row_per_token=per_token, row_four_six=four_six, gelu=gelu)
    torch.cuda.synchronize()
    return q


@pytest.mark.parametrize("shape", ACT_SHAPES)
@pytest.mark.parametrize("per_token,four_six", [(True, True), (True, False), (False, True)])
def test_activation_copy(bbs, shape, per_token, four_six):
    R, C = shape
    announce(f"activation copy {R}x{C} per_token={per_token} four_six={four_six}")
    x = synth.normal_with_outliers(R, C, 700 + R + C)
    g = _gpu_quantize_act(bbs, x, per_token, four_six)
    o = O.nvfp4_quantize_act(x, per_token, four_six)
    assert np.array_equal(host(g.scales), o.scales), "scales differ"
    gc = host(g.codes)
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        raise AssertionError(f"{len(bad)} code bytes differ, first at {bad[0].tolist()}")
    sd = host(g.s_dec)
    assert np.array_equal(sd, np.atleast_1d(o.s_dec)), "decode scales differ"


def test_activation_copy_degenerate_rows(bbs):
    """All-zero rows (s_dec 1), a row of one repeated value (the top-4 scale
    saturates: ties keep the top-6 encoding) and a tiny-valued row."""
    announce("activation copy with zero / constant / tiny rows")
    x = synth.normal_with_outliers(32, 512, 91)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    xf[3] = 0.0
    xf[7] = 3.0
    xf[11] *= np.float32(2.0 ** -60)
    xb = synth.bf16_bits(xf)
    for pt, fs in [(True, True), (False, True)]:
        g = _gpu_quantize_act(bbs, xb, pt, fs)
        o = O.nvfp4_quantize_act(xb, pt, fs)
        assert np.array_equal(host(g.codes), o.codes)
        assert np.array_equal(host(g.scales), o.scales)
        assert np.array_equal(host(g.s_dec), np.atleast_1d(o.s_dec))


def test_full_activation_copy(bbs):
    """X of the dense forward (8192 x 4096) as the activation copy: per-token
    outer scale + Four Over Six, in the configuration bench.py times."""
    announce("full activation copy 8192x4096 per-token + 4/6")
    x = synth.dense_forward()["x"]
    g = _gpu_quantize_act(bbs, x, True, True)
    o = O.nvfp4_quantize_act(x, True, True)
    assert np.array_equal(host(g.scales), o.scales)
    assert np.array_equal(host(g.codes), o.codes)
    assert np.array_equal(host(g.s_dec), o.s_dec)


# ---------------------------------------------------------------------------
# Fused GELU + quantize (the copies are of GELU(x))
# ---------------------------------------------------------------------------

GELU_SHAPES = [(16, 16), (48, 80), (64, 1040), (256, 256), (144, 528), (272, 4096)]


def _gpu_gelu(bbs, x, *, row=True, mx=False, row_round=O.RTN, row_rng=(0, 0), mx_round=O.RTN,
              mx_rng=(0, 0)):
    R, C = x.shape
    rq = bbs.NVFP4Tensor.empty(R, C, device=dev()) if row else None
    mq = bbs.MXFP8Tensor.empty(R, C, device=dev()) if mx else None
    bbs.nvfp4_quantize(to_dev(x), rq, None, mq, row_round=row_round, row_rng=row_rng,
                       mx8_round=mx_round, mx8_rng=mx_rng, gelu=True)
    torch.cuda.synchronize()
    return rq, mq


@pytest.mark.parametrize("shape", GELU_SHAPES)
def test_gelu_quantize(bbs, shape):
    R, C = shape
    announce(f"GELU + quantize {R}x{C}")
    x = synth.normal_with_outliers(R, C, 900 + R + C)
    rq, _ = _gpu_gelu(bbs, x)
    _same_fp4(rq, O.gelu_quantize(x)[0], "GELU row RTN")
    if C % 32 == 0:
        rq, mq = _gpu_gelu(bbs, x, mx=True, row_round=O.SR, row_rng=(31, 2), mx_round=O.SR,
                           mx_rng=(32, 3))
        oq, om = O.gelu_quantize(x, mode=O.SR, seed=31, stream=2, mx_mode=O.SR, mx_seed=32,
                                 mx_stream=3)
        _same_fp4(rq, oq, "GELU row SR")
        _same_mx8(mq, om, "GELU MXFP8 SR")
        _, mq = _gpu_gelu(bbs, x, row=False, mx=True)
        _same_mx8(mq, O.gelu_quantize(x, mx_mode=O.RTN)[1], "GELU MXFP8 RTN alone")


def test_gelu_quantize_every_bf16_value(bbs):
    """Every finite BF16 value (a seeded shuffle, zero-padded to 256 x 256)
    through the fused GELU copies: the kernels' GELU table, its range
    boundaries and the identities outside it, against the oracle."""
    announce("GELU + quantize over every finite BF16 value")
    h = np.arange(65536, dtype=np.uint32)
    f = (h << 16).view(np.float32)
    vals = h[np.isfinite(f)].astype(np.uint16)
    x = np.zeros(65536, np.uint16)
    x[:len(vals)] = np.random.default_rng(23).permutation(vals)
    x = x.reshape(256, 256)
    rq, mq = _gpu_gelu(bbs, x, mx=True, row_round=O.SR, row_rng=(5, 1), mx_round=O.SR,
                       mx_rng=(6, 2))
    oq, om = O.gelu_quantize(x, mode=O.SR, seed=5, stream=1, mx_mode=O.SR, mx_seed=6,
                             mx_stream=2)
    _same_fp4(rq, oq, "GELU row SR, all BF16")
    _same_mx8(mq, om, "GELU MXFP8 SR, all BF16")
    for pt, fs in [(True, True), (False, True), (True, False)]:
        g = _gpu_quantize_act(bbs, x, pt, fs, gelu=True)
        o = O.nvfp4_quantize_act(x, pt, fs, gelu=True)
        assert np.array_equal(host(g.scales), o.scales)
        assert np.array_equal(host(g.codes), o.codes)
        assert np.array_equal(host(g.s_dec), np.atleast_1d(o.s_dec))


def _gelu_edge_inputs():
    """Inputs whose |GELU| maximum lies on the negative side (or is 0), so
    the quantizers must evaluate the negative elements: all negative, all
    small, zeros, and rows of large values next to rows of negatives."""
    rng = np.random.default_rng(17)
    base = rng.standard_normal((64, 544)).astype(np.float32)
    cases = {
        "all negative": -np.abs(base),
        "all small": base * np.float32(0.05),
        "near the minimum": np.float32(-0.75) + base * np.float32(0.01),
        "zeros": np.zeros_like(base),
    }
    mixed = -np.abs(base)
    mixed[:16] = np.abs(base[:16]) * 4
    cases["mixed rows"] = mixed
    return {k: synth.bf16_bits(v) for k, v in cases.items()}


def test_gelu_quantize_negative_side(bbs):
    announce("GELU + quantize where the negative side sets the amax")
    for name, x in _gelu_edge_inputs().items():
        rq, mq = _gpu_gelu(bbs, x, mx=True)
        oq, om = O.gelu_quantize(x, mx_mode=O.RTN)
        _same_fp4(rq, oq, f"GELU row, {name}")
        _same_mx8(mq, om, f"GELU MXFP8, {name}")
        for pt, fs in [(True, True), (True, False), (False, True)]:
            g = _gpu_quantize_act(bbs, x, pt, fs, gelu=True)
            o = O.nvfp4_quantize_act(x, pt, fs, gelu=True)
            assert np.array_equal(host(g.scales), o.scales), f"{name} {pt} {fs}"
            assert np.array_equal(host(g.codes), o.codes), f"{name} {pt} {fs}"
            assert np.array_equal(host(g.s_dec), np.atleast_1d(o.s_dec)), f"{name} {pt} {fs}"


@pytest.mark.parametrize("shape", ACT_SHAPES)
@pytest.mark.parametrize("per_token,four_six", [(True, True), (True, False), (False, True)])
def test_gelu_activation_copy(bbs, shape, per_token, four_six):
    R, C = shape
    announce(f"GELU activation copy {R}x{C} per_token={per_token} four_six={four_six}")
    x = synth.normal_with_outliers(R, C, 950 + R + C)
    g = _gpu_quantize_act(bbs, x, per_token, four_six, gelu=True)
    o = O.nvfp4_quantize_act(x, per_token, four_six, gelu=True)
    assert np.array_equal(host(g.scales), o.scales), "scales differ"
    gc = host(g.codes)
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        raise AssertionError(f"{len(bad)} code bytes differ, first at {bad[0].tolist()}")
    assert np.array_equal(host(g.s_dec), np.atleast_1d(o.s_dec)), "decode scales differ"


def test_full_gelu_quantize(bbs):
    """The MLP hidden tensor H (8192 x 14336), as bench.py times it: the
    NVFP4 copy of GELU(H) (RTN) and its MXFP8 copy (SR) from one pass."""
    announce("full GELU + quantize 8192x14336 row RTN + MXFP8 SR")
    d = synth.mlp_hidden()
    rq, mq = _gpu_gelu(bbs, d["h"], mx=True, mx_round=O.SR, mx_rng=(d["seeds"]["mx8"], 0))
    oq, om = O.gelu_quantize(d["h"], mx_mode=O.SR, mx_seed=d["seeds"]["mx8"])
    _same_fp4(rq, oq, "GELU(H) row")
    _same_mx8(mq, om, "GELU(H) MXFP8")


def test_full_gelu_activation_copy(bbs):
    """GELU(H) as the activation copy: per-token outer scale + Four Over Six
    (rows of 14336 are read twice: the amax, then the encode)."""
    announce("full GELU activation copy 8192x14336 per-token + 4/6")
    h = synth.mlp_hidden()["h"]
    g = _gpu_quantize_act(bbs, h, True, True, gelu=True)
    o = O.nvfp4_quantize_act(h, True, True, gelu=True)
    assert np.array_equal(host(g.scales), o.scales)
    assert np.array_equal(host(g.codes), o.codes)
    assert np.array_equal(host(g.s_dec), o.s_dec)

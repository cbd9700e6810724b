"""Every finite BF16 value, subnormals included, through every quantizer copy
and the requantizer, bit-exact against the oracle.

The pages define the E2M1 subnormal (exponent 0) and the E4M3 minimum 2^-9
(4bit.vizuara.ai, sections 3-4), and a block's scale is set by its largest
value, so small values inside a block with a large maximum and values far
below the tensor maximum are where the two-level scaling is tested hardest.
The finite BF16 magnitudes (exponent fields 0 .. 254, 128 mantissas each)
are split into windows of 16 exponent fields; the windows overlap by 8, and
each window's 2048 magnitudes with both signs (and zeros for the rest) fill
a 96 x 64 tensor in a seeded shuffle, so every 1x16 block, 16x16 tile and
32-block spans up to 16 binades.  The lowest windows also hold one value 2^-98, so that the tensor
amax (and that of the RHT'd copy) meets the library's documented
precondition (0, or at least 2^-100).
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import announce, dev, host, to_dev, upload_nvfp4

torch = pytest.importorskip("torch")

SIGNS = 0x6A3C


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _windows():
    out = []
    for w in range(0, 255, 8):
        e1 = min(w + 16, 255)
        mags = np.arange(w << 7, e1 << 7, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        rng = np.random.default_rng(5000 + w)
        x = np.zeros(96 * 64, np.uint16)      # the rest are zeros
        x[:vals.size] = vals
        if e1 <= 30:                          # amax below 2^-97: add one 2^-98
            x[vals.size] = 0x0E80
        out.append((w, e1, rng.permutation(x).reshape(96, 64)))
    return out


WINDOWS = _windows()


def test_windows_cover_every_finite_bf16():
    seen = np.zeros(65536, bool)
    for _, _, x in WINDOWS:
        seen[x.ravel()] = True
    finite = np.ones(65536, bool)
    finite[0x7F80:0x8000] = False
    finite[0xFF80:] = False
    assert seen[finite].all()


def _same_fp4(gq, oq, what):
    assert host(gq.s_dec)[0] == oq.s_dec, f"{what}: s_dec"
    assert np.array_equal(host(gq.scales), oq.scales), f"{what}: scales"
    g = host(gq.codes)
    if not np.array_equal(g, oq.codes):
        bad = np.argwhere(g != oq.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()}")


def _same_mx8(gm, om, what):
    assert np.array_equal(host(gm.scales), om.scales), f"{what}: E8M0 scales"
    g = host(gm.codes)
    if not np.array_equal(g, om.codes):
        bad = np.argwhere(g != om.codes)
        raise AssertionError(f"{what}: {len(bad)} E4M3 bytes differ, first at {bad[0].tolist()}")


@pytest.mark.gpu
@pytest.mark.parametrize("w,e1,x", WINDOWS, ids=[f"exp{w}-{e1}" for w, e1, _ in WINDOWS])
def test_every_copy_over_a_window(bbs, w, e1, x):
    announce(f"BF16 exponent fields [{w}, {e1}): every copy, RTN and SR")
    R, C = x.shape
    xd = to_dev(x)
    T = bbs.NVFP4Tensor
    ws = bbs.amax_workspace(dev())
    for mode in (O.RTN, O.SR):
        rq, cq, mq = T.empty(R, C, device=dev()), T.empty(C, R, device=dev()), \
            bbs.MXFP8Tensor.empty(R, C, device=dev())
        bbs.nvfp4_quantize(xd, rq, cq, mq, row_round=mode, row_rng=(w + 1, 1), col_round=mode,
                           col_rng=(w + 1, 2), mx8_round=mode, mx8_rng=(w + 1, 3), amax_ws=ws)
        # the 16-point RHT can grow a magnitude by up to 4x: windows reaching
        # exponent field 253 would overflow inside the transform (outside
        # the finite-input precondition) and take only the plain copies
        rht_ok = e1 <= 253
        hq = T.empty(C, R, device=dev())
        if rht_ok:
            bbs.nvfp4_quantize(xd, None, hq, col_round=mode, col_rng=(w + 1, 4), col_rht=True,
                               rht_signs=SIGNS, amax_ws=ws)
        torch.cuda.synchronize()
        tag = "RTN" if mode == O.RTN else "SR"
        _same_fp4(rq, O.nvfp4_quantize(x, mode=mode, seed=w + 1, stream=1), f"row {tag}")
        _same_fp4(cq, O.nvfp4_quantize(x, transpose=True, mode=mode, seed=w + 1, stream=2),
                  f"col {tag}")
        _same_mx8(mq, O.mxfp8_quantize(x, mode=mode, seed=w + 1, stream=3), f"MXFP8 {tag}")
        if rht_ok:
            _same_fp4(hq, O.nvfp4_quantize(x, transpose=True, rht=True, signs=SIGNS, mode=mode,
                                           seed=w + 1, stream=4), f"col RHT {tag}")
    # 16x16 tiles: row copy and its bit-identical transpose
    tr, tc = T.empty(R, C, tile2d=True, device=dev()), T.empty(C, R, tile2d=True, device=dev())
    bbs.nvfp4_quantize(xd, tr, tc, tile2d=True, amax_ws=ws)
    torch.cuda.synchronize()
    ot = O.nvfp4_quantize(x, tile2d=True)
    _same_fp4(tr, ot, "16x16 row")
    _same_fp4(tc, O.nvfp4_quantize(x, transpose=True, tile2d=True), "16x16 col")
    # requantize both NVFP4 layouts (uploaded from the oracle) to MXFP8 of the transpose
    o1 = O.nvfp4_quantize(x)
    for src, what in ((ot, "16x16"), (o1, "1x16")):
        for mode in (O.RTN, O.SR):
            dst = bbs.MXFP8Tensor.empty(C, R, device=dev())
            bbs.mxfp8_requantize_t(upload_nvfp4(src, bbs), dst, mode, (w + 7, 5))
            torch.cuda.synchronize()
            _same_mx8(dst, O.mxfp8_requantize_t(src, mode=mode, seed=w + 7, stream=5),
                      f"requantize {what} {'RTN' if mode == O.RTN else 'SR'}")

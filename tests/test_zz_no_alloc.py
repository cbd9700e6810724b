"""The quantizer entry point that allocates nothing (nvfp4_quantize_noalloc)
against nvfp4_quantize with a caller workspace: every code, scale and decode
scale byte must be identical.  Each case makes two calls in a row, the second
on a smaller input with a smaller amax, so partials the first call left in
the library's scratch would show up in the second call's scales."""
import numpy as np
import pytest

import oracle as O
from gpu_util import announce, dev, host, to_dev
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _inputs(seed, big, small):
    """A large input with a few large outliers, then a smaller, quieter one."""
    x1 = synth.normal_with_outliers(big[0], big[1], seed)
    f = synth.bf16_to_f32(x1)
    f[3, 7] = 900.0
    f[big[0] - 1, big[1] - 2] = -1200.0
    x1 = synth.bf16_bits(f)
    x2 = synth.laplace(small[0], small[1], seed + 1, 1e-3)
    return x1, x2


def _copies(bbs, R, C, *, row, col, mx, tile2d):
    rq = bbs.NVFP4Tensor.empty(R, C, tile2d, device=dev()) if row else None
    cq = bbs.NVFP4Tensor.empty(C, R, tile2d, device=dev()) if col else None
    mq = bbs.MXFP8Tensor.empty(R, C, device=dev()) if mx else None
    return rq, cq, mq


def _same(a, b, what):
    for name in ("codes", "scales", "s_dec"):
        if a is None:
            assert b is None
            return
        if not hasattr(a, name):
            continue
        ga, gb = host(getattr(a, name)), host(getattr(b, name))
        assert ga.shape == gb.shape, f"{what}: {name} shapes differ"
        if not np.array_equal(ga.view(np.uint8), gb.view(np.uint8)):
            bad = np.argwhere(ga.view(np.uint8) != gb.view(np.uint8))
            raise AssertionError(f"{what}: {len(bad)} {name} bytes differ, first at {bad[0]}")


CASES = [
    # (label, options, copies)
    ("row RTN + col RHT SR", dict(col_round=O.SR, col_rng=(405, 0), col_rht=True,
                                  rht_signs=0xA5C3), dict(row=True, col=True, mx=False)),
    ("col RHT SR + MXFP8 SR", dict(col_round=O.SR, col_rng=(403, 0), col_rht=True,
                                   rht_signs=0x3C5A, mx8_round=O.SR, mx8_rng=(404, 0)),
     dict(row=False, col=True, mx=True)),
    ("16x16 row + col RTN", dict(tile2d=True), dict(row=True, col=True, mx=False)),
    ("row SR + col SR", dict(row_round=O.SR, row_rng=(0x2001, 0), col_round=O.SR,
                             col_rng=(0x2001, 1)), dict(row=True, col=True, mx=False)),
    ("GELU row + MXFP8 SR", dict(gelu=True, mx8_round=O.SR, mx8_rng=(602, 0)),
     dict(row=True, col=False, mx=True)),
]


@pytest.mark.parametrize("label,opts,copies", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry_point(bbs, label, opts, copies):
    tile2d = opts.get("tile2d", False)
    x1, x2 = _inputs(8800 + len(label), (512, 1024), (96, 160))
    for i, x in enumerate((x1, x2)):
        R, C = x.shape
        announce(f"noalloc {label}, call {i + 1}, {R}x{C}")
        xd = to_dev(x)
        ref = _copies(bbs, R, C, tile2d=tile2d, **copies)
        got = _copies(bbs, R, C, tile2d=tile2d, **copies)
        bbs.nvfp4_quantize(xd, *ref, amax_ws=bbs.amax_workspace(dev()), **opts)
        bbs.nvfp4_quantize_noalloc(xd, *got, **opts)
        torch.cuda.synchronize()
        for a, b, what in zip(got, ref, ("row", "col", "mx8")):
            _same(a, b, f"{label} call {i + 1} {what}")


def test_noalloc_matches_oracle_after_a_larger_call(bbs):
    # the scratch keeps the larger first call's partials; the second call's
    # tensor scale must still be the oracle's
    x1, x2 = _inputs(8900, (1024, 2048), (64, 96))
    for i, x in enumerate((x1, x2)):
        R, C = x.shape
        announce(f"noalloc vs oracle, call {i + 1}, {R}x{C}")
        rq = bbs.NVFP4Tensor.empty(R, C, device=dev())
        bbs.nvfp4_quantize_noalloc(to_dev(x), rq)
        torch.cuda.synchronize()
        oq = O.nvfp4_quantize(x)
        assert np.array_equal(host(rq.codes), oq.codes), f"call {i + 1}: codes differ"
        assert np.array_equal(host(rq.scales), oq.scales), f"call {i + 1}: scales differ"
        assert host(rq.s_dec)[0] == oq.s_dec, f"call {i + 1}: s_dec differs"


def test_noalloc_rejects_a_workspace(bbs):
    import ctypes as C
    x = torch.zeros((32, 32), dtype=torch.int16, device=dev())
    rq = bbs.NVFP4Tensor.empty(32, 32, device=dev())
    d = rq.desc()
    a = bbs.QuantArgs(x.data_ptr(), 32, 32, 32, C.pointer(d), 0, bbs.Rng(0, 0), None, 0,
                      bbs.Rng(0, 0), 0, 0, None, 0, bbs.Rng(0, 0), 0,
                      bbs.amax_workspace(dev()).data_ptr(), 0, 0, 0)
    assert bbs.lib.nvfp4_quantize_noalloc(C.byref(a), None) == bbs.BBS_EINVAL
    assert b"amax_ws must be NULL" in bbs.lib.bbs_last_error()

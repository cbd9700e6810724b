"""GPU parity of the combine wire format (32-point RHT + block-scaled S2F6)
against the CPU oracle: codes and scales bit for bit, the receiver's FP32
sums bit for bit (BF16 output: the oracle's FP32 rounded to nearest even).
Inputs are seeded synthetic tensors; expected values come from oracle/ only.
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import announce, dev, host, to_dev
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SIGNS = 0xB5297A4D


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _encode(bbs, x, rht, signs=SIGNS, ld=None):
    R, C = x.shape
    xd = to_dev(x)
    if ld is not None:
        pad = torch.zeros((R, ld), dtype=torch.int16, device=dev())
        pad[:, :C] = xd
        xd = pad[:, :C]
    q = bbs.S2F6Tensor.empty(R, C, device=dev())
    bbs.s2f6_quantize(xd, q, rht=rht, signs=signs)
    torch.cuda.synchronize()
    return q


def _same_s2f6(g, o, what):
    assert np.array_equal(host(g.scales), o.scales), f"{what}: scales differ"
    gc = host(g.codes)
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {bad[0].tolist()}")


SHAPES = [(1, 32), (16, 64), (37, 96), (64, 4096), (300, 544)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("rht", [True, False])
def test_encode(bbs, shape, rht):
    R, C = shape
    announce(f"S2F6 encode {R}x{C} rht={rht}")
    x = synth.normal_with_outliers(R, C, 800 + R + C, frac=0.0035, factor=10.0)
    _same_s2f6(_encode(bbs, x, rht), O.s2f6_quantize(x, rht=rht, signs=SIGNS), "encode")


def test_encode_row_stride_and_edges(bbs):
    """A row stride beyond cols; zero blocks; blocks at the top of the grid,
    just above it, tiny (subnormal BF16) and huge values."""
    announce("S2F6 encode: row stride, zero / exact / tiny / huge blocks")
    x = synth.bf16_to_f32(synth.normal_with_outliers(8, 128, 44)).copy()
    x[0] = 0.0
    x[1, :32] = 127.0 / 64
    x[1, 32:64] = 2.0
    x[2] *= np.float32(2.0 ** -130)
    x[3] *= np.float32(2.0 ** 100)
    x[4, 5] = -2.0
    xb = synth.bf16_bits(x)
    for rht in (True, False):
        _same_s2f6(_encode(bbs, xb, rht, ld=200), O.s2f6_quantize(xb, rht=rht, signs=SIGNS),
                   f"edges rht={rht}")


def _combine(bbs, q, src, w, rht, bf16, ldo=None):
    T, K = src.shape
    C = q.cols
    ldo = ldo or C
    out = torch.zeros((T, ldo), dtype=torch.int16 if bf16 else torch.float32, device=dev())
    bbs.s2f6_combine(q, to_dev(src), out, None if w is None else to_dev(w), rht=rht,
                     signs=SIGNS, out_dtype=bbs.OUT_BF16 if bf16 else bbs.OUT_F32, ldo=ldo)
    torch.cuda.synchronize()
    return host(out)[:, :C]


def _upload_s2f6(bbs, o):
    return bbs.S2F6Tensor(to_dev(o.codes), to_dev(o.scales), o.rows, o.cols)


@pytest.mark.parametrize("rht", [True, False])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("k", [5, 8])
def test_combine(bbs, rht, weighted, bf16, k):
    announce(f"S2F6 combine rht={rht} weighted={weighted} bf16={bf16} k={k}")
    rng = np.random.default_rng(31)
    x = synth.normal_with_outliers(96, 544, 55, frac=0.0035, factor=10.0)
    o = O.s2f6_quantize(x, rht=rht, signs=SIGNS)
    src = rng.integers(0, 96, (40, k)).astype(np.int32)
    src[3, 2] = -1
    src[7, :] = -1                                  # a token with no rows: zeros
    w = rng.uniform(0.05, 1.0, (40, k)).astype(np.float32) if weighted else None
    ref = O.s2f6_combine(o, src, w, rht=rht, signs=SIGNS)
    got = _combine(bbs, _upload_s2f6(bbs, o), src, w, rht, bf16, ldo=544 + 32)
    if bf16:
        assert np.array_equal(got.view(np.uint16), synth.bf16_bits(ref))
    else:
        bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
        assert len(bad) == 0, f"{len(bad)} values differ, first {got.reshape(-1)[bad[0]]} vs {ref.reshape(-1)[bad[0]]}"


@pytest.mark.parametrize("k", [4, 8])
def test_combine_out_of_range_rows_skipped(bbs, k):
    """Source indices at or past the number of encoded rows are skipped like
    negative ones (a dropped slot): the result equals the oracle's with those
    slots set to -1."""
    announce(f"S2F6 combine with out-of-range source rows, k={k}")
    rng = np.random.default_rng(32)
    x = synth.normal_with_outliers(64, 256, 57, frac=0.0035, factor=10.0)
    o = O.s2f6_quantize(x, rht=True, signs=SIGNS)
    src = rng.integers(0, 64, (24, k)).astype(np.int32)
    src[1, 0], src[5, 3], src[9, :] = 64, 1 << 30, 70
    src[11, 1] = -1
    w = rng.uniform(0.05, 1.0, (24, k)).astype(np.float32)
    clean = np.where(src >= 64, -1, src).astype(np.int32)
    ref = O.s2f6_combine(o, clean, w, rht=True, signs=SIGNS)
    got = _combine(bbs, _upload_s2f6(bbs, o), src, w, True, False)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_encode_then_combine_round_trip(bbs):
    """Device encode then device combine of single copies: within the wire
    format's error of the input."""
    announce("S2F6 encode -> combine round trip")
    x = synth.normal_with_outliers(128, 1024, 66, frac=0.0035, factor=10.0)
    q = _encode(bbs, x, True)
    got = _combine(bbs, q, np.arange(128, dtype=np.int32)[:, None], None, True, False)
    assert O.rel_fro(got.astype(np.float64), synth.bf16_to_f32(x).astype(np.float64)) < 0.012


def test_full_moe_combine_sampled(bbs):
    """The MoE combine at full size as bench.py times it: 524288 expert-output
    rows of 4096 encoded, then 65536 tokens x 8 rows combined with gate
    weights into BF16.  Sampled rows / tokens are recomputed by the oracle
    from the same inputs."""
    announce("full MoE combine: encode 524288x4096, combine 65536 tokens x 8")
    d = synth.moe_combine(device=dev())
    y, src, w, signs = d["y"], d["src"], d["w"], d["signs"]
    R, C = y.shape
    q = bbs.S2F6Tensor.empty(R, C, device=dev())
    bbs.s2f6_quantize(y, q, rht=True, signs=signs)
    out = torch.empty((src.shape[0], C), dtype=torch.int16, device=dev())
    bbs.s2f6_combine(q, to_dev(src), out, to_dev(w), rht=True, signs=signs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(src.shape[0], 96, replace=False))
    tokens[-1] = src.shape[0] - 1
    rows = np.unique(src[tokens].reshape(-1))
    yr = host(y[torch.from_numpy(rows).to(dev())]).view(np.uint16)
    o = O.s2f6_quantize(yr, rht=True, signs=signs)
    assert np.array_equal(host(q.codes[torch.from_numpy(rows).to(dev())]), o.codes)
    assert np.array_equal(host(q.scales[torch.from_numpy(rows).to(dev())]), o.scales)
    local = np.searchsorted(rows, src[tokens]).astype(np.int32)
    ref = O.s2f6_combine(o, local, w[tokens], rht=True, signs=signs)
    assert np.array_equal(host(out[torch.from_numpy(tokens).to(dev())]).view(np.uint16),
                          synth.bf16_bits(ref))

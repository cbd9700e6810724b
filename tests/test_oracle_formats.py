"""Pins of the oracle's number formats against the pages and brute force."""
import numpy as np

import oracle as O
from golden_data import golden


def test_e2m1_decode_table():
    g = golden("e2m1_magnitudes")
    mags = [O.e2m1_value(c) for c in range(8)]
    assert mags == g["value"]
    for c in range(8):
        v = O.e2m1_value(8 | c)
        assert v == -g["value"][c] and np.signbit(v)
    e = golden("e2m1_0111")
    assert O.e2m1_value(e["code"]) == e["value"]


def test_e4m3_widget_and_limits():
    w = golden("e4m3_widget")
    assert int(w["bits"].replace(" ", ""), 2) == w["byte"]
    assert O.e4m3_value(w["byte"]) == w["value"]
    assert O.e2m1_value(int(w["fp4_bits"].replace(" ", ""), 2)) == w["fp4_value"]
    assert w["value"] * w["fp4_value"] == w["reconstructed"]
    lim = golden("e4m3_limits")
    finite = [O.e4m3_value(b) for b in range(0x7F)]
    assert max(finite) == lim["max"] == O.e4m3_value(0x7E)
    assert min(v for v in finite if v > 0) == lim["min_positive"] == O.e4m3_value(0x01)
    assert len(set(finite)) == lim["distinct_magnitudes_incl_zero"]
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))


def test_code_roundtrip_exhaustive():
    for c in range(16):
        assert O.e2m1_code(np.float32(O.e2m1_value(c)))[()] == c
    for b in range(256):
        if b & 0x7F == 0x7F:
            continue
        assert O.e4m3_code(np.float32(O.e4m3_value(b)))[()] == b


def test_worked_rounding():
    e = golden("round_3p2")
    r = O.round_to(np.float32(e["input"]), O.E2M1)[()]
    assert r == e["output"]
    assert abs((r - e["input"]) - e["error"]) < 1e-6
    # 5.5 lies between 4 and 6 and is nearer 6; 7 and 100 saturate at 6.
    assert list(O.round_to(np.float32([5.5, 7.0, 100.0, -100.0]), O.E2M1)) == [6, 6, 6, -6]
    # Ties go to the even code (reading; one page's example rounds 0.75 down).
    assert list(O.round_to(np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]), O.E2M1)) == \
        [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    # Signed zero is kept.
    z = O.round_to(np.float32([-0.1, -0.0]), O.E2M1)
    assert np.all(z == 0) and np.all(np.signbit(z))
    assert list(O.e2m1_code(z)) == [8, 8]


def _table_nearest_even(x: np.ndarray, table: np.ndarray, vmax: float) -> np.ndarray:
    """Brute force: nearest table entry, ties to the even code, saturating."""
    a = np.minimum(np.abs(x.astype(np.float64)), vmax)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.arange(table.size)
    # among tied candidates choose the one with an even code
    even = cand & (idx[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return np.copysign(table[pick], x.astype(np.float64))


def _sweep(lo: float, hi: float, grid: np.ndarray, stride: int) -> np.ndarray:
    bl = np.float32(lo).view(np.uint32)
    bh = np.float32(hi).view(np.uint32)
    pats = np.arange(int(bl), int(bh), stride, dtype=np.uint64).astype(np.uint32)
    xs = pats.view(np.float32)
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(np.inf)), grid.astype(np.float32)])
    xs = np.concatenate([xs, near, -xs, -near]).astype(np.float32)
    return xs


def test_e2m1_rtn_bruteforce():
    table = np.array([O.e2m1_value(c) for c in range(8)])
    xs = _sweep(0.0, 9.0, table, 1009)
    got = O.round_to(xs, O.E2M1).astype(np.float64)
    ref = _table_nearest_even(xs, table, 6.0)
    assert np.array_equal(got, ref)
    codes = O.e2m1_code(got.astype(np.float32))
    assert np.all(codes < 16)
    dec = np.array([O.e2m1_value(c) for c in range(16)])
    assert np.array_equal(dec[codes], got)


def test_e4m3_rtn_bruteforce():
    table = np.array([O.e4m3_value(b) for b in range(0x7F)])
    assert np.all(np.diff(table) > 0)
    xs = _sweep(0.0, 520.0, table, 20011)
    got = O.round_to(xs, O.E4M3).astype(np.float64)
    ref = _table_nearest_even(xs, table, 448.0)
    assert np.array_equal(got, ref)


def test_nvfp4_range_and_storage():
    r = golden("nvfp4_range")
    prods = [O.e2m1_value(c) * O.e4m3_value(s) for c in range(1, 8) for s in range(1, 0x7F)]
    assert min(prods) == r["min"] and max(prods) == r["max"]
    assert min(prods) * 2 == r["outer2_min"] and max(prods) * 2 == r["outer2_max"]
    b = golden("bits_per_value")
    R, Cc = 64, 256
    q = O.nvfp4_quantize(np.zeros((R, Cc), np.uint16))
    assert (q.codes.nbytes + q.scales.nbytes) * 8 / (R * Cc) == b["nvfp4"]
    m = O.mxfp8_quantize(np.zeros((R, Cc), np.uint16))
    assert (m.codes.nbytes + m.scales.nbytes) * 8 / (R * Cc) == b["mxfp8"]


def test_block_minus54():
    e = golden("block_minus54")
    # A tensor whose amax is 2688 has s_enc = s_dec = 1, so the block scale is 54/6.
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2688.0
    x[0, 16] = e["block_max"]
    x[0, 17] = 13.5          # 13.5 / 9 = 1.5, a grid point
    x[0, 18] = 27.0          # 27 / 9 = 3
    s_enc = O.tensor_s_enc(2688.0)
    assert s_enc == 1.0
    q = O.nvfp4_encode_f32(x, s_enc)
    assert q.scales[0, 1] == e["scale_code"]
    assert O.e4m3_value(int(q.scales[0, 1])) == e["scale"]
    assert (q.codes[0, 8] & 0xF) == e["code"]
    assert O.e2m1_value(e["code"]) == e["stored"]
    assert (q.codes[0, 8] >> 4) == 3 and (q.codes[0, 9] & 0xF) == 5


def test_widget_saturation():
    # Block max 593.7 in a tensor with s_enc = 1: the scale rounds to 96 and
    # the value saturates at 6, giving 576 (error -17.7).
    w = golden("e4m3_widget")
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2688.0
    x[0, 16] = np.float32(w["reconstructed"] - w["quant_error"])
    q = O.nvfp4_encode_f32(x, 1.0)
    assert q.scales[0, 1] == w["byte"]
    deq = q.dequant_f64()[0, 16]
    assert deq == w["reconstructed"]
    assert abs((deq - x[0, 16]) - w["quant_error"]) < 1e-3


def test_tensor_scale_rules():
    assert O.tensor_s_enc(2688.0) == 1.0
    assert O.tensor_s_enc(0.0) == 1.0
    assert O.tensor_s_enc(1.0) == np.float32(2688.0)
    assert np.float32(O.tensor_s_enc(3.0)) == np.float32(2688.0) / np.float32(3.0)
    # The largest block scale of any tensor maps to (at most) 448.
    for amax in [1e-3, 0.37, 1.0, 6.0, 17.25, 1e4]:
        s = O.tensor_s_enc(amax)
        assert O.block_scale_code(amax, s) == 0x7E


def test_block_scale_floor_is_one():
    # A block whose scale would round to E4M3 zero keeps code 1 (2^-9).
    assert O.block_scale_code(0.0, 1.0) == 1
    assert O.block_scale_code(1e-6, 1.0) == 1


def test_e8m0_rule():
    p = golden("pow2_scale_example")
    k = O.e8m0_k_for(p["amax"], p["elem_max"])
    assert 2.0 ** k == p["scale"]
    # Exact boundaries: amax = 448 * 2^k needs exactly 2^k; one ulp more needs 2^(k+1).
    for k in [-20, -3, 0, 1, 7, 30]:
        a = np.float32(448.0 * 2.0 ** k)
        assert O.e8m0_k(a)[()] == k
        assert O.e8m0_k(np.nextafter(a, np.float32(np.inf)))[()] == k + 1
    assert O.e8m0_k(np.float32(0.0))[()] == -127
    # Away from boundaries the rule is ceil(log2(amax / 448)).
    rng = np.random.default_rng(0)
    a = (10.0 ** rng.uniform(-20, 20, 20000)).astype(np.float32)
    ref = np.ceil(np.log2(a.astype(np.float64) / 448.0)).astype(np.int64)
    got = O.e8m0_k(a)
    frac = np.log2(a.astype(np.float64) / 448.0) % 1.0
    safe = (frac > 1e-6) & (frac < 1 - 1e-6)
    assert np.array_equal(got[safe], ref[safe])

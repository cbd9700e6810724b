"""GEMMs with the NVFP4 quantize in their epilogue (4bit.vizuara.ai, section
13; End-to-End 4-Bit Training, kernels for low-precision training).

The epilogue encodes the BF16 value the plain GEMM would store (and GELU of
it), so its result is the BF16 GEMM followed by the quantizer.  Where the
FP32 products are exact (integer-valued codes with unit block scales and
power-of-two decode scales) the codes, scales, decode scale and output amax
must equal the oracle's encode of the exact product (rounded to BF16) bit for
bit, with and without GELU.  Elsewhere the FP32 sum order is free, so a
value near a rounding boundary may round either way (two correct results,
4bit.vizuara.ai section 13).  There every block that differs from the
oracle's encode of the FP64 product must be the oracle's encode of a BF16
row the FP32 accumulation could have produced: each value inside the BF16
rounding of [y - E, y + E], E the accumulation bound (K + 4) 2^-24 sum |a b|
(gpu_util.accumulation_bound).  No block may be left unexplained.
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import (accumulation_bound, announce, bf16_from_key, bf16_window, dev, host,
                      to_dev, upload_nvfp4)
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _unit_scale_operand(R, K, seed, s_dec, tile2d=False):
    rng = np.random.default_rng(seed)
    shape = (R // 16, K // 16) if tile2d else (R, K // 16)
    return O.NVFP4(rng.integers(0, 256, (R, K // 2), dtype=np.uint8),
                   np.full(shape, 0x38, np.uint8), np.float32(s_dec), R, K, tile2d)


def _ref(a, b, gelu):
    y = O.bf16_rne(O.gemm_f64(a.dequant_f64(), b.dequant_f64())).astype(np.float32)
    return O.gelu_f32(y) if gelu else y


def _run(bbs, a, b, s_enc, gelu, M, N):
    Y = bbs.NVFP4Tensor.empty(M, N, device=dev())
    se = torch.tensor([s_enc], dtype=torch.float32, device=dev())
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=dev())
    bbs.nvfp4_gemm_quant(a, b, se, Y, gelu=gelu, amax=amax)
    torch.cuda.synchronize()
    return Y, float(host(amax)[0])


@pytest.mark.parametrize("gelu", [False, True])
@pytest.mark.parametrize("M,N,K,tb", [(272, 400, 1024, True), (128, 256, 128, False),
                                      (304, 16, 256, True)])
def test_exact_case(bbs, gelu, M, N, K, tb):
    announce(f"quantizing GEMM, exact products M={M} N={N} K={K} gelu={gelu}")
    a = _unit_scale_operand(M, K, M + K, 0.5)
    b = _unit_scale_operand(N, K, N + K, 0.25, tb)
    y = _ref(a, b, gelu)
    amax = float(np.abs(y).max())
    s_enc = O.tensor_s_enc(amax)
    Y, got_amax = _run(bbs, upload_nvfp4(a, bbs), upload_nvfp4(b, bbs), s_enc, gelu, M, N)
    o = O.nvfp4_encode_f32(y, s_enc)
    assert np.array_equal(host(Y.scales), o.scales)
    assert np.array_equal(host(Y.codes), o.codes)
    assert host(Y.s_dec)[0] == o.s_dec
    assert got_amax == amax


@pytest.mark.parametrize("gelu", [False, True])
def test_per_token_A_exact(bbs, gelu):
    """A with a decode scale per row (the per-token activation copy): each
    output row is scaled by its own row's s_dec before the BF16 rounding,
    GELU and the encode.  Power-of-two row scales keep every product exact."""
    announce(f"quantizing GEMM, per-row A decode scales, exact products, gelu={gelu}")
    M, N, K = 272, 288, 512
    a = _unit_scale_operand(M, K, 93, 1.0)
    s_rows = np.float32(2.0) ** -(np.arange(M) % 5).astype(np.float32)
    ar = O.NVFP4Rows(a.codes, a.scales, s_rows, M, K)
    b = _unit_scale_operand(N, K, 94, 0.5, True)
    y = O.bf16_rne(O.gemm_f64(ar.dequant_f64(), b.dequant_f64())).astype(np.float32)
    if gelu:
        y = O.gelu_f32(y)
    amax = float(np.abs(y).max())
    s_enc = O.tensor_s_enc(amax)
    A = bbs.NVFP4Tensor(to_dev(a.codes), to_dev(a.scales), to_dev(s_rows), M, K, False, True)
    Y, got_amax = _run(bbs, A, upload_nvfp4(b, bbs), s_enc, gelu, M, N)
    o = O.nvfp4_encode_f32(y, s_enc)
    assert np.array_equal(host(Y.scales), o.scales)
    assert np.array_equal(host(Y.codes), o.codes)
    assert got_amax == amax


def test_saturating_scale(bbs):
    """An encode scale chosen for a smaller amax (a stale one) saturates the
    block scale at 448, exactly as the oracle's encode does."""
    announce("quantizing GEMM with a stale (too large) encode scale")
    a = _unit_scale_operand(128, 256, 5, 1.0)
    b = _unit_scale_operand(128, 256, 6, 1.0, True)
    y = _ref(a, b, False)
    s_enc = O.tensor_s_enc(float(np.abs(y).max()) / 8)
    Y, _ = _run(bbs, upload_nvfp4(a, bbs), upload_nvfp4(b, bbs), s_enc, False, 128, 128)
    o = O.nvfp4_encode_f32(y, s_enc)
    assert (host(Y.scales) == 0x7E).any()
    assert np.array_equal(host(Y.scales), o.scales)
    assert np.array_equal(host(Y.codes), o.codes)


def _explain_blocks(codes, scales, y64, E, s_enc, gelu):
    """Blocks of the GPU's 1x16 NVFP4 output (codes, scales: rows x N/2,
    rows x N/16) against the oracle: returns (differing blocks, unexplained
    blocks).  A differing block is explained when some admissible BF16 row
    (each value within the BF16 rounding of [y64 - E, y64 + E], GELU of it
    with `gelu`) encodes to exactly the GPU's scale code and 16 codes: every
    code must be the nearest-even E2M1 code of an admissible value times the
    block's encode scale, and the scale code must be that of a block maximum
    the admissible values can reach."""
    f_ref = O.bf16_rne(y64).astype(np.float32)
    if gelu:
        f_ref = O.gelu_f32(f_ref)
    o = O.nvfp4_encode_f32(f_ref, s_enc)
    R, N = y64.shape
    nb = N // 16
    diff = (scales != o.scales) | (codes.reshape(R, nb, 8) != o.codes.reshape(R, nb, 8)).any(axis=2)
    s_dec = np.float32(1.0) / np.float32(s_enc)
    unexplained = 0
    for m, b in zip(*np.nonzero(diff)):
        lo, hi = bf16_window(y64[m, 16 * b:16 * b + 16], E[m, 16 * b:16 * b + 16])
        sc = int(scales[m, b])
        s_b = np.float32(1.0) / (np.float32(O.e4m3_value(sc)) * s_dec)
        cb = codes[m, 8 * b:8 * b + 8]
        want = np.stack([cb & 0xF, cb >> 4], axis=1).reshape(16)
        allowed = []
        for i in range(16):
            h = bf16_from_key(np.arange(lo[i], hi[i] + 1))
            v = (h.astype(np.uint32) << 16).view(np.float32)
            if gelu:
                v = O.gelu_f32(v)
            c = O.e2m1_code(O.round_to(v * s_b, O.E2M1, O.RTN))
            allowed.append(np.abs(v[c == want[i]]))
        if any(a.size == 0 for a in allowed):
            unexplained += 1
            continue
        floor = max(float(a.min()) for a in allowed)
        maxima = np.unique(np.concatenate([a[a >= floor] for a in allowed]))
        if not any(O.block_scale_code(float(mx), float(s_enc)) == sc for mx in maxima):
            unexplained += 1
    return int(diff.sum()), unexplained


def _amax_window(y64, E, gelu):
    """Bounds on the max |value| an admissible BF16 output (GELU of it with
    `gelu`) can have, from each window's end points: a window holding 0 can
    give 0; GELU is non-decreasing for x >= 0 and below 0.171875 in
    magnitude for x < 0 (the oracle's GELU pins), so a window reaching below
    0 can give at most 0.171875 there and, wholly below 0, is bounded below
    by 0 only."""
    lo, hi = bf16_window(y64.ravel(), E.ravel())
    a = (bf16_from_key(lo).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b = (bf16_from_key(hi).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if not gelu:
        small = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(a), np.abs(b)))
        big = np.maximum(np.abs(a), np.abs(b))
    else:
        ga, gb = O.gelu_f32(a.astype(np.float32)), O.gelu_f32(b.astype(np.float32))
        small = np.where(lo > 0, np.abs(ga), 0.0)
        big = np.where(hi > 0, np.abs(gb), 0.0)
        big = np.where(lo < 0, np.maximum(big, 0.171875), big)
    return float(small.max()), float(big.max())


@pytest.mark.parametrize("gelu", [False, True])
def test_general_operands(bbs, gelu):
    announce(f"quantizing GEMM, quantized X / W operands gelu={gelu}")
    x = synth.normal_with_outliers(256, 1024, 90)
    w = synth.normal(384, 1024, 91, 0.05)
    ox, ow = O.nvfp4_quantize(x), O.nvfp4_quantize(w, tile2d=True)
    y = _ref(ox, ow, gelu)
    s_enc = O.tensor_s_enc(float(np.abs(y).max()))
    Y, got_amax = _run(bbs, upload_nvfp4(ox, bbs), upload_nvfp4(ow, bbs), s_enc, gelu, 256, 384)
    A64, B64 = ox.dequant_f64(), ow.dequant_f64()
    y64 = O.gemm_f64(A64, B64)
    E = accumulation_bound(O.gemm_f64(np.abs(A64), np.abs(B64)), 1024)
    n_diff, n_bad = _explain_blocks(host(Y.codes), host(Y.scales), y64, E, s_enc, gelu)
    print(f"  {n_diff} of {256 * 24} blocks differ from the encode of RN(y), {n_bad} unexplained")
    assert n_bad == 0
    lo, hi = _amax_window(y64, E, gelu)
    assert lo <= got_amax <= hi, (lo, got_amax, hi)


def test_grouped_exact_case(bbs):
    """The grouped (MoE) GEMM with the row gather and per-expert decode
    scales, exact products, GELU + quantize in the epilogue."""
    announce("quantizing grouped GEMM, exact products, GELU")
    G, N, K, T = 4, 128, 256, 96
    a = _unit_scale_operand(T, K, 40, 0.5)
    rng = np.random.default_rng(41)
    counts = np.array([40, 0, 100, 52])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(offsets[-1])
    row_index = rng.integers(0, T, rows).astype(np.int32)
    ws = [_unit_scale_operand(N, K, 50 + g, 2.0 ** -(g + 1), True) for g in range(G)]
    y = np.zeros((rows, N), np.float32)
    A64 = a.dequant_f64()
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        y[r0:r1] = O.bf16_rne(O.gemm_f64(A64[row_index[r0:r1]], ws[g].dequant_f64()))
    y = O.gelu_f32(y)
    s_enc = O.tensor_s_enc(float(np.abs(y).max()))
    B = bbs.NVFP4Tensor.empty(G * N, K, tile2d=True, n_scales=G, device=dev())
    for g in range(G):
        B.codes[g * N:(g + 1) * N] = to_dev(ws[g].codes)
        B.scales[g * N // 16:(g + 1) * N // 16] = to_dev(ws[g].scales)
        B.s_dec[g] = float(ws[g].s_dec)
    Y = bbs.NVFP4Tensor.empty(rows, N, device=dev())
    se = torch.tensor([s_enc], dtype=torch.float32, device=dev())
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    bbs.grouped_nvfp4_gemm_quant(upload_nvfp4(a, bbs), to_dev(row_index), to_dev(offsets), G, rows,
                                 B, N, se, Y, gelu=True, amax=amax)
    torch.cuda.synchronize()
    o = O.nvfp4_encode_f32(y, s_enc)
    assert np.array_equal(host(Y.scales), o.scales)
    assert np.array_equal(host(Y.codes), o.codes)
    assert float(host(amax)[0]) == float(np.abs(y).max())


def test_full_size_sampled(bbs):
    """The dense forward 8192 x 14336 x 4096 with GELU + quantize in the
    epilogue, in the configuration bench.py times: sampled rows against the
    oracle's encode of the FP64 product."""
    announce("quantizing GEMM 8192x14336x4096 + GELU (sampled rows)")
    d = synth.dense_forward()
    ox, ow = O.nvfp4_quantize(d["x"]), O.nvfp4_quantize(d["w"], tile2d=True)
    rows = np.sort(np.random.default_rng(3).choice(8192, 48, replace=False))
    rows[-1] = 8191
    sub = O.NVFP4(np.ascontiguousarray(ox.codes[rows]), np.ascontiguousarray(ox.scales[rows]),
                  ox.s_dec, len(rows), 4096, False)
    A64, B64 = sub.dequant_f64(), ow.dequant_f64()
    y64 = O.gemm_f64(A64, B64)
    E = accumulation_bound(O.gemm_f64(np.abs(A64), np.abs(B64)), 4096)
    s_enc = O.tensor_s_enc(40.0)
    xq, wq = upload_nvfp4(ox, bbs), upload_nvfp4(ow, bbs)
    Y, got_amax = _run(bbs, xq, wq, s_enc, True, 8192, 14336)
    ridx = torch.from_numpy(rows).to(dev())
    n_diff, n_bad = _explain_blocks(host(Y.codes[ridx]), host(Y.scales[ridx]), y64, E, s_enc, True)
    print(f"  {n_diff} of {len(rows) * 896} sampled blocks differ from the encode of RN(y), "
          f"{n_bad} unexplained")
    assert n_bad == 0
    assert got_amax >= _amax_window(y64, E, True)[0]
    # at full size, beside the oracle check above: the fused kernel equals the
    # library's BF16 GEMM followed by its fused GELU quantizer (whose amax
    # pass finds the same amax) bit for bit, the header's promise
    h = torch.empty((8192, 14336), dtype=torch.int16, device=dev())
    bbs.nvfp4_gemm(bbs.FMT_NVFP4, xq, wq, h, bbs.OUT_BF16)
    U = bbs.NVFP4Tensor.empty(8192, 14336, device=dev())
    bbs.nvfp4_quantize(h, U, gelu=True)
    Y2, amax2 = _run(bbs, xq, wq, np.float32(2688.0) / np.float32(got_amax), True, 8192, 14336)
    assert amax2 == got_amax
    torch.cuda.synchronize()
    assert torch.equal(U.s_dec, Y2.s_dec)
    assert torch.equal(U.scales, Y2.scales)
    assert torch.equal(U.codes, Y2.codes)


def test_grouped_dropped_slots(bbs):
    """Dropped slots (row_index < 0 or >= A.rows) of the quantizing grouped
    GEMM are encoded as zero rows and leave the reported amax unchanged."""
    announce("quantizing grouped GEMM with dropped slots, GELU")
    G, N, K, T = 3, 128, 256, 64
    a = _unit_scale_operand(T, K, 42, 0.5)
    counts = np.array([40, 0, 72])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(offsets[-1])
    rng = np.random.default_rng(43)
    row_index = rng.integers(0, T, rows).astype(np.int32)
    drop = rng.choice(rows, 20, replace=False)
    row_index[drop[:10]] = -3
    row_index[drop[10:]] = T + 7
    ws = [_unit_scale_operand(N, K, 55 + g, 2.0 ** -(g + 1), True) for g in range(G)]
    y = np.zeros((rows, N), np.float32)
    A64 = a.dequant_f64()
    for g in range(G):
        for i in range(offsets[g], offsets[g + 1]):
            if 0 <= row_index[i] < T:
                y[i] = O.bf16_rne(A64[row_index[i]] @ ws[g].dequant_f64().T)
    y = O.gelu_f32(y)
    s_enc = O.tensor_s_enc(float(np.abs(y).max()))
    B = bbs.NVFP4Tensor.empty(G * N, K, tile2d=True, n_scales=G, device=dev())
    for g in range(G):
        B.codes[g * N:(g + 1) * N] = to_dev(ws[g].codes)
        B.scales[g * N // 16:(g + 1) * N // 16] = to_dev(ws[g].scales)
        B.s_dec[g] = float(ws[g].s_dec)
    Y = bbs.NVFP4Tensor.empty(rows, N, device=dev())
    se = torch.tensor([s_enc], dtype=torch.float32, device=dev())
    amax = torch.zeros(1, dtype=torch.float32, device=dev())
    bbs.grouped_nvfp4_gemm_quant(upload_nvfp4(a, bbs), to_dev(row_index), to_dev(offsets), G, rows,
                                 B, N, se, Y, gelu=True, amax=amax)
    torch.cuda.synchronize()
    o = O.nvfp4_encode_f32(y, s_enc)
    assert np.array_equal(host(Y.scales), o.scales)
    assert np.array_equal(host(Y.codes), o.codes)
    assert float(host(amax)[0]) == float(np.abs(y).max())

"""GEMMs with the combine wire format encode in the epilogue (4bit.vizuara.ai,
section 11; End-to-End 4-Bit Training, "quantized communication"): the
experts' down projection writes its output as RHT-32 + S2F6 directly.

The epilogue encodes the BF16 value the plain GEMM would store, so its result
is the BF16 GEMM followed by the combine encode.  With integer-valued codes,
unit block scales and power-of-two decode scales every FP32 product and sum
is exact, so codes and scales must equal the oracle's encode of the exact
product (rounded to BF16) bit for bit, at small sizes and on sampled rows of
the full MoE down projection (524288 routed rows x 4096, K = 1536, 64
experts), where the fused kernel must also equal the library's own unfused
GEMM + encode bit for bit.
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import announce, dev, host, to_dev, upload_nvfp4
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SIGNS = 0xB5297A4D


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _unit_scale_operand(R, K, seed, s_dec, tile2d=False):
    rng = np.random.default_rng(seed)
    shape = (R // 16, K // 16) if tile2d else (R, K // 16)
    return O.NVFP4(rng.integers(0, 256, (R, K // 2), dtype=np.uint8),
                   np.full(shape, 0x38, np.uint8), np.float32(s_dec), R, K, tile2d)


def _same(Y, o, what):
    assert np.array_equal(host(Y.scales), o.scales), f"{what}: scales differ"
    g = host(Y.codes)
    if not np.array_equal(g, o.codes):
        bad = np.argwhere(g != o.codes)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {bad[0].tolist()}")


@pytest.mark.parametrize("rht", [True, False])
@pytest.mark.parametrize("M,N,K", [(272, 416, 1024), (128, 256, 128), (48, 32, 256)])
def test_exact_case(bbs, rht, M, N, K):
    announce(f"encoding GEMM, exact products M={M} N={N} K={K} rht={rht}")
    a = _unit_scale_operand(M, K, M + K, 0.5)
    b = _unit_scale_operand(N, K, N + K + 1, 0.125, True)
    y = O.bf16_rne(O.gemm_f64(a.dequant_f64(), b.dequant_f64())).astype(np.float32)
    Y = bbs.S2F6Tensor.empty(M, N, device=dev())
    bbs.nvfp4_gemm_s2f6(upload_nvfp4(a, bbs), upload_nvfp4(b, bbs), Y, rht=rht, signs=SIGNS)
    torch.cuda.synchronize()
    _same(Y, O.s2f6_encode_f32(y, rht=rht, signs=SIGNS), "dense")


def test_per_token_A_exact(bbs):
    """A with a decode scale per row (the per-token activation copy): each
    output row is scaled by its own row's s_dec before the BF16 rounding and
    the encode.  Power-of-two row scales keep every product exact."""
    announce("encoding GEMM, per-row A decode scales, exact products")
    M, N, K = 272, 288, 512
    a = _unit_scale_operand(M, K, 91, 1.0)
    s_rows = np.float32(2.0) ** -(np.arange(M) % 5).astype(np.float32)
    ar = O.NVFP4Rows(a.codes, a.scales, s_rows, M, K)
    b = _unit_scale_operand(N, K, 92, 0.5, True)
    y = O.bf16_rne(O.gemm_f64(ar.dequant_f64(), b.dequant_f64())).astype(np.float32)
    A = bbs.NVFP4Tensor(to_dev(a.codes), to_dev(a.scales), to_dev(s_rows), M, K, False, True)
    Y = bbs.S2F6Tensor.empty(M, N, device=dev())
    bbs.nvfp4_gemm_s2f6(A, upload_nvfp4(b, bbs), Y, rht=True, signs=SIGNS)
    torch.cuda.synchronize()
    _same(Y, O.s2f6_encode_f32(y, rht=True, signs=SIGNS), "per-row A")


def test_grouped_exact_case(bbs):
    """Row gather, empty and ragged groups, per-expert decode scales."""
    announce("encoding grouped GEMM, exact products")
    G, N, K, T = 4, 96, 256, 80
    a = _unit_scale_operand(T, K, 60, 0.25)
    counts = np.array([36, 0, 97, 20])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(offsets[-1])
    row_index = np.random.default_rng(61).integers(0, T, rows).astype(np.int32)
    ws = [_unit_scale_operand(N, K, 70 + g, 2.0 ** -(g + 2), True) for g in range(G)]
    A64 = a.dequant_f64()
    y = np.zeros((rows, N), np.float32)
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        y[r0:r1] = O.bf16_rne(O.gemm_f64(A64[row_index[r0:r1]], ws[g].dequant_f64()))
    B = bbs.NVFP4Tensor.empty(G * N, K, tile2d=True, n_scales=G, device=dev())
    for g in range(G):
        B.codes[g * N:(g + 1) * N] = to_dev(ws[g].codes)
        B.scales[g * N // 16:(g + 1) * N // 16] = to_dev(ws[g].scales)
        B.s_dec[g] = float(ws[g].s_dec)
    Y = bbs.S2F6Tensor.empty(rows, N, device=dev())
    bbs.grouped_nvfp4_gemm_s2f6(upload_nvfp4(a, bbs), to_dev(row_index), to_dev(offsets), G, rows,
                                B, N, Y, rht=True, signs=SIGNS)
    torch.cuda.synchronize()
    _same(Y, O.s2f6_encode_f32(y, rht=True, signs=SIGNS), "grouped")


def test_full_moe_down_projection(bbs):
    """The MoE down projection as bench.py times it (524288 routed rows,
    1536 -> 4096, 64 experts of 16x16-scaled NVFP4 weights, Zipf top-8
    routing): exact products, sampled rows of three experts against the
    oracle, and the whole output against the unfused GEMM + encode."""
    announce("encoding grouped GEMM, full MoE down projection 524288x4096x1536")
    T, H, F, E, KT = 65536, 4096, 1536, 64, 8
    _, offsets = synth.moe_routing(T, E, KT, 502)
    rows = int(offsets[-1])
    gen = torch.Generator(device=dev()).manual_seed(77)
    A = bbs.NVFP4Tensor.empty(rows, F, device=dev())
    A.codes.copy_(torch.randint(0, 256, A.codes.shape, dtype=torch.uint8, device=dev(),
                                generator=gen))
    A.scales.fill_(0x38)
    A.s_dec.fill_(0.5)
    W = bbs.NVFP4Tensor.empty(E * H, F, tile2d=True, n_scales=E, device=dev())
    W.codes.copy_(torch.randint(0, 256, W.codes.shape, dtype=torch.uint8, device=dev(),
                                generator=gen))
    W.scales.fill_(0x38)
    W.s_dec.copy_(torch.tensor([2.0 ** -(g % 5) for g in range(E)], device=dev()))
    off = to_dev(offsets)
    Y = bbs.S2F6Tensor.empty(rows, H, device=dev())
    bbs.grouped_nvfp4_gemm_s2f6(A, None, off, E, rows, W, H, Y, rht=True, signs=SIGNS)
    h = torch.empty((rows, H), dtype=torch.int16, device=dev())
    bbs.grouped_nvfp4_gemm(A, None, off, E, rows, W, H, h, bbs.OUT_BF16)
    U = bbs.S2F6Tensor.empty(rows, H, device=dev())
    bbs.s2f6_quantize(h, U, rht=True, signs=SIGNS)
    torch.cuda.synchronize()
    assert torch.equal(Y.scales, U.scales)
    assert torch.equal(Y.codes, U.codes)
    del h, U
    counts = np.diff(offsets)
    busy = [int(g) for g in np.argsort(-counts)[:2]] + [int(np.flatnonzero(counts)[-1])]
    for g in busy:
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        pick = np.unique(np.concatenate([[r0, r1 - 1], np.random.default_rng(g).integers(r0, r1, 14)]))
        ridx = torch.from_numpy(pick).to(dev())
        a = O.NVFP4(host(A.codes[ridx]), host(A.scales[ridx]), np.float32(0.5), len(pick), F, False)
        w = O.NVFP4(host(W.codes[g * H:(g + 1) * H]), host(W.scales[g * H // 16:(g + 1) * H // 16]),
                    np.float32(2.0 ** -(g % 5)), H, F, True)
        y = O.bf16_rne(O.gemm_f64(a.dequant_f64(), w.dequant_f64())).astype(np.float32)
        o = O.s2f6_encode_f32(y, rht=True, signs=SIGNS)
        assert np.array_equal(host(Y.scales[ridx]), o.scales), f"expert {g}: scales differ"
        assert np.array_equal(host(Y.codes[ridx]), o.codes), f"expert {g}: codes differ"


def test_grouped_dropped_slots(bbs):
    """Dropped slots of the encoding grouped GEMM come out as the encode of
    a zero row (scale byte 0, codes 0)."""
    announce("encoding grouped GEMM with dropped slots")
    G, N, K, T = 3, 96, 256, 48
    a = _unit_scale_operand(T, K, 62, 0.25)
    counts = np.array([30, 50, 0])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(offsets[-1])
    rng = np.random.default_rng(63)
    row_index = rng.integers(0, T, rows).astype(np.int32)
    drop = rng.choice(rows, 16, replace=False)
    row_index[drop[:8]] = -1
    row_index[drop[8:]] = T
    ws = [_unit_scale_operand(N, K, 72 + g, 2.0 ** -(g + 2), True) for g in range(G)]
    A64 = a.dequant_f64()
    y = np.zeros((rows, N), np.float32)
    for g in range(G):
        for i in range(offsets[g], offsets[g + 1]):
            if 0 <= row_index[i] < T:
                y[i] = O.bf16_rne(A64[row_index[i]] @ ws[g].dequant_f64().T)
    B = bbs.NVFP4Tensor.empty(G * N, K, tile2d=True, n_scales=G, device=dev())
    for g in range(G):
        B.codes[g * N:(g + 1) * N] = to_dev(ws[g].codes)
        B.scales[g * N // 16:(g + 1) * N // 16] = to_dev(ws[g].scales)
        B.s_dec[g] = float(ws[g].s_dec)
    Y = bbs.S2F6Tensor.empty(rows, N, device=dev())
    bbs.grouped_nvfp4_gemm_s2f6(upload_nvfp4(a, bbs), to_dev(row_index), to_dev(offsets), G, rows,
                                B, N, Y, rht=True, signs=SIGNS)
    torch.cuda.synchronize()
    _same(Y, O.s2f6_encode_f32(y, rht=True, signs=SIGNS), "grouped dropped slots")

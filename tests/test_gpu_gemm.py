"""GPU parity of the block-scaled GEMMs against the oracle's FP64 accumulation.

Operands are produced by the oracle (or drawn at random), uploaded byte for
byte, and multiplied on the GPU; the reference is the FP64 sum over the same
dequantized operands.  Bar: relative Frobenius error <= 1e-3 (FP32 output
against the raw FP64 sum; BF16 output against the FP64 sum rounded to BF16).
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import (accumulation_bound, announce, bf16_bits_to_f64, check_bounded_outputs, dev,
                      host, tile_samples, to_dev, upload_mxfp8, upload_nvfp4)
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 1e-3


@pytest.fixture(scope="module")
def bbs():
    import bit_block_scaled_amd as b
    return b


def _run_gemm(bbs, fmt, a, b, M, N, bf16):
    c = torch.empty((M, N), dtype=torch.int16 if bf16 else torch.float32, device=dev())
    bbs.nvfp4_gemm(fmt, a, b, c, bbs.OUT_BF16 if bf16 else bbs.OUT_F32)
    torch.cuda.synchronize()
    y = host(c)
    return bf16_bits_to_f64(y.view(np.uint16)) if bf16 else y.astype(np.float64)


def _check(y, ref, bf16, what):
    r = O.bf16_rne(ref) if bf16 else ref
    err = O.rel_fro(y, r)
    print(f"  {what}: rel err {err:.3e}", flush=True)
    assert err <= TOL, f"{what}: relative error {err}"
    return err


def _random_nvfp4(R, C, seed, tile2d=False, s_dec=0.5):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    shape = (R // 16, C // 16) if tile2d else (R, C // 16)
    scales = rng.integers(1, 0x7F, size=shape, dtype=np.uint8)
    return O.NVFP4(codes, scales, np.float32(s_dec), R, C, tile2d)


def test_tiny_linear(bbs):
    announce("tiny linear 256^3, 1x16 X, 16x16 W, FP32 out")
    d = synth.tiny_linear()
    ox = O.nvfp4_quantize(d["x"])
    ow = O.nvfp4_quantize(d["w"], tile2d=True)
    y = _run_gemm(bbs, bbs.FMT_NVFP4, upload_nvfp4(ox, bbs), upload_nvfp4(ow, bbs), 256, 256,
                  False)
    err = _check(y, O.gemm_f64(ox.dequant_f64(), ow.dequant_f64()), False, "tiny")
    assert err < 1e-5


def test_integer_case_bit_exact(bbs):
    # all block scales 1.0 (0x38) and s_dec = 1: every partial sum is a
    # multiple of 1/4 below 2^22, so FP32 accumulation is exact.
    announce("integer special case, exact")
    rng = np.random.default_rng(11)
    M, N, K = 64, 96, 256
    a = O.NVFP4(rng.integers(0, 256, (M, K // 2), dtype=np.uint8),
                np.full((M, K // 16), 0x38, np.uint8), np.float32(1), M, K, False)
    b = O.NVFP4(rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
                np.full((N // 16, K // 16), 0x38, np.uint8), np.float32(1), N, K, True)
    y = _run_gemm(bbs, bbs.FMT_NVFP4, upload_nvfp4(a, bbs), upload_nvfp4(b, bbs), M, N, False)
    assert np.array_equal(y, O.gemm_f64(a.dequant_f64(), b.dequant_f64()))


@pytest.mark.parametrize("M,N,K,ta,tb,bf16", [
    (16, 16, 16, False, False, False),       # one block
    (144, 80, 80, False, True, False),       # ragged M/N, K not a multiple of the K slab
    (272, 272, 528, True, True, True),       # tile2d on both sides, BF16 out
    (272, 400, 1040, False, True, True),
    (48, 528, 4096, False, False, False),
    (272, 400, 1024, True, True, True),      # large-tile path, ragged M and N
    (528, 272, 512, False, False, False),
    (16, 4112, 128, False, True, True),
])
def test_random_operands(bbs, M, N, K, ta, tb, bf16):
    announce(f"random NVFP4 operands M={M} N={N} K={K} tile2d=({ta},{tb}) bf16={bf16}")
    a = _random_nvfp4(M, K, M + K, ta, 0.25)
    b = _random_nvfp4(N, K, N + 3 * K, tb, 0.125)
    y = _run_gemm(bbs, bbs.FMT_NVFP4, upload_nvfp4(a, bbs), upload_nvfp4(b, bbs), M, N, bf16)
    _check(y, O.gemm_f64(a.dequant_f64(), b.dequant_f64()), bf16, "random")


def _sampled_check(y_full, A64, B64, bf16, what, per_tile=4, seed=0):
    """Sampled outputs of a full-size GEMM: per_tile outputs inside every
    256 x 256 output tile, the whole last row and 2048 more at random, each
    held to its accumulation bound against the FP64 sum (gpu_util); prints
    the global relative error and the worst tile."""
    M, N = y_full.shape
    rows, cols, tiles = tile_samples(M, N, per_tile, seed, extra=2048)
    y64 = O.gemm_f64_sampled(A64, B64, rows, cols)
    E = accumulation_bound(O.gemm_f64_sampled(np.abs(A64), np.abs(B64), rows, cols),
                           A64.shape[1])
    return check_bounded_outputs(y_full[rows, cols], y64, E, bf16, what, tiles)


def test_full_dense_forward(bbs):
    announce("dense forward 8192x14336x4096, BF16 out (sampled outputs)")
    d = synth.dense_forward()
    ox = O.nvfp4_quantize(d["x"])
    ow = O.nvfp4_quantize(d["w"], tile2d=True)
    y = _run_gemm(bbs, bbs.FMT_NVFP4, upload_nvfp4(ox, bbs), upload_nvfp4(ow, bbs), 8192, 14336,
                  True)
    _sampled_check(y, ox.dequant_f64(), ow.dequant_f64(), True, "fprop")


def test_full_wgrad(bbs):
    announce("wgrad 14336x4096x8192 (RHT'd column copies), FP32 out (sampled)")
    fw, bw = synth.dense_forward(), synth.backward()
    s, seeds = bw["rht_signs"], bw["seeds"]
    og = O.nvfp4_quantize(bw["dy"], transpose=True, rht=True, signs=s, mode=O.SR,
                          seed=seeds["dy_col"])
    ox = O.nvfp4_quantize(fw["x"], transpose=True, rht=True, signs=s, mode=O.SR,
                          seed=seeds["x_col"])
    y = _run_gemm(bbs, bbs.FMT_NVFP4, upload_nvfp4(og, bbs), upload_nvfp4(ox, bbs), 14336, 4096,
                  False)
    _sampled_check(y, og.dequant_f64(), ox.dequant_f64(), False, "wgrad")


# ---------------------------------------------------------------------------
# MXFP8 (dgrad)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(32, 32, 32), (144, 80, 96), (256, 256, 512), (80, 272, 1056),
                                   # large-tile kernel: one, two and three slabs, ragged tiles
                                   # (M = 300: a row group of the last tile only partly in A)
                                   (256, 256, 128), (272, 400, 256), (528, 272, 384),
                                   (300, 208, 256)])
def test_mxfp8_small(bbs, M, N, K):
    announce(f"MXFP8 GEMM M={M} N={N} K={K}")
    a = O.mxfp8_quantize(synth.laplace(M, K, M + K, 1e-3), mode=O.SR, seed=1)
    w = O.nvfp4_quantize(synth.normal(K, N, N + K, 0.02), tile2d=True)
    b = O.mxfp8_requantize_t(w, mode=O.SR, seed=2)            # N x K
    for bf16 in (False, True):
        y = _run_gemm(bbs, bbs.FMT_MXFP8, upload_mxfp8(a, bbs), upload_mxfp8(b, bbs), M, N, bf16)
        _check(y, O.gemm_f64(a.dequant_f64(), b.dequant_f64()), bf16, "mxfp8")


def test_full_dgrad(bbs):
    announce("dgrad 8192x4096x14336 MXFP8, BF16 out (sampled)")
    fw, bw = synth.dense_forward(), synth.backward()
    seeds = bw["seeds"]
    og = O.mxfp8_quantize(bw["dy"], mode=O.SR, seed=seeds["dy_mx8"])
    ow = O.mxfp8_requantize_t(O.nvfp4_quantize(fw["w"], tile2d=True), mode=O.SR,
                              seed=seeds["w_req"])
    y = _run_gemm(bbs, bbs.FMT_MXFP8, upload_mxfp8(og, bbs), upload_mxfp8(ow, bbs), 8192, 4096,
                  True)
    _sampled_check(y, og.dequant_f64(), ow.dequant_f64(), True, "dgrad")


# ---------------------------------------------------------------------------
# Grouped (MoE)
# ---------------------------------------------------------------------------

def _grouped_case(bbs, tokens, hidden, ffn, experts, sizes, gather, bf16, seed, row_index=None):
    rng = np.random.default_rng(seed)
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    total = int(offsets[-1])
    if not gather:                       # A holds the routed rows themselves
        tokens = max(16, (total + 15) // 16 * 16)
    x = synth.normal_with_outliers(tokens, hidden, seed)
    ox = O.nvfp4_quantize(x)
    if gather and row_index is None:
        row_index = rng.integers(0, tokens, total).astype(np.int32)
    ws = [O.nvfp4_quantize(w, tile2d=True) for w in synth.moe_weights(experts, ffn, hidden, seed + 1)]
    codes = np.concatenate([w.codes for w in ws])
    scales = np.concatenate([w.scales for w in ws])
    sdec = np.array([w.s_dec for w in ws], np.float32)
    B = O.NVFP4(codes, scales, np.float32(0), experts * ffn, hidden, True)
    bd = upload_nvfp4(B, bbs, n_scales=sdec)
    ad = upload_nvfp4(ox, bbs)
    c = torch.full((max(total, 1), ffn), -1, dtype=torch.int16 if bf16 else torch.float32,
                   device=dev())
    bbs.grouped_nvfp4_gemm(ad, to_dev(row_index) if gather else None, to_dev(offsets), experts,
                           total, bd, ffn, c, bbs.OUT_BF16 if bf16 else bbs.OUT_F32)
    torch.cuda.synchronize()
    y = host(c)
    y = bf16_bits_to_f64(y.view(np.uint16)) if bf16 else y.astype(np.float64)
    A64 = ox.dequant_f64()
    src = row_index if gather else np.arange(total)
    ref = np.zeros((total, ffn))
    for g in range(experts):
        r0, r1 = offsets[g], offsets[g + 1]
        if r1 > r0:
            ref[r0:r1] = O.gemm_f64(A64[src[r0:r1]], ws[g].dequant_f64())
    return y[:total], ref


@pytest.mark.parametrize("sizes,gather,bf16", [
    ([0, 5, 1, 0, 200, 131, 0, 64], True, False),
    ([128, 0, 0, 1, 257, 3], False, True),
    ([300], True, True),
])
def test_grouped_small(bbs, sizes, gather, bf16):
    experts = len(sizes)
    announce(f"grouped sizes={sizes} gather={gather} bf16={bf16}")
    y, ref = _grouped_case(bbs, 512, 256, 144, experts, np.array(sizes), gather, bf16,
                           8000 + experts)
    _check(y, ref, bf16, "grouped")


def _unit(R, K, seed, tile2d):
    rng = np.random.default_rng(seed)
    shape = (R // 16, K // 16) if tile2d else (R, K // 16)
    return O.NVFP4(rng.integers(0, 256, (R, K // 2), dtype=np.uint8),
                   np.full(shape, 0x38, np.uint8), np.float32(1), R, K, tile2d)


@pytest.mark.parametrize("K,bf16", [(128, False), (256, True), (384, False), (512, False),
                                    (512, True)])
def test_persistent_handover_exact(bbs, K, bf16):
    """More tiles than CUs (17 x 17) with one to four slabs per tile: each
    workgroup takes several tiles and copies the next tile's first slabs
    during the current tile's last ones.  Unit scales make every sum exact,
    so sampled outputs must equal the oracle bit for bit (BF16 out: its
    rounding of the exact sum)."""
    M, N = 17 * 256, 16 * 256 + 64
    announce(f"persistent GEMM hand-over M={M} N={N} K={K} bf16={bf16}")
    a, b = _unit(M, K, K + 1, False), _unit(N, K, K + 2, True)
    y = _run_gemm(bbs, bbs.FMT_NVFP4, upload_nvfp4(a, bbs), upload_nvfp4(b, bbs), M, N, bf16)
    rng = np.random.default_rng(K)
    rows = np.concatenate([rng.integers(0, M, 6000), np.arange(M), np.full(N, M - 1)])
    cols = np.concatenate([rng.integers(0, N, 6000), np.arange(M) % N, np.arange(N)])
    ref = O.gemm_f64_sampled(a.dequant_f64(), b.dequant_f64(), rows, cols)
    if bf16:
        ref = O.bf16_rne(ref)
    assert np.array_equal(y[rows, cols], ref)


def test_grouped_persistent_handover_exact(bbs):
    """The grouped kernel with more tiles than CUs at K = 256 (two slabs per
    tile): 64 experts of 300-ish rows, N = 1024, unit scales, exact."""
    announce("grouped persistent hand-over, 64 experts, K=256, N=1024")
    G, N, K = 64, 1024, 256
    sizes = np.random.default_rng(5).integers(200, 420, G)
    sizes[[3, 40]] = 0
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    rows = int(offsets[-1])
    a = _unit((rows + 15) // 16 * 16, K, 11, False)         # A rows: a multiple of 16
    ws = [_unit(N, K, 100 + g, True) for g in range(G)]
    B = O.NVFP4(np.concatenate([w.codes for w in ws]), np.concatenate([w.scales for w in ws]),
                np.float32(1), G * N, K, True)
    c = torch.empty((rows, N), dtype=torch.float32, device=dev())
    bbs.grouped_nvfp4_gemm(upload_nvfp4(a, bbs), None, to_dev(offsets), G, rows,
                           upload_nvfp4(B, bbs, n_scales=np.ones(G, np.float32)), N, c, bbs.OUT_F32)
    torch.cuda.synchronize()
    y = host(c)
    A64 = a.dequant_f64()
    for g in [0, 1, 2, 39, 41, 63]:
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        ref = O.gemm_f64(A64[r0:r1], ws[g].dequant_f64())
        assert np.array_equal(y[r0:r1].astype(np.float64), ref), f"expert {g}"


def test_grouped_routed_medium(bbs):
    announce("grouped, Zipf top-8 routing, 2048 tokens, 64 experts, 512 -> 192")
    row_index, offsets = synth.moe_routing(2048, 64, 8, 77)
    sizes = np.diff(offsets)
    assert (sizes == 0).sum() >= 4
    y, ref = _grouped_case(bbs, 2048, 512, 192, 64, sizes, True, True, 8100, row_index)
    _check(y, ref, True, "grouped-routed")


def _moe_operands(n_rows, k, experts, seed0):
    """Stacked per-expert NVFP4 weights (16x16 scales, own s_dec each)."""
    ws = [O.nvfp4_quantize(synth.normal(n_rows, k, seed0 + g, 0.02), tile2d=True)
          for g in range(experts)]
    B = O.NVFP4(np.concatenate([w.codes for w in ws]), np.concatenate([w.scales for w in ws]),
                np.float32(0), experts * n_rows, k, True)
    return ws, B, np.array([w.s_dec for w in ws], np.float32)


def _moe_sampled_ref(A, a_rows, ws, offsets, rows, cols, chunk=4096):
    """FP64 reference of sampled outputs (rows, cols) of a grouped GEMM whose
    routed row i reads A row a_rows[i] and expert g = the group holding i,
    and the sum of |products| of each (for its accumulation bound)."""
    g_of = np.searchsorted(offsets, rows, side="right") - 1
    ref, ab = np.zeros(rows.size), np.zeros(rows.size)
    Bs = {}
    for c0 in range(0, rows.size, chunk):
        sl = slice(c0, c0 + chunk)
        toks = np.unique(a_rows[rows[sl]])
        sub = O.NVFP4(np.ascontiguousarray(A.codes[toks]), np.ascontiguousarray(A.scales[toks]),
                      A.s_dec, len(toks), A.cols, False).dequant_f64()
        pos = np.searchsorted(toks, a_rows[rows[sl]])
        for g in np.unique(g_of[sl]):
            if g not in Bs:
                Bs[g] = ws[g].dequant_f64()
            sel = np.nonzero(g_of[sl] == g)[0]
            arows, brows = sub[pos[sel]], Bs[g][cols[sl][sel]]
            ref[c0 + sel] = np.einsum("ij,ij->i", arows, brows)
            ab[c0 + sel] = np.einsum("ij,ij->i", np.abs(arows), np.abs(brows))
    assert np.abs(ref).max() > 0
    return ref, ab


def _moe_samples(offsets, n_cols, seed, per_tile=1, tile=256):
    """Samples in every tile x tile output tile of every expert (the grouped
    GEMM tiles each expert's rows from its own offset), plus each expert's
    first and last row; returns rows, cols and a tile id per sample."""
    rng = np.random.default_rng(seed)
    rows, cols, tiles = [], [], []
    tn = (n_cols + tile - 1) // tile
    tid = 0
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 <= r0:
            continue
        for m0 in range(r0, r1, tile):
            m1 = min(m0 + tile, r1)
            for tj in range(tn):
                n0, n1 = tj * tile, min((tj + 1) * tile, n_cols)
                rows.append(rng.integers(m0, m1, per_tile))
                cols.append(rng.integers(n0, n1, per_tile))
                tiles.append(np.full(per_tile, tid))
                tid += 1
        rows.append(np.array([r0, r1 - 1]))
        cols.append(rng.integers(0, n_cols, 2))
        tiles.append(np.array([tid - 1, tid - 1]))
    return (np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64),
            np.concatenate(tiles).astype(np.int64))


def test_moe_full_size_sampled(bbs):
    """The MoE expert forward at its full shape (65536 tokens x hidden 4096,
    64 experts, top-8 Zipf(1.1) routing with 4 empty experts): the gathered
    up-projection 4096 -> 1536 and the down-projection 1536 -> 4096, in the
    launch configuration the benchmark times, checked on sampled outputs."""
    announce("MoE full size: grouped up 524288x1536x4096 (gather) + down 524288x4096x1536")
    T, H, F, E = 65536, 4096, 1536, 64
    d = synth.moe_forward(T, H, F, E, 8, with_weights=False)
    ri, off = d["row_index"], d["group_offsets"]
    R = int(off[-1])
    assert R == T * 8 and int((np.diff(off) == 0).sum()) == 4
    ox = O.nvfp4_quantize(d["x"])
    del d
    ws, B, sdec = _moe_operands(F, H, E, 503)
    c = torch.empty((R, F), dtype=torch.int16, device=dev())
    bbs.grouped_nvfp4_gemm(upload_nvfp4(ox, bbs), to_dev(ri), to_dev(off), E, R,
                           upload_nvfp4(B, bbs, n_scales=sdec), F, c, bbs.OUT_BF16)
    torch.cuda.synchronize()
    rows, cols, tiles = _moe_samples(off, F, 11)
    y = bf16_bits_to_f64(host(c[to_dev(rows), to_dev(cols)]).view(np.uint16))
    del c
    ref, ab = _moe_sampled_ref(ox, ri, ws, off, rows, cols)
    check_bounded_outputs(y, ref, accumulation_bound(ab, H), True, "moe-up", tiles)
    del ws, B
    # down-projection: synthetic stand-in for the routed hidden rows
    oh = O.nvfp4_quantize(synth.normal(R, F, 600, 1.0))
    ws, B, sdec = _moe_operands(H, F, E, 503 + E)
    c = torch.empty((R, H), dtype=torch.int16, device=dev())
    bbs.grouped_nvfp4_gemm(upload_nvfp4(oh, bbs), None, to_dev(off), E, R,
                           upload_nvfp4(B, bbs, n_scales=sdec), H, c, bbs.OUT_BF16)
    torch.cuda.synchronize()
    rows, cols, tiles = _moe_samples(off, H, 12)
    y = bf16_bits_to_f64(host(c[to_dev(rows), to_dev(cols)]).view(np.uint16))
    del c
    ref, ab = _moe_sampled_ref(oh, np.arange(R), ws, off, rows, cols)
    check_bounded_outputs(y, ref, accumulation_bound(ab, F), True, "moe-down", tiles)


# ---------------------------------------------------------------------------
# GEMMs over an activation copy with per-row (per-token) decode scales
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,bf16", [(272, 400, 1024, True), (96, 144, 512, False)])
def test_gemm_per_token_A(bbs, M, N, K, bf16):
    announce(f"gemm per-token A {M}x{N}x{K} bf16={bf16}")
    oa = O.nvfp4_quantize_act(synth.normal_with_outliers(M, K, 810), True, True)
    ob = O.nvfp4_quantize(synth.normal(N, K, 811, 0.02), tile2d=True)
    A = bbs.NVFP4Tensor(to_dev(oa.codes), to_dev(oa.scales), to_dev(oa.s_dec), M, K, False, True)
    c = torch.empty((M, N), dtype=torch.int16 if bf16 else torch.float32, device=dev())
    bbs.nvfp4_gemm(bbs.FMT_NVFP4, A, upload_nvfp4(ob, bbs), c, bbs.OUT_BF16 if bf16 else bbs.OUT_F32)
    torch.cuda.synchronize()
    y = host(c)
    y = bf16_bits_to_f64(y.view(np.uint16)) if bf16 else y.astype(np.float64)
    _check(y, O.gemm_f64(oa.dequant_f64(), ob.dequant_f64()), bf16, "per-token A")


def test_full_dense_forward_per_token(bbs):
    announce("dense forward 8192x14336x4096 with a per-token 4/6 X copy (sampled outputs)")
    d = synth.dense_forward()
    oa = O.nvfp4_quantize_act(d["x"], True, True)
    ow = O.nvfp4_quantize(d["w"], tile2d=True)
    M, K = d["x"].shape
    N = d["w"].shape[0]
    A = bbs.NVFP4Tensor(to_dev(oa.codes), to_dev(oa.scales), to_dev(oa.s_dec), M, K, False, True)
    c = torch.empty((M, N), dtype=torch.int16, device=dev())
    bbs.nvfp4_gemm(bbs.FMT_NVFP4, A, upload_nvfp4(ow, bbs), c, bbs.OUT_BF16)
    torch.cuda.synchronize()
    y = bf16_bits_to_f64(host(c).view(np.uint16))
    _sampled_check(y, oa.dequant_f64(), ow.dequant_f64(), True, "fprop per-token")


def test_grouped_per_token_A(bbs):
    """Gathered grouped GEMM whose A rows carry per-token decode scales: each
    output row takes the scale of the token it was gathered from."""
    announce("grouped, per-token A, gather, 6 experts")
    rng = np.random.default_rng(820)
    sizes = np.array([40, 0, 300, 7, 0, 129])
    E, H, F, T = len(sizes), 512, 144, 256
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    total = int(off[-1])
    ri = rng.integers(0, T, total).astype(np.int32)
    ox = O.nvfp4_quantize_act(synth.normal_with_outliers(T, H, 821), True, True)
    ws, B, sdec = _moe_operands(F, H, E, 822)
    A = bbs.NVFP4Tensor(to_dev(ox.codes), to_dev(ox.scales), to_dev(ox.s_dec), T, H, False, True)
    c = torch.empty((total, F), dtype=torch.float32, device=dev())
    bbs.grouped_nvfp4_gemm(A, to_dev(ri), to_dev(off), E, total,
                           upload_nvfp4(B, bbs, n_scales=sdec), F, c, bbs.OUT_F32)
    torch.cuda.synchronize()
    A64 = ox.dequant_f64()
    ref = np.zeros((total, F))
    for g in range(E):
        if off[g + 1] > off[g]:
            ref[off[g]:off[g + 1]] = O.gemm_f64(A64[ri[off[g]:off[g + 1]]], ws[g].dequant_f64())
    _check(host(c).astype(np.float64), ref, False, "grouped per-token")


@pytest.mark.parametrize("K,bf16", [(256, True), (256, False), (272, True)])
def test_grouped_dropped_slots(bbs, K, bf16):
    """row_index entries that are negative or >= A.rows (dropped MoE slots)
    give +0 output rows, on the large-tile kernel (K % 128 == 0) and the
    small-tile one (K = 272); the other rows are unaffected.  Unit scales
    make every product exact, so the comparison is bit for bit."""
    announce(f"grouped GEMM with dropped slots K={K} bf16={bf16}")
    G, N, T = 3, 144, 64
    a = _unit(T, K, 70, False)
    counts = np.array([50, 0, 90])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(off[-1])
    rng = np.random.default_rng(71)
    ri = rng.integers(0, T, rows).astype(np.int32)
    dropped = rng.choice(rows, 24, replace=False)
    ri[dropped[:12]] = -1
    ri[dropped[12:18]] = T
    ri[dropped[18:]] = T + 1000
    ws = [_unit(N, K, 80 + g, True) for g in range(G)]
    B = O.NVFP4(np.concatenate([w.codes for w in ws]), np.concatenate([w.scales for w in ws]),
                np.float32(1), G * N, K, True)
    c = torch.full((rows, N), 7, dtype=torch.int16 if bf16 else torch.float32, device=dev())
    bbs.grouped_nvfp4_gemm(upload_nvfp4(a, bbs), to_dev(ri), to_dev(off), G, rows,
                           upload_nvfp4(B, bbs, n_scales=np.ones(G, np.float32)), N, c,
                           bbs.OUT_BF16 if bf16 else bbs.OUT_F32)
    torch.cuda.synchronize()
    y = host(c)
    A64 = a.dequant_f64()
    ref = np.zeros((rows, N))
    for g in range(G):
        for i in range(off[g], off[g + 1]):
            if 0 <= ri[i] < T:
                ref[i] = A64[ri[i]] @ ws[g].dequant_f64().T
    if bf16:
        assert np.array_equal(y.view(np.uint16), (O.bf16_rne(ref).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    else:
        assert np.array_equal(y.view(np.uint32), ref.astype(np.float32).view(np.uint32))

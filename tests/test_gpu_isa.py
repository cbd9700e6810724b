"""Checks of the gfx950 instruction behaviour the kernels are built on:
the operand / scale layout of v_mfma_scale_f32_16x16x128_f8f6f4 with 8-bit
operands, the exactness of v_cvt_scalef32_pk_f16_fp4 at scale 1.0 (the NVFP4
GEMM's expansion), and the rounding of the FP4 / FP8 conversions the
quantizers use: v_cvt_scalef32_pk_fp4_f32 (round to nearest even) and the
stochastic v_cvt_scalef32_sr_pk_fp4_f32 / v_cvt_scalef32_sr_fp8_f32."""
import ctypes as C
import os

import numpy as np
import pytest

import oracle as O
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libprobe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libprobe.so is not built (run __graft_entry__.build())")
    return C.CDLL(LIB)


def test_scaled_fp8_mfma_layout(probe):
    announce("v_mfma_scale_f32_16x16x128_f8f6f4 lane layout")
    one = torch.ones(1, dtype=torch.int32, device=dev())
    for which in (0, 1):
        out = torch.zeros(2048 * 64 * 4, dtype=torch.float32, device=dev())
        assert probe.probe_mfma_scale_layout(which, C.c_void_p(one.data_ptr()),
                                             C.c_void_p(out.data_ptr())) == 0
        acc = out.cpu().numpy().reshape(64, 32, 64, 4)     # [hot lane][hot byte][lane][v]
        for L in range(64):
            for J in range(32):
                D = np.zeros((16, 16))
                a = acc[L, J]
                for lane in range(64):
                    D[4 * (lane // 16):4 * (lane // 16) + 4, lane % 16] = a[lane]
                # hot element: row / column L % 16, K index 16*(L//16) + J (+48 for J >= 16)
                g = L // 16
                k = 16 * g + J if J < 16 else 64 + 16 * g + (J - 16)
                block = k // 32
                want = np.zeros((16, 16))
                if which == 0:
                    want[L % 16, :] = 2.0 ** block
                else:
                    want[:, L % 16] = 2.0 ** block
                assert np.array_equal(D, want), (which, L, J)


def test_fp4_to_f16_conversion_exact(probe):
    announce("v_cvt_scalef32_pk_bf16_fp4 scale handling")
    scales = np.array([1.0, 2.0, 0.25], np.float32)
    sd = torch.from_numpy(scales).to(dev())
    out = torch.zeros(len(scales) * 256 * 4, dtype=torch.int32, device=dev())
    assert probe.probe_cvt_bf16_fp4(C.c_void_p(sd.data_ptr()), len(scales),
                                    C.c_void_p(out.data_ptr())) == 0
    r = out.cpu().numpy().view(np.uint32).reshape(len(scales), 256, 4)
    dec = np.array([O.e2m1_value(c) for c in range(16)])
    for si, s in enumerate(scales):
        for b in range(256):
            w = r[si, b, 0]
            lo = np.array([w << 16], np.uint32).view(np.float32)[0]
            hi = np.array([w & 0xFFFF0000], np.uint32).view(np.float32)[0]
            assert (lo, hi) == (dec[b & 15] * s, dec[b >> 4] * s)


def test_fp4_rtn_conversion_matches_oracle(probe):
    announce("v_cvt_scalef32_pk_fp4_f32 rounding")
    grid = np.array([O.e2m1_value(c) for c in range(8)], np.float32)
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    x = np.concatenate([np.linspace(0, 8, 200001, dtype=np.float32), mids,
                        np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9)),
                        np.float32([1e-40, 0.0, 100.0])]).astype(np.float32)
    xd = torch.from_numpy(x).to(dev())
    s1 = torch.ones(1, dtype=torch.float32, device=dev())
    o = torch.zeros(len(x), dtype=torch.uint8, device=dev())
    assert probe.probe_cvt_fp4_f32(C.c_void_p(xd.data_ptr()), len(x), C.c_void_p(s1.data_ptr()),
                                   C.c_void_p(o.data_ptr())) == 0
    o = o.cpu().numpy()
    assert np.array_equal(o & 0xF, O.e2m1_code(O.round_to(x, O.E2M1)))
    assert np.array_equal(o >> 4, O.e2m1_code(O.round_to(-x, O.E2M1)))


def test_sr_conversions_match_oracle(probe):
    """The stochastic E2M1 / E4M3 conversions, issued as the quantizers issue
    them (random operand (h << 16) | 0x8000, one value per instruction),
    round exactly like the oracle's floor(t + (h + 1/2) / 2^16)."""
    announce("v_cvt_scalef32_sr_pk_fp4_f32 / v_cvt_scalef32_sr_fp8_f32 rounding")
    rng = np.random.default_rng(5)
    n = 1 << 20
    x = (2.0 ** rng.uniform(-14, 9, n) * (rng.integers(0, 2, n) * 2 - 1)).astype(np.float32)
    x[:64] = 0.0
    x[64:128] = -0.0
    h = rng.integers(0, 1 << 16, n).astype(np.uint32)
    h[:4096] = np.arange(4096) % 2 * 65535                # both ends of the uniform range
    xd, hd = torch.from_numpy(x).to(dev()), torch.from_numpy(h.view(np.int32)).to(dev())
    s1 = torch.ones(1, dtype=torch.float32, device=dev())
    o4 = torch.zeros(n, dtype=torch.uint8, device=dev())
    o8 = torch.zeros(n, dtype=torch.uint8, device=dev())
    assert probe.probe_cvt_sr(C.c_void_p(xd.data_ptr()), C.c_void_p(hd.data_ptr()), n,
                              C.c_void_p(s1.data_ptr()), C.c_void_p(o4.data_ptr()),
                              C.c_void_p(o8.data_ptr())) == 0
    u = ((h.astype(np.float64) + 0.5) / 65536.0).astype(np.float32)
    want4 = O.e2m1_code(O.round_to(x, O.E2M1, O.SR, u))   # saturates at 6 like the oracle
    got4 = o4.cpu().numpy()
    assert np.array_equal(got4 & 0xF, want4), np.nonzero((got4 & 0xF) != want4)[0][:5]
    assert np.all(got4 >> 4 == 0)
    in8 = np.abs(x) <= 448                                # MXFP8 inputs never exceed 448
    want8 = O.e4m3_code(O.round_to(x[in8], O.E4M3, O.SR, u[in8]))
    assert np.array_equal(o8.cpu().numpy()[in8], want8)


def test_gelu_and_exp_match_oracle(probe):
    """The library's GELU and exp equal the oracle's bit for bit on every
    finite BF16 input (the fused GELU + quantize sees BF16 inputs only) and
    on a dense FP32 grid through both exp cut-offs; and the two properties
    the GELU amax shortcut relies on hold for the device values."""
    announce("GELU / exp on every finite BF16 value")
    b = np.arange(65536, dtype=np.uint32)
    xb = (b << 16).view(np.float32)
    xb = xb[np.isfinite(xb)]
    grid = np.linspace(-100.0, 100.0, 1 << 18).astype(np.float32)
    x = np.concatenate([xb, grid, np.float32([-87.0, 88.5, 88.49999, -86.99999])])
    xd = torch.from_numpy(x).to("cuda:0")
    g = torch.empty_like(xd)
    e = torch.empty_like(xd)
    assert probe.probe_gelu(C.c_void_p(xd.data_ptr()), len(x), C.c_void_p(g.data_ptr()),
                            C.c_void_p(e.data_ptr())) == 0
    gh, eh = g.cpu().numpy(), e.cpu().numpy()
    og, oe = O.gelu_f32(x), O.exp_f32(x)
    bad = np.flatnonzero(gh.view(np.uint32) != og.view(np.uint32))
    assert len(bad) == 0, f"GELU differs at x={x[bad[:4]]}: {gh[bad[:4]]} vs {og[bad[:4]]}"
    bad = np.flatnonzero(eh.view(np.uint32) != oe.view(np.uint32))
    assert len(bad) == 0, f"exp differs at x={x[bad[:4]]}: {eh[bad[:4]]} vs {oe[bad[:4]]}"
    n = len(xb)
    pos = xb >= 0
    order = np.argsort(xb[pos], kind="stable")
    assert np.all(np.diff(gh[:n][pos][order]) >= 0), "GELU decreases somewhere on x >= 0"
    assert np.abs(gh[:n][~pos]).max() < 0.171875
    # the identities the quantizers' GELU table relies on (BF16 exponent field
    # below 102: 0.5 x; 130 and above: x, or -0 for negative x)
    hb = xb.view(np.uint32) >> 16
    ef = (hb >> 7) & 0xFF
    gb = gh[:n]
    tiny = ef < 102
    assert np.array_equal(gb[tiny].view(np.uint32), (np.float32(0.5) * xb[tiny]).view(np.uint32))
    big = ef >= 130
    assert np.array_equal(gb[big & pos], xb[big & pos])
    assert np.all(gb[big & ~pos].view(np.uint32) == 0x80000000)


def test_scaled_fp4_mfma_layout(probe):
    """E2M1 operands of v_mfma_scale_f32_16x16x128_f8f6f4 (format 4): which
    row each lane feeds and which 32-block scale each of its 32 nibbles is
    multiplied by (the MXFP4 GEMM relies on it)."""
    announce("v_mfma_scale_f32_16x16x128_f8f6f4 E2M1 lane layout")
    one = torch.ones(1, dtype=torch.int32, device=dev())
    blocks = np.full((2, 64, 32), -1)
    for which in (0, 1):
        out = torch.zeros(2048 * 64 * 4, dtype=torch.float32, device=dev())
        assert probe.probe_mfma_scale_layout_fp4(which, C.c_void_p(one.data_ptr()),
                                                 C.c_void_p(out.data_ptr())) == 0
        acc = out.cpu().numpy().reshape(64, 32, 64, 4)
        for L in range(64):
            for J in range(32):
                D = np.zeros((16, 16))
                a = acc[L, J]
                for lane in range(64):
                    D[4 * (lane // 16):4 * (lane // 16) + 4, lane % 16] = a[lane]
                nz = np.unique(D[D != 0])
                assert len(nz) == 1, (which, L, J, nz)
                b = int(np.log2(nz[0]))
                want = np.zeros((16, 16))
                if which == 0:
                    want[L % 16, :] = 2.0 ** b
                else:
                    want[:, L % 16] = 2.0 ** b
                assert np.array_equal(D, want), (which, L, J)
                blocks[which, L, J] = b
    # lane l feeds row l % 16 and the 32 values of block l // 16 (its 16
    # bytes), scaled by the scale that lane group supplies
    for which in (0, 1):
        for L in range(64):
            assert np.all(blocks[which, L] == L // 16), (which, L)


def test_scaled_fp4_mfma32_layout(probe):
    """E2M1 operands of v_mfma_scale_f32_32x32x64_f8f6f4 (the full-rate FP4
    form): lane l feeds row l % 32 and the 32 values of block l / 32 (its
    first 16 bytes), scaled by the scale that lane half supplies; the output
    register v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32."""
    announce("v_mfma_scale_f32_32x32x64_f8f6f4 E2M1 lane layout")
    one = torch.ones(1, dtype=torch.int32, device=dev())
    for which in (0, 1):
        out = torch.zeros(2048 * 64 * 16, dtype=torch.float32, device=dev())
        assert probe.probe_mfma32_scale_layout_fp4(which, C.c_void_p(one.data_ptr()),
                                                   C.c_void_p(out.data_ptr())) == 0
        acc = out.cpu().numpy().reshape(64, 32, 64, 16)
        for L in range(64):
            for J in range(32):
                D = np.zeros((32, 32))
                a = acc[L, J]
                for lane in range(64):
                    for v in range(16):
                        D[8 * (v // 4) + 4 * (lane // 32) + v % 4, lane % 32] = a[lane, v]
                want = np.zeros((32, 32))
                if which == 0:
                    want[L % 32, :] = 2.0 ** (L // 32)
                else:
                    want[:, L % 32] = 2.0 ** (L // 32)
                assert np.array_equal(D, want), (which, L, J)


def test_fp4_to_f16_scale_uses_exponent_only(probe):
    """v_cvt_scalef32_pk_f16_fp4 multiplies by 2^exponent(scale) only, so an
    E4M3 block scale (with mantissa bits) cannot ride in the conversion: the
    NVFP4 GEMM multiplies by the decoded block scale separately."""
    announce("v_cvt_scalef32_pk_f16_fp4: scale exponent only")
    scales = np.array([1.0, 1.125, 0.6875, 448.0, 3.0], np.float32)
    sd = torch.from_numpy(scales).to(dev())
    out = torch.zeros(len(scales) * 256, dtype=torch.int32, device=dev())
    assert probe.probe_cvt_f16_fp4(C.c_void_p(sd.data_ptr()), len(scales),
                                   C.c_void_p(out.data_ptr())) == 0
    r = out.cpu().numpy().view(np.uint32).reshape(len(scales), 256)
    dec = np.array([O.e2m1_value(c) for c in range(16)])
    for si, s in enumerate(scales):
        lo = (r[si] & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
        p2 = 2.0 ** np.floor(np.log2(s))
        assert np.array_equal(lo, dec[np.arange(256) & 15] * p2), s


def test_div6_equals_ieee_division_everywhere(probe):
    """The block scale's amax / 6 is taken as q = a RN(1/6) plus one FMA
    correction (exact below 2^-124 by a division): it must equal the
    correctly rounded quotient for every non-negative finite FP32 a."""
    announce("div6 vs IEEE a / 6 over all 2^31 non-negative FP32")
    bad = torch.zeros(1, dtype=torch.int64, device=dev())
    assert probe.probe_div6(C.c_void_p(bad.data_ptr())) == 0
    assert int(bad.item()) == 0


def test_e8m0_byte_equals_frexp_rule(probe):
    """The MXFP8 scale byte from the FP32 bits equals k + 127 of the rule
    'smallest k with amax <= 448 * 2^k' (clamped) for every amax."""
    announce("e8m0_byte vs frexp rule over all 2^31 non-negative FP32")
    bad = torch.zeros(1, dtype=torch.int64, device=dev())
    assert probe.probe_e8m0(C.c_void_p(bad.data_ptr())) == 0
    assert int(bad.item()) == 0


def test_fp8_conversion_scale_divides_exactly(probe):
    """v_cvt_scalef32_sr_fp8_f32 / v_cvt_scalef32_pk_fp8_f32 at scale 2^k
    round x / 2^k (exactly scaled) as the same instruction rounds
    ldexp(x, -k) at scale 1.0: the MXFP8 copies pass their block's power of
    two as the conversion scale (byte 0 as 2x at 2^-126), for every byte."""
    announce("FP8 conversions at scale 2^k, k = -127 .. 127")
    bad = torch.zeros(2, dtype=torch.int64, device=dev())
    assert probe.probe_fp8_scale(4096, C.c_void_p(bad.data_ptr())) == 0
    sr_bad, rne_bad = (int(v) for v in bad.cpu())
    assert sr_bad == 0 and rne_bad == 0, (sr_bad, rne_bad)

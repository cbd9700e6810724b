"""The quantized linear layer (bit_block_scaled_amd.layer) end to end: its
forward output and both gradients against the oracle's FP64 GEMMs over the
oracle's own copies of the same tensors, drawn with the same Philox streams
(relative Frobenius error <= 1e-3 against the BF16-rounded FP64 result).
"""
import numpy as np
import pytest

import oracle as O
from gpu_util import (accumulation_bound, announce, bf16_bits_to_f64, check_bounded_outputs,
                      dev, host, tile_samples, to_dev)
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 1e-3
SEED, SIGNS = 0x51F7, 0x5A3C


@pytest.fixture(scope="module")
def layer_mod():
    import bit_block_scaled_amd.layer as L
    return L


def _bf(t):
    return bf16_bits_to_f64(host(t.view(torch.int16)).view(np.uint16))


def _oracle(xb, wb, gb, step):
    ox = O.nvfp4_quantize(xb)
    oxc = O.nvfp4_quantize(xb, transpose=True, rht=True, signs=SIGNS, mode=O.SR, seed=SEED,
                           stream=4 * step)
    ow = O.nvfp4_quantize(wb, tile2d=True)
    ogc = O.nvfp4_quantize(gb, transpose=True, rht=True, signs=SIGNS, mode=O.SR, seed=SEED,
                           stream=4 * step + 1)
    ogm = O.mxfp8_quantize(gb, mode=O.SR, seed=SEED, stream=4 * step + 2)
    owt = O.mxfp8_requantize_t(ow, mode=O.SR, seed=SEED, stream=4 * step + 3)
    return {"y": (ox, ow), "dx": (ogm, owt), "dw": (ogc, oxc)}


def _run(L, xb, wb, gb, step=0):
    M, K = xb.shape
    N = wb.shape[0]
    layer = L.QLinear(K, N, seed=SEED, rht_signs=SIGNS, device=dev())
    with torch.no_grad():
        layer.weight.copy_(to_dev(wb).view(torch.bfloat16))
    layer.step = step
    x = to_dev(xb).view(torch.bfloat16).reshape(2, M // 2, K).requires_grad_(True)
    y = layer(x)
    y.backward(to_dev(gb).view(torch.bfloat16).reshape(2, M // 2, N))
    torch.cuda.synchronize()
    assert layer.step == step + 1
    return y.reshape(M, N).detach(), x.grad.reshape(M, K), layer.weight.grad


def _err(got, ref):
    return O.rel_fro(got, O.bf16_rne(ref))


def test_layer_forward_backward(layer_mod):
    announce("QLinear fwd+bwd 256x512 -> 384 against the oracle")
    M, K, N = 256, 512, 384
    xb = synth.normal_with_outliers(M, K, 71)
    wb = synth.normal(N, K, 72, 0.05)
    gb = synth.laplace(M, N, 73, 1e-2)
    y, dx, dw = _run(layer_mod, xb, wb, gb, step=3)
    o = _oracle(xb, wb, gb, 3)
    assert y.dtype == torch.bfloat16 and dx.dtype == torch.bfloat16 and dw.dtype == torch.bfloat16
    assert _err(_bf(y), O.gemm_f64(o["y"][0].dequant_f64(), o["y"][1].dequant_f64())) <= TOL
    assert _err(_bf(dx), O.gemm_f64(o["dx"][0].dequant_f64(), o["dx"][1].dequant_f64())) <= TOL
    assert _err(_bf(dw), O.gemm_f64(o["dw"][0].dequant_f64(), o["dw"][1].dequant_f64())) <= TOL


def test_layer_steps_draw_new_streams(layer_mod):
    """Consecutive calls draw fresh stochastic roundings (the gradients
    differ slightly); the same step reproduces the same bits."""
    announce("QLinear: per-step Philox streams")
    M, K, N = 128, 256, 128
    xb = synth.normal_with_outliers(M, K, 81)
    wb = synth.normal(N, K, 82, 0.05)
    gb = synth.laplace(M, N, 83, 1e-2)
    _, dx0, dw0 = _run(layer_mod, xb, wb, gb, step=0)
    _, dx0b, dw0b = _run(layer_mod, xb, wb, gb, step=0)
    _, dx1, dw1 = _run(layer_mod, xb, wb, gb, step=1)
    assert torch.equal(dx0, dx0b) and torch.equal(dw0, dw0b)
    assert not torch.equal(dx0, dx1) and not torch.equal(dw0, dw1)


def test_layer_rejects_bad_shapes(layer_mod):
    with pytest.raises(ValueError):
        layer_mod.QLinear(48, 64, device=dev())
    layer = layer_mod.QLinear(64, 64, device=dev())
    with pytest.raises(ValueError):
        layer(torch.zeros((16, 64), dtype=torch.bfloat16, device=dev()))


def test_full_layer_sampled(layer_mod):
    """The dense layer X 8192 x 4096, W 14336 x 4096, dY 8192 x 14336 as one
    forward + backward through the autograd function: outputs of Y, dX and
    dW sampled in every 256 x 256 tile, each within its accumulation bound of
    the oracle's FP64 sum (all three written in BF16 by the kernels)."""
    announce("QLinear full size 8192x4096 -> 14336 fwd+bwd (sampled)")
    fw, bw = synth.dense_forward(), synth.backward()
    xb, wb, gb = fw["x"], fw["w"], bw["dy"]
    y, dx, dw = _run(layer_mod, xb, wb, gb, step=0)
    o = _oracle(xb, wb, gb, 0)
    for name, out in (("y", y), ("dx", dx), ("dw", dw)):
        A, B = o[name][0].dequant_f64(), o[name][1].dequant_f64()
        R, C = out.shape
        rows, cols, tiles = tile_samples(R, C, 2, 1, extra=2048)
        ref = O.gemm_f64_sampled(A, B, rows, cols)
        E = accumulation_bound(O.gemm_f64_sampled(np.abs(A), np.abs(B), rows, cols), A.shape[1])
        check_bounded_outputs(_bf(out)[rows, cols], ref, E, True, name, tiles)

"""NVFP4 quantized linear layer: a torch.autograd.Function over the C ABI.

The recipe of 4bit.vizuara.ai, sections 8-10 and 13 (Figure 13) and of
Pretraining LLMs with NVFP4 ("Random Hadamard Transforms", "Two-Dimensional
Weight Scaling", "Stochastic Rounding"):

forward   X -> NVFP4 rows (1x16, nearest) for the forward GEMM, and the
          NVFP4 copy of X^T (16-point RHT, stochastic) kept for wgrad;
          W -> NVFP4 with 16x16 tile scales (nearest); Y = X W^T (NVFP4
          GEMM, BF16 out).
backward  dY -> the NVFP4 copy of dY^T (RHT, stochastic) and the MXFP8 rows
          of dY (stochastic); W's NVFP4 copy -> MXFP8 of W^T (stochastic);
          dX = dY W (MXFP8 GEMM, BF16 out); dW = dY^T X (NVFP4 GEMM over the
          two RHT'd copies, FP32 accumulation, written by the kernel in the
          weight's dtype: BF16, nearest even, or FP32).

Every step runs in the library's kernels; this module only allocates the
outputs and passes pointers.  The stochastic roundings of call t draw from
Philox streams 4t .. 4t + 3 under the layer's seed, so a run is reproducible.
Shapes: tokens, in_features and out_features multiples of 32 (the MXFP8
copies block 32 values).
"""
import torch

from . import (FMT_MXFP8, FMT_NVFP4, OUT_BF16, OUT_F32, SR, MXFP8Tensor, NVFP4Tensor,
               amax_workspace, mxfp8_requantize_t, nvfp4_gemm, nvfp4_quantize)


def _bits(t):
    """A BF16 tensor as its 16-bit patterns (no copy when already BF16 and contiguous)."""
    return t.to(torch.bfloat16).contiguous().view(torch.int16)


class QLinearFn(torch.autograd.Function):
    """y = x @ w^T with the NVFP4 recipe; x [..., in], w [out, in] (BF16)."""

    @staticmethod
    def forward(ctx, x, w, seed, step, signs):
        lead = x.shape[:-1]
        K = x.shape[-1]
        N = w.shape[0]
        x2 = _bits(x.reshape(-1, K))
        M = x2.shape[0]
        dev = x.device
        ws = amax_workspace(dev)
        xq = NVFP4Tensor.empty(M, K, device=dev)
        xc = NVFP4Tensor.empty(K, M, device=dev)
        nvfp4_quantize(x2, xq, xc, col_round=SR, col_rng=(seed, 4 * step), col_rht=True,
                       rht_signs=signs, amax_ws=ws)
        wq = NVFP4Tensor.empty(N, K, tile2d=True, device=dev)
        nvfp4_quantize(_bits(w), wq, tile2d=True, amax_ws=ws)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        nvfp4_gemm(FMT_NVFP4, xq, wq, y.view(torch.int16), OUT_BF16)
        ctx.save_for_backward(xc.codes, xc.scales, xc.s_dec, wq.codes, wq.scales, wq.s_dec)
        ctx.dims = (M, K, N, lead, w.dtype)
        ctx.rng = (seed, step, signs)
        return y.reshape(*lead, N)

    @staticmethod
    def backward(ctx, dy):
        M, K, N, lead, wdtype = ctx.dims
        seed, step, signs = ctx.rng
        xcc, xcs, xcd, wqc, wqs, wqd = ctx.saved_tensors
        xc = NVFP4Tensor(xcc, xcs, xcd, K, M, False)
        wq = NVFP4Tensor(wqc, wqs, wqd, N, K, True)
        dev = dy.device
        g = _bits(dy.reshape(M, N))
        gc = NVFP4Tensor.empty(N, M, device=dev)
        gm = MXFP8Tensor.empty(M, N, device=dev)
        nvfp4_quantize(g, None, gc, gm, col_round=SR, col_rng=(seed, 4 * step + 1), col_rht=True,
                       rht_signs=signs, mx8_round=SR, mx8_rng=(seed, 4 * step + 2),
                       amax_ws=amax_workspace(dev))
        wt = MXFP8Tensor.empty(K, N, device=dev)
        mxfp8_requantize_t(wq, wt, SR, (seed, 4 * step + 3))
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        nvfp4_gemm(FMT_MXFP8, gm, wt, dx.view(torch.int16), OUT_BF16)
        if wdtype == torch.bfloat16:
            dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
            nvfp4_gemm(FMT_NVFP4, gc, xc, dw.view(torch.int16), OUT_BF16)
        else:
            dw = torch.empty((N, K), dtype=torch.float32, device=dev)
            nvfp4_gemm(FMT_NVFP4, gc, xc, dw, OUT_F32)
            dw = dw.to(wdtype)
        return dx.reshape(*lead, K), dw, None, None, None


class QLinear(torch.nn.Module):
    """Linear layer without bias whose forward and backward GEMMs run in
    NVFP4 / MXFP8 as above.  weight: [out_features, in_features], BF16."""

    def __init__(self, in_features, out_features, seed=0, rht_signs=0x5A3C, device="cuda",
                 dtype=torch.bfloat16):
        super().__init__()
        for n in (in_features, out_features):
            if n % 32:
                raise ValueError("in_features and out_features must be multiples of 32")
        self.in_features, self.out_features = in_features, out_features
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), device=device,
                                                     dtype=dtype))
        torch.nn.init.normal_(self.weight, std=in_features ** -0.5)
        self.seed, self.rht_signs = seed, rht_signs
        self.step = 0

    def forward(self, x):
        if x.shape[-1] != self.in_features:
            raise ValueError("last dimension of x must be in_features")
        if x.numel() // self.in_features % 32:
            raise ValueError("the number of tokens must be a multiple of 32")
        y = QLinearFn.apply(x, self.weight, self.seed, self.step, self.rht_signs)
        self.step += 1
        return y

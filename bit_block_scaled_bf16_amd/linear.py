"""A linear layer whose three GEMMs run on NVFP4 operands, as a
torch.autograd.Function, with a per-layer switch back to bf16.

Source: gist.science summary of "Pretraining Large Language Models with
NVFP4", Resumen técnico §2: "Precisión Mixta Selectiva" (the linear layers'
GEMMs run in NVFP4, some layers are kept in higher precision),
"Transformadas de Hadamard Aleatorias (RHT)" (the weight-gradient inputs get
a 16x16 random Hadamard transform), "Escalado Bidimensional (2D) y Redondeo
Estocástico" (16x16 weight blocks, so that W and W^T quantize identically;
gradients are rounded stochastically).

With X [T, H], W [F, H] and Y = X W^T [T, F]:
  fprop  Y  = deq(Q_1x16(X)) . deq(Q_16x16(W))^T
  dgrad  dX = deq(Q_SR,1x16(dY)) . deq(Q_16x16(W))       (W^T's copy as B)
  wgrad  dW = deq(Q_SR(RHT(dY))) . deq(Q(RHT(X)))^T      (both transposed
                                                          copies, K = tokens)
Every step runs in the library's kernels (quantizers and GEMMs); the only
torch work is allocating their outputs. T, H and F must be multiples of 16.

When W needs a gradient, the forward pass quantizes X into both of its
copies in one call (the 1x16 row copy for fprop, the Hadamard copy for
wgrad) and keeps only the Hadamard copy for the backward pass: 0.5625 bytes
per element instead of X's 2.
"""

from __future__ import annotations

import torch

from . import (BLOCK_2D, OUT_COL, OUT_ROW, ROUND_RN, ROUND_SR, gemm, quantize, quantize_row_rht,
               rht_quantize)


class NVFP4LinearFunction(torch.autograd.Function):
    """Y = X W^T with NVFP4 fprop, dgrad and wgrad GEMMs (bf16 in and out)."""

    @staticmethod
    def forward(ctx, x, w, rht_seed: int, sr_seed: int, sr_offset: int):
        if not (x.is_cuda and w.is_cuda):
            raise RuntimeError("NVFP4 linear: tensors must be on the GPU (no CPU path)")
        if ctx.needs_input_grad[1]:
            qx, qxt, _ = quantize_row_rht(x, rht_seed, rounding_t=ROUND_RN)
        else:
            (qx, _, _), qxt = quantize(x, outputs=OUT_ROW), None
        qw, qwt, _ = quantize(w, block=BLOCK_2D, outputs=OUT_ROW | OUT_COL)
        y = gemm(qx, qw)
        ctx.qxt = qxt
        ctx.qwt = qwt
        ctx.seeds = (rht_seed, sr_seed, sr_offset)
        return y

    @staticmethod
    def backward(ctx, dy):
        rht_seed, sr_seed, sr_offset = ctx.seeds
        dy = dy.contiguous()
        dx = dw = None
        if ctx.needs_input_grad[0]:
            qdy, _, _ = quantize(dy, rounding=ROUND_SR, seed=sr_seed, offset=sr_offset,
                                 outputs=OUT_ROW)
            dx = gemm(qdy, ctx.qwt)
        if ctx.needs_input_grad[1]:
            qdyt, _ = rht_quantize(dy, rht_seed, rounding=ROUND_SR, seed=sr_seed,
                                   offset=sr_offset)
            dw = gemm(qdyt, ctx.qxt)
        return dx, dw, None, None, None


class NVFP4Linear(torch.nn.Module):
    """Linear layer without bias, weight [out_features, in_features] in bf16.

    nvfp4=False is the per-layer opt-out the recipe keeps for a few
    sensitive layers: the layer then runs a plain bf16 matmul. Each backward
    pass advances the stochastic-rounding counter (Philox counter word 2), so
    successive steps draw fresh random bits.
    """

    def __init__(self, in_features: int, out_features: int, nvfp4: bool = True,
                 rht_seed: int = 7, sr_seed: int = 7, device=None):
        super().__init__()
        self.weight = torch.nn.Parameter(
            torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.nvfp4 = nvfp4
        self.rht_seed = rht_seed
        self.sr_seed = sr_seed
        self.sr_offset = 0

    def forward(self, x):
        if not self.nvfp4:
            return x @ self.weight.t()
        offset = self.sr_offset
        self.sr_offset = (self.sr_offset + 1) & 0xFFFFFFFF
        return NVFP4LinearFunction.apply(x, self.weight, self.rht_seed, self.sr_seed, offset)

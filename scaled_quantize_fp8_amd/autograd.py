"""torch.autograd wrapper of the FP8 linear layer over the C ABI.

Fp8Linear is a drop-in for torch.nn.Linear on bf16 activations: the forward
is fp8_linear_fwd (X and W quantized to e4m3 with delayed-scaling rings, the
bias fused), the backward is fp8_linear_bwd_dw on the bf16 output gradient
(quantized once to e5m2 with its ring; dW and, when the bias needs a
gradient, db from the bf16 gradient) followed by fp8_linear_bwd_dx on that
quantized gradient ([P1] entry on the autograd backward reading its formats
from the forward instead of global state; [P4] entry on the bias column sum
running only when the bias requires a gradient; [P4] entry on 3D [B, L, d]
inputs flattened before the GEMM and the bias gradient reduced over the
leading dims).  Every step of the computation runs in the library; this
module allocates outputs and marshals arguments.
"""

from __future__ import annotations

import torch

from . import (FP8_E4M3, FP8_E5M2, Quantized, ScaleRing, fp8_db_workspace_bytes,
               fp8_linear_bwd_dw, fp8_linear_bwd_dx, fp8_linear_fwd)


class _Fp8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, mod):
        lead = x.shape[:-1]
        K = x.shape[-1]
        N = weight.shape[0]
        x2 = x.reshape(-1, K)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        M = x2.shape[0]
        dev = x.device
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        x8 = torch.empty(M, K, dtype=torch.uint8, device=dev)
        w8 = torch.empty(N, K, dtype=torch.uint8, device=dev)
        sx = torch.empty(1, dtype=torch.float32, device=dev)
        sw = torch.empty(1, dtype=torch.float32, device=dev)
        fp8_linear_fwd(x2, weight, bias, FP8_E4M3, y, mod.ring_x, mod.ring_w, x8, w8, sx, sw)
        ctx.save_for_backward(x8, w8, sx, sw)
        ctx.mod = mod
        ctx.shape = (lead, M, N, K)
        ctx.bias_grad = bias is not None and ctx.needs_input_grad[2]
        return y.view(*lead, N)

    @staticmethod
    def backward(ctx, gy):
        x8, w8, sx, sw = ctx.saved_tensors
        lead, M, N, K = ctx.shape
        mod = ctx.mod
        dev = gy.device
        g = gy.reshape(M, N)
        if g.dtype != torch.bfloat16:
            g = g.to(torch.bfloat16)
        if not g.is_contiguous():
            g = g.contiguous()
        g8 = torch.empty(M, N, dtype=torch.uint8, device=dev)
        sg = torch.empty(1, dtype=torch.float32, device=dev)
        dw = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        db = ws = None
        if ctx.bias_grad:
            db = torch.empty(N, dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(1, fp8_db_workspace_bytes(M, N) // 4), dtype=torch.float32,
                             device=dev)
        fp8_linear_bwd_dw(g, FP8_E5M2, Quantized(x8, FP8_E4M3, sx), dw, db, ws, mod.ring_g, g8,
                          sg)
        dx = None
        if ctx.needs_input_grad[0]:
            dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
            fp8_linear_bwd_dx(Quantized(g8, FP8_E5M2, sg), FP8_E5M2, Quantized(w8, FP8_E4M3, sw),
                              dx)
            dx = dx.view(*lead, K)
        return dx, dw, db, None


class Fp8Linear(torch.nn.Module):
    """y = x W^T + b with FP8 GEMMs: bf16 parameters and activations, e4m3
    forward operands, e5m2 gradients, delayed scaling with history hist_len
    for X, W and the output gradient."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 hist_len: int = 16, device=None):
        super().__init__()
        self.in_features, self.out_features, self.hist_len = in_features, out_features, hist_len
        self.weight = torch.nn.Parameter(
            torch.empty(out_features, in_features, dtype=torch.bfloat16, device=device))
        self.bias = (torch.nn.Parameter(torch.zeros(out_features, dtype=torch.bfloat16,
                                                    device=device)) if bias else None)
        torch.nn.init.normal_(self.weight, std=0.02)
        self.ring_x = self.ring_w = self.ring_g = None

    def _rings(self, device):
        if self.ring_x is None:
            self.ring_x, self.ring_w, self.ring_g = (ScaleRing(self.hist_len, device=device)
                                                     for _ in range(3))

    def forward(self, x):
        self._rings(x.device)
        return _Fp8LinearFn.apply(x, self.weight, self.bias, self)

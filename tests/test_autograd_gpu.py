"""The torch.autograd wrapper (Fp8Linear) on the GPU: one training step of
the layer against the oracle on a 3-D input, and a small transformer whose
FP8 linears train like their bf16 counterparts on a fixed synthetic batch."""

import math

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as O
from scaled_quantize_fp8_amd import e2e as E
from scaled_quantize_fp8_amd import workloads as WL
from scaled_quantize_fp8_amd.autograd import Fp8Linear
from tests.gpu_util import DEV, bf16_bits, check_gemm, f32

pytestmark = pytest.mark.gpu


def test_fp8_linear_step_matches_oracle():
    """y, dX, dW and db of one step of Fp8Linear on X [2, 64, 256] (flattened
    to 128 tokens) equal the oracle's fwd -> bwd_dw -> bwd_dx chain."""
    B, T, K, N = 2, 64, 256, 192
    X = WL.normal_bf16((B, T, K), 1.0, 61)
    W = WL.normal_bf16((N, K), 0.02, 62)
    b = WL.normal_bf16((N,), 0.01, 63)
    G = WL.normal_bf16((B, T, N), 1e-3, 64)
    mod = Fp8Linear(K, N, device=DEV)
    with torch.no_grad():
        mod.weight.copy_(W)
        mod.bias.copy_(b)
    x = X.to(DEV).requires_grad_(True)
    y = mod(x)
    y.backward(G.to(DEV))
    torch.cuda.synchronize()

    rx, rw, rg = O.ScaleRing(16), O.ScaleRing(16), O.ScaleRing(16)
    x8, sx, _ = O.quantize_step(f32(X).reshape(B * T, K), O.E4M3, rx)
    w8, sw, _ = O.quantize_step(f32(W), O.E4M3, rw)
    beta = O.bias_values(b.view(torch.int16).numpy().view(np.uint16), "bf16")
    g2 = f32(G).reshape(B * T, N)
    g8, sg, _ = O.quantize_step(g2, O.E5M2, rg)
    check_gemm(bf16_bits(y).reshape(B * T, N), O.linear_fwd(x8, w8, O.E4M3, sx, sw, beta), "y")
    check_gemm(bf16_bits(mod.weight.grad), O.linear_bwd_dw(g8, O.E5M2, x8, O.E4M3, sg, sx), "dW")
    check_gemm(bf16_bits(mod.bias.grad), O.bias_grad(g2.astype(np.float64)), "db")
    check_gemm(bf16_bits(x.grad).reshape(B * T, K), O.linear_bwd_dx(g8, O.E5M2, w8, O.E4M3, sg, sw),
               "dX")


def _train(lin, steps=40):
    m = E.Transformer(lin, layers=2, d=256, heads=4, ffn=1024, vocab=1000, device=DEV)
    tok, tgt = E.synthetic_batch(2, 128, 1000, DEV, seed=9)
    opt = torch.optim.AdamW(m.parameters(), lr=2e-3)
    losses = []
    with E.attention_backends():
        for _ in range(steps):
            opt.zero_grad(set_to_none=True)
            loss = m.loss(tok, tgt)
            loss.backward()
            opt.step()
            losses.append(loss.item())
    return losses


def test_small_transformer_trains_like_bf16():
    bf = _train(E.bf16_linear)
    f8 = _train(E.fp8_linear)
    assert all(math.isfinite(v) for v in f8)
    assert abs(f8[0] - bf[0]) < 0.05 * bf[0]        # same initial model, same loss
    assert f8[-1] < f8[0] - 2.0 and bf[-1] < bf[0] - 2.0  # both memorize the batch
    assert abs(f8[-1] - bf[-1]) < 0.25 * bf[0]


def test_graph_replays_match_eager_steps():
    """The whole FP8 training step captured as one HIP graph: every replay
    gives the loss the eager step gives (same model, same batch, same
    optimizer state), so graph timings time the same computation."""
    dims = dict(layers=2, d=256, heads=4, ffn=1024, vocab=1000)
    eager, _ = E.train(E.fp8_linear, 6, DEV, graph=False, dims=dims, batch=(2, 128))
    replay, _ = E.train(E.fp8_linear, 6, DEV, graph=True, dims=dims, batch=(2, 128))
    assert all(math.isfinite(v) for v in replay)
    np.testing.assert_allclose(replay, eager, rtol=1e-5, atol=1e-5)


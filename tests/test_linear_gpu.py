"""End-to-end GPU parity of one FP8 linear layer step (fwd -> bwd_dw ->
bwd_dx) on the five workloads, against the oracle run on the same inputs.

Quantized bytes, amax, scales and ring state are compared bit for bit;
GEMM outputs against the 2^-7 contract and the 2^-10 diagnostic bound.  The
full-size workloads compare every element of Y, dX, dW and db of every
linear of one whole layer (the dim1024 layer, the dim1536 layer at M = 2048
and at M = 512, the generic 4096 <-> 11008 pair); their seeding steps and
the pre-quantized workload's eight drift steps compare a seeded sample of
rows plus the first and last (stated where they run).  As a sanity check
beside parity, the fp8 outputs keep the direction of the unquantized bf16
products (cosine close to 1, against the pages' regression signature of a
cosine near 0.05 for a wrong amax).
"""

from dataclasses import dataclass

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from oracle import fp8_oracle as O
from scaled_quantize_fp8_amd import workloads as WL
from tests.gpu_util import (DEV, assert_ring_matches, bf16_bits, check_gemm, f32, f32_scalar,
                            scalar_dev, to_dev, u8)

pytestmark = pytest.mark.gpu

FX, FG = O.E4M3, O.E5M2


@dataclass
class Rings:
    x: object
    w: object
    g: object
    ox: object
    ow: object
    og: object


def make_rings(hist_len, delayed=True, w_ring=True):
    if not delayed:
        return Rings(None, None, None, None, None, None)
    return Rings(F.ScaleRing(hist_len), F.ScaleRing(hist_len) if w_ring else None,
                 F.ScaleRing(hist_len), O.ScaleRing(hist_len),
                 O.ScaleRing(hist_len) if w_ring else None, O.ScaleRing(hist_len))


def _rows(M, rng, k=40):
    """A seeded sample of k rows, plus the first and last 32 rows (the
    corner tiles' edges); every row when M <= 256."""
    if M <= 256:
        return np.arange(M)
    edges = np.concatenate([np.arange(32), np.arange(M - 32, M)])
    return np.unique(np.concatenate([edges, rng.choice(M, k, replace=False)]))


def _cos(a, b):
    a, b = np.asarray(a, np.float64).ravel(), np.asarray(b, np.float64).ravel()
    return float(np.dot(a, b) / np.sqrt(np.dot(a, a) * np.dot(b, b)))


def direction_sanity(X, W, G, y, dx, dw, beta):
    """Cosine of each fp8 output with the same product of the unquantized
    bf16 operands (torch CPU float32): dX is the one the pages' wrong-amax
    regression collapsed to about 0.05."""
    Xf, Wf, Gf = X.float(), W.float(), G.float()
    refs = {"y": (Xf @ Wf.T).numpy() + beta, "dx": (Gf @ Wf).numpy(), "dw": (Gf.T @ Xf).numpy()}
    for name, got in (("y", y), ("dx", dx), ("dw", dw)):
        c = _cos(O.bf16_value(got), refs[name])
        assert c > 0.99, f"{name}: cosine {c} with the bf16 product"


def layer_step(X, W, b, G, rings, rng, w_pre=None, bias_pre=None, check_all=False,
               direction=False, sample=40):
    """One fwd + bwd_dw(+db) + bwd_dx on the GPU and in the oracle.
    X, W, b, G: bf16 CPU tensors.  w_pre: (w8 codes, s_w) pre-quantized
    weight; bias_pre: (b8 codes, bias_scale).  check_all: every output
    element against the oracle (else `sample` seeded rows plus the edge
    rows); direction: also the cosine sanity check.  Returns a dict of
    results."""
    M, K = X.shape
    N = W.shape[0]
    f32_ = lambda: torch.empty(1, dtype=torch.float32, device=DEV)
    xd, gd = X.to(DEV), G.to(DEV)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    x8 = torch.empty(M, K, dtype=torch.uint8, device=DEV)
    sx, ax, sw, aw = f32_(), f32_(), f32_(), f32_()
    if w_pre is None:
        w_arg = W.to(DEV)
        w8 = torch.empty(N, K, dtype=torch.uint8, device=DEV)
    else:
        w_arg = F.Quantized(to_dev(w_pre[0]), FX, scalar_dev(w_pre[1]))
        w8 = None
    if bias_pre is None:
        bias_arg = b.to(DEV)
        beta = O.bias_values(b.view(torch.int16).numpy().view(np.uint16), "bf16")
    else:
        bias_arg = F.Quantized(to_dev(bias_pre[0]), FX, scalar_dev(bias_pre[1]))
        beta = O.bias_values(bias_pre[0], "e4m3", bias_pre[1])
    F.fp8_linear_fwd(xd, w_arg, bias_arg, FX, y, rings.x, rings.w, x8, w8, sx, sw, ax, aw)
    # backward: dW (quantizes G once, db from the bf16 G), then dX from G8
    g8 = torch.empty(M, N, dtype=torch.uint8, device=DEV)
    sg, ag = f32_(), f32_()
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    db = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, F.fp8_db_workspace_bytes(M, N) // 4), dtype=torch.float32, device=DEV)
    x8q = F.Quantized(x8, FX, sx)
    w8q = F.Quantized(w8, FX, sw) if w8 is not None else w_arg
    F.fp8_linear_bwd_dw(gd, FG, x8q, dw, db, ws, rings.g, g8, sg, ag)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    F.fp8_linear_bwd_dx(F.Quantized(g8, FG, sg), FG, w8q, dx)
    torch.cuda.synchronize()

    # oracle
    ox8, osx, oax = O.quantize_step(f32(X), FX, rings.ox)
    if w_pre is None:
        ow8, osw, oaw = O.quantize_step(f32(W), FX, rings.ow)
    else:
        ow8, osw, oaw = w_pre[0], np.float32(w_pre[1]), np.float32(0.0)
    og8, osg, oag = O.quantize_step(f32(G), FG, rings.og)
    out = dict(sx=f32_scalar(sx), sw=f32_scalar(sw), sg=f32_scalar(sg), ax=f32_scalar(ax),
               aw=f32_scalar(aw), ag=f32_scalar(ag), osx=osx, osw=osw, osg=osg, y=bf16_bits(y),
               x8=u8(x8), w8=ow8, beta=beta)
    assert out["sx"] == osx and out["ax"] == oax
    assert out["sw"] == osw and out["aw"] == oaw
    assert out["sg"] == osg and out["ag"] == oag
    assert np.array_equal(u8(x8), ox8)
    if w8 is not None:
        assert np.array_equal(u8(w8), ow8)
    assert np.array_equal(u8(g8), og8)
    if rings.ox is not None:
        assert_ring_matches(rings.x, rings.ox)
        assert_ring_matches(rings.g, rings.og)
        if rings.ow is not None:
            assert_ring_matches(rings.w, rings.ow)
    rows = np.arange(M) if check_all else _rows(M, rng, sample)
    nrows = np.arange(N) if check_all else _rows(N, rng, sample)
    check_gemm(out["y"][rows], O.linear_fwd(ox8[rows], ow8, FX, osx, osw, beta), "fwd")
    check_gemm(bf16_bits(dx)[rows], O.linear_bwd_dx(og8[rows], FG, ow8, FX, osg, osw), "dx")
    check_gemm(bf16_bits(dw)[nrows], O.linear_bwd_dw(og8[:, nrows], FG, ox8, FX, osg, osx), "dw")
    check_gemm(bf16_bits(db), O.bias_grad(f32(G).astype(np.float64)), "db")
    if direction:
        direction_sanity(X, W, G, out["y"], bf16_bits(dx), bf16_bits(dw), beta)
    return out


def test_tiny_four_steps_full_outputs():
    wl = WL.WORKLOADS["tiny"]
    X0, W, b, G = WL.layer_inputs(wl, 0)
    rings = make_rings(wl.hist_len)
    rng = np.random.default_rng(0)
    res = []
    for c in WL.TINY_STEP_FACTORS:
        Xt = (X0.float() * c).to(torch.bfloat16)
        res.append(layer_step(Xt, W, b, G, rings, rng, check_all=True))
    S = O.scale_from_amax(O.amax(f32(X0)), FX, 1.0)
    assert [r["sx"] for r in res] == [S, S, S / 4, S / 4]
    assert np.array_equal(res[3]["x8"], res[1]["x8"])


@pytest.mark.parametrize("wl_name,M", [("dim1024_m2048", None), ("dim1536_m2048", None),
                                       ("dim1536_m512", None)])
def test_layer_workloads_two_steps(wl_name, M):
    """Every linear of one whole layer, two delayed-scaling steps: the
    seeding step on a row sample, the steady step (X scaled by 1.5, so the
    scale used is the one published by the first step) on every element."""
    wl = WL.WORKLOADS[wl_name]
    rng = np.random.default_rng(1)
    for li in range(len(wl.linears)):
        X, W, b, G = WL.layer_inputs(wl, li, M=M)
        rings = make_rings(wl.hist_len)
        for step in range(2):
            Xs = X if step == 0 else (X.float() * 1.5).to(torch.bfloat16)
            layer_step(Xs, W, b, G, rings, rng, check_all=step == 1, direction=step == 1)


def test_generic_dynamic_scaling():
    """Both generic linears (4096 -> 11008, 11008 -> 4096, M = 4096), dynamic
    scaling, every element of Y, dX, dW and db."""
    wl = WL.WORKLOADS["generic_m4096"]
    rng = np.random.default_rng(2)
    for li in range(len(wl.linears)):
        X, W, b, G = WL.layer_inputs(wl, li)
        layer_step(X, W, b, G, make_rings(wl.hist_len, delayed=False), rng, check_all=True,
                   direction=True)


def test_prequantized_weight_leaves_its_ring_untouched():
    """A pre-quantized W passed together with a ring: its quantize is skipped,
    so the ring's bytes stay as they were, amax_w is 0 and sw_used is the
    operand's own scale ([P1] entry on pre-quantized weights, amax_w = 0)."""
    wl = WL.WORKLOADS["prequant_dim1536_m2048"]
    X, W, b, G = WL.layer_inputs(wl, 0, M=256)
    M, K = X.shape
    N = W.shape[0]
    sw_ = O.scale_from_amax(O.amax(f32(W)), FX, 1.0)
    w8 = O.quantize_with_scale(f32(W), sw_, FX)
    rx, rw = F.ScaleRing(wl.hist_len), F.ScaleRing(wl.hist_len)
    # give ring_w a history of its own first, so "unchanged" is not all zeros
    wq = torch.empty(N * K, dtype=torch.uint8, device=DEV)
    F.fp8_quantize(W.to(DEV), FX, wq, rw, scalar_dev(0.0), None)
    torch.cuda.synchronize()
    before = rw.buf.clone()
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    x8 = torch.empty(M, K, dtype=torch.uint8, device=DEV)
    sx, ax = scalar_dev(0.0), scalar_dev(0.0)
    sw, aw = scalar_dev(-1.0), scalar_dev(-1.0)
    for _ in range(2):
        F.fp8_linear_fwd(X.to(DEV), F.Quantized(to_dev(w8), FX, scalar_dev(sw_)), b.to(DEV), FX, y,
                         rx, rw, x8, None, sx, sw, ax, aw)
    torch.cuda.synchronize()
    assert torch.equal(rw.buf, before)
    assert rw.seeded
    assert f32_scalar(aw) == 0.0 and f32_scalar(sw) == sw_
    ox8, osx, _ = O.quantize_step(f32(X), FX, O.ScaleRing(wl.hist_len))
    check_gemm(bf16_bits(y), O.linear_fwd(u8(x8), w8, FX, f32_scalar(sx), sw_,
                                          O.bias_values(b.view(torch.int16).numpy().view(np.uint16),
                                                        "bf16")), "fwd")


def test_prequantized_weight_and_bias_eight_steps_non_leak():
    """W and the bias pre-quantized (e4m3 with their scales), eight delayed
    steps of log-uniform amax drift on X.  Every element of every output on
    the up linear (the largest shape) at every step; on the other linears a
    seeded sample of 256 rows plus the first and last 32 (the corner tiles'
    edges).  amax_w is 0, and a leaked scale would have been visible."""
    wl = WL.WORKLOADS["prequant_dim1536_m2048"]
    rng = np.random.default_rng(3)
    detectable = 0
    for li in range(len(wl.linears)):
        X0, W, b, G = WL.layer_inputs(wl, li)
        sw_ = O.scale_from_amax(O.amax(f32(W)), FX, 1.0)
        w8 = O.quantize_with_scale(f32(W), sw_, FX)
        sb_ = O.scale_from_amax(O.amax(f32(b)), FX, 1.0)
        b8 = O.quantize_with_scale(f32(b), sb_, FX)
        drift = WL.log_uniform_drift(WL.PREQUANT_STEPS, WL.seed_for(0, "drift", li))
        a0 = float(O.amax(f32(X0)))
        rings = make_rings(wl.hist_len, w_ring=False)
        for t, d in enumerate(drift):
            Xt = (X0.float() * (d / a0)).to(torch.bfloat16)
            out = layer_step(Xt, W, b, G, rings, rng, w_pre=(w8, sw_), bias_pre=(b8, sb_),
                             check_all=wl.linears[li].name == "up", sample=256)
            assert out["aw"] == 0.0
            # the scale the ring publishes after this step differs from the
            # one used: a leak would be visible in Y
            s_next = np.float32(rings.ox.scale)
            if t > 0 and s_next != out["sx"]:
                rows = np.arange(0, Xt.shape[0], 97)
                leak = O.linear_fwd(out["x8"][rows], w8, FX, s_next, sw_, out["beta"])
                err = np.abs(O.bf16_value(out["y"][rows]) - leak.r)
                if np.any(err > O.gemm_tolerance(leak)):
                    detectable += 1
    assert detectable >= 1

"""The allocation-free weight-gradient entry point (fp8_linear_bwd_dw_noalloc)
against fp8_linear_bwd_dw with a caller workspace: the same inputs and ring
sequence through both, two calls in a row (the second smaller, so it reuses
the library's array after a larger call left data in it), with G in bf16
and pre-quantized; every output byte and the ring state must be identical
(the two run the same kernels in the same order)."""

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from oracle import fp8_oracle as O
from tests.gpu_util import DEV, bf16_bits, check_gemm, f32, f32_scalar, u8

pytestmark = pytest.mark.gpu

FX, FG = F.FP8_E4M3, F.FP8_E5M2


def _case(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    G = (torch.randn(M, N, generator=g) * 1e-3).to(torch.bfloat16)
    X = torch.randn(M, K, generator=g).to(torch.bfloat16)
    return G, X


def _outs(M, N, K):
    """Output buffers pre-filled with NaN (codes 0x7F), so an element a call
    does not write cannot match."""
    e = lambda *s, dt: torch.full(s, 0x7F if dt == torch.uint8 else float("nan"), dtype=dt,
                                  device=DEV)
    return dict(dw=e(N, K, dt=torch.bfloat16), db=e(N, dt=torch.bfloat16),
                g8=e(M, N, dt=torch.uint8), sg=e(1, dt=torch.float32),
                ag=e(1, dt=torch.float32))


def test_noalloc_matches_workspace_entry_point():
    ring_ws, ring_na = F.ScaleRing(16), F.ScaleRing(16)
    for step, (M, N, K) in enumerate(((2048, 6912, 1536), (300, 200, 136))):
        G, X = _case(M, N, K, step)
        x8 = torch.empty(M, K, dtype=torch.uint8, device=DEV)
        sx = torch.empty(1, dtype=torch.float32, device=DEV)
        F.fp8_quantize(X.to(DEV), FX, x8, None, sx, torch.empty(1, device=DEV))
        x8q = F.Quantized(x8, FX, sx)
        Gd = G.to(DEV)
        a, b = _outs(M, N, K), _outs(M, N, K)
        ws = torch.empty(max(1, F.fp8_db_workspace_bytes(M, N) // 4), dtype=torch.float32,
                         device=DEV)
        F.fp8_linear_bwd_dw(Gd, FG, x8q, a["dw"], a["db"], ws, ring_ws, a["g8"], a["sg"], a["ag"])
        F.fp8_linear_bwd_dw_noalloc(Gd, FG, x8q, b["dw"], b["db"], ring_na, b["g8"], b["sg"],
                                    b["ag"])
        torch.cuda.synchronize()
        for k in a:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), (step, k)
        assert torch.equal(ring_ws.buf, ring_na.buf), step
        # and against the oracle: the call's dW and db
        og8 = u8(a["g8"])
        osg = f32_scalar(a["sg"])
        check_gemm(bf16_bits(b["dw"]), O.linear_bwd_dw(og8, O.E5M2, u8(x8), O.E4M3, osg,
                                                       f32_scalar(sx)), f"dw {step}")
        check_gemm(bf16_bits(b["db"]), O.bias_grad(f32(G).astype(np.float64)), f"db {step}")
        # pre-quantized G: db from dec(g8)/sg through the same array
        c, d = _outs(M, N, K), _outs(M, N, K)
        g8q = F.Quantized(a["g8"], FG, a["sg"])
        F.fp8_linear_bwd_dw(g8q, FG, x8q, c["dw"], c["db"], ws, None, None, c["sg"], c["ag"])
        F.fp8_linear_bwd_dw_noalloc(g8q, FG, x8q, d["dw"], d["db"], None, None, d["sg"], d["ag"])
        torch.cuda.synchronize()
        for k in ("dw", "db", "sg", "ag"):
            assert torch.equal(c[k].view(torch.uint8), d[k].view(torch.uint8)), (step, "pre", k)


def test_noalloc_rejects_sizes_beyond_its_array():
    M, N, K = 4096, 8192, 64  # db partials: 4 * 8192 * 128 = 4 MiB: fits
    assert F.fp8_db_workspace_bytes(M, N) <= 8 << 20
    M2 = 8192 + 32            # 4 * 8192 * 257 > 8 MiB: refused when db is wanted
    assert F.fp8_db_workspace_bytes(M2, N) > 8 << 20
    G = torch.zeros(M2, N, dtype=torch.bfloat16, device=DEV)
    x8 = F.Quantized(torch.zeros(M2, K, dtype=torch.uint8, device=DEV), FX,
                     torch.ones(1, device=DEV))
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    db = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    g8 = torch.empty(M2, N, dtype=torch.uint8, device=DEV)
    sg, ag = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    with pytest.raises(F.Fp8Error) as e:
        F.fp8_linear_bwd_dw_noalloc(G, FG, x8, dw, db, None, g8, sg, ag)
    assert e.value.status == F.FP8_ERR_SHAPE
    # without db the same call needs no partials and runs
    F.fp8_linear_bwd_dw_noalloc(G, FG, x8, dw, None, None, g8, sg, ag)
    torch.cuda.synchronize()
    assert not dw.float().abs().max().item()

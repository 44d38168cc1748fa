"""GPU parity of the backward entry point fp8_linear_bwd: on two streams,
and on one stream, where the dX and dW GEMMs run as one grouped launch.

By contract its results are those of fp8_linear_bwd_dw followed by
fp8_linear_bwd_dx from the same g: the kernels are the same and
deterministic, so every output byte (G8, dX, dW, db, scales, amax, ring
state) must equal the pair's, run on copies of the same inputs (the
grouped launch runs each GEMM on the kernel its own launch would take).
Three cases are also checked against the oracle directly, every element.  The two streams are torch streams of default
priority; the dW stream is joined back before anything is read.
"""

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from oracle import fp8_oracle as O
from tests.gpu_util import DEV, assert_ring_matches, bf16_bits, check_gemm, f32, f32_scalar, \
    ring_state, scalar_dev, to_dev, u8

pytestmark = pytest.mark.gpu

FX, FG = F.FP8_E4M3, F.FP8_E5M2


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


class Bwd:
    """Buffers of one backward; run() through the pair or the two-stream call."""

    def __init__(self, G, x8, sx, w8, sw, ring, g_pre=None, want_db=True):
        M, N = G.shape
        K = x8.shape[1]
        e = lambda *s, dt=torch.uint8: torch.empty(*s, dtype=dt, device=DEV)
        z = lambda: torch.zeros(1, dtype=torch.float32, device=DEV)
        self.G = G.to(DEV)
        self.g_pre = None if g_pre is None else F.Quantized(to_dev(g_pre[0]), FG,
                                                              scalar_dev(g_pre[1]))
        self.x8q = F.Quantized(to_dev(x8), FX, scalar_dev(sx))
        self.w8q = F.Quantized(to_dev(w8), FX, scalar_dev(sw))
        self.g8, self.sg, self.ag = e(M, N), z(), z()
        self.dx, self.dw = e(M, K, dt=torch.bfloat16), e(N, K, dt=torch.bfloat16)
        self.db = e(N, dt=torch.bfloat16) if want_db else None
        self.ws = e(max(1, F.fp8_db_workspace_bytes(M, N) // 4), dt=torch.float32)
        self.ring = ring

    def g_arg(self):
        return self.G if self.g_pre is None else self.g_pre

    def run_pair(self):
        F.fp8_linear_bwd_dw(self.g_arg(), FG, self.x8q, self.dw, self.db, self.ws, self.ring,
                            self.g8, self.sg, self.ag)
        if self.g_pre is None:
            g8q = F.Quantized(self.g8, FG, self.sg)
        else:
            g8q = self.g_pre
        F.fp8_linear_bwd_dx(g8q, FG, self.w8q, self.dx, None, None,
                            None if self.g_pre is None else self.sg,
                            None if self.g_pre is None else self.ag)
        torch.cuda.synchronize()

    def run_two_stream(self, side):
        main = torch.cuda.current_stream()
        F.fp8_linear_bwd(self.g_arg(), FG, self.x8q, self.w8q, self.dx, self.dw, self.db,
                         self.ws, self.ring, self.g8, self.sg, self.ag, stream=main,
                         stream_dw=side)
        if side is not None:
            main.wait_stream(side)
        torch.cuda.synchronize()

    def snapshot(self):
        out = {k: getattr(self, k).cpu().view(torch.uint8).numpy().copy()
               for k in ("dx", "dw", "sg", "ag") if getattr(self, k) is not None}
        if self.g_pre is None:
            out["g8"] = u8(self.g8)
        if self.db is not None:
            out["db"] = self.db.cpu().view(torch.uint8).numpy().copy()
        if self.ring is not None:
            for k, v in ring_state(self.ring).items():
                out[f"ring.{k}"] = np.asarray(v).copy()
        return out


def _inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    G = _bf16(rng.standard_normal((M, N)) * 1e-3)
    tab = O.decode_table(O.E4M3)
    fin = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    x8 = rng.choice(fin, size=(M, K))
    w8 = rng.choice(fin, size=(N, K))
    return G, x8, w8, rng


def _assert_same(a, b, what):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what}: {k} differs from the one-stream pair"


# (256, 384, 320): 128x128 tiles, ragged nothing; (2048, 6912, 1536): the up
# projection's backward (dW on the 256x256 kernel, dX on the 8-wave 128x128);
# (2048, 1536, 6912): the down projection's; (200, 264, 136): the general
# kernel (dimensions not multiples of 16)
SHAPES = [(256, 384, 320), (2048, 6912, 1536), (2048, 1536, 6912), (200, 264, 136)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode", ["ring", "dynamic", "prequantized"])
def test_two_stream_matches_pair(M, N, K, mode):
    G, x8, w8, rng = _inputs(M, N, K, seed=M + 3 * N + K)
    g_pre = None
    if mode == "prequantized":
        tab = O.decode_table(O.E5M2)
        fin = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
        g_pre = (rng.choice(fin, size=(M, N)), 64.0)
    side = torch.cuda.Stream()
    ring_a = F.ScaleRing(4) if mode == "ring" else None
    ring_b = F.ScaleRing(4) if mode == "ring" else None
    a = Bwd(G, x8, 2.0, w8, 0.5, ring_a, g_pre)
    b = Bwd(G, x8, 2.0, w8, 0.5, ring_b, g_pre)
    steps = 3 if mode == "ring" else 1  # the first step seeds the ring
    for step in range(steps):
        f = 1.0 + step
        a.G.copy_((a.G.float() * f).to(torch.bfloat16))
        b.G.copy_((b.G.float() * f).to(torch.bfloat16))
        a.run_pair()
        b.run_two_stream(side)
        _assert_same(a.snapshot(), b.snapshot(), f"step {step}")


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode", ["ring", "dynamic", "prequantized"])
def test_grouped_one_stream_matches_pair(M, N, K, mode):
    """stream_dw = stream: dX and dW as one grouped launch (the 200x264x136
    case takes the general kernel one GEMM at a time)."""
    G, x8, w8, rng = _inputs(M, N, K, seed=M + 5 * N + K)
    g_pre = None
    if mode == "prequantized":
        tab = O.decode_table(O.E5M2)
        fin = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
        g_pre = (rng.choice(fin, size=(M, N)), 64.0)
    ring_a = F.ScaleRing(4) if mode == "ring" else None
    ring_b = F.ScaleRing(4) if mode == "ring" else None
    a = Bwd(G, x8, 2.0, w8, 0.5, ring_a, g_pre)
    b = Bwd(G, x8, 2.0, w8, 0.5, ring_b, g_pre)
    steps = 3 if mode == "ring" else 1
    for step in range(steps):
        f = 1.0 + step
        a.G.copy_((a.G.float() * f).to(torch.bfloat16))
        b.G.copy_((b.G.float() * f).to(torch.bfloat16))
        a.run_pair()
        b.run_two_stream(None)
        _assert_same(a.snapshot(), b.snapshot(), f"step {step}")


@pytest.mark.parametrize("M,N,K", [(2048, 4608, 1536), (512, 1536, 6912)])
def test_grouped_against_oracle_full(M, N, K):
    """The one-stream backward of the qkv projection (its dW on 256x128
    tiles, launched alone) and a few-tile small-M case (the down projection
    at M = 512), every element of dX, dW and db against the oracle over two
    ring steps."""
    G, x8, w8, _ = _inputs(M, N, K, seed=23 + M)
    ring, oring = F.ScaleRing(4), O.ScaleRing(4)
    b = Bwd(G, x8, 2.0, w8, 0.5, ring)
    for step in range(2):
        Gs = (G.float() * (1.0 + step)).to(torch.bfloat16)
        b.G.copy_(Gs.to(DEV))
        b.run_two_stream(None)
        og8, osg, oag = O.quantize_step(f32(Gs), O.E5M2, oring)
        assert np.array_equal(u8(b.g8), og8)
        assert f32_scalar(b.sg) == osg and f32_scalar(b.ag) == oag
        assert_ring_matches(ring, oring)
        check_gemm(bf16_bits(b.dx), O.linear_bwd_dx(og8, O.E5M2, w8, O.E4M3, osg, 0.5), "dx")
        check_gemm(bf16_bits(b.dw), O.linear_bwd_dw(og8, O.E5M2, x8, O.E4M3, osg, 2.0), "dw")
        check_gemm(bf16_bits(b.db), O.bias_grad(f32(Gs).astype(np.float64)), "db")


# empty problems: no G rows (dW and db are zeros), no G columns (dX is
# zeros), no features (only db has elements)
@pytest.mark.parametrize("M,N,K", [(0, 64, 32), (48, 0, 32), (48, 64, 0)])
@pytest.mark.parametrize("mode", ["ring", "prequantized"])
def test_two_stream_degenerate_sizes(M, N, K, mode):
    G, x8, w8, rng = _inputs(M, N, K, seed=17 + M + N + K)
    g_pre = None
    if mode == "prequantized":
        g_pre = (np.full((M, N), 0x3C, np.uint8), 2.0)  # e5m2 1.0
    side = torch.cuda.Stream()
    a = Bwd(G, x8, 1.0, w8, 1.0, F.ScaleRing(4) if mode == "ring" else None, g_pre)
    b = Bwd(G, x8, 1.0, w8, 1.0, F.ScaleRing(4) if mode == "ring" else None, g_pre)
    for step in range(2):
        a.run_pair()
        b.run_two_stream(side)
        _assert_same(a.snapshot(), b.snapshot(), f"step {step}")
    if M == 0 or K == 0:
        assert not torch.any(b.dw.float() != 0) and not torch.any(b.dx.float() != 0)
    if M == 0:
        assert not torch.any(b.db.float() != 0)
    if mode == "prequantized" and N > 0 and K == 0:
        # db = sum over rows of dec(g8) / sg = M * 1.0 / 2.0
        assert torch.all(b.db.float() == M / 2.0)


def test_same_stream_and_no_db():
    """stream_dw = stream (the grouped launch), without db."""
    M, N, K = 384, 512, 256
    G, x8, w8, _ = _inputs(M, N, K, seed=5)
    a = Bwd(G, x8, 1.0, w8, 4.0, F.ScaleRing(8), want_db=False)
    b = Bwd(G, x8, 1.0, w8, 4.0, F.ScaleRing(8), want_db=False)
    for _ in range(2):
        a.run_pair()
        b.run_two_stream(None)  # stream_dw = stream: one grouped launch
        _assert_same(a.snapshot(), b.snapshot(), "same stream")


def test_two_stream_against_oracle():
    M, N, K = 256, 384, 320
    G, x8, w8, _ = _inputs(M, N, K, seed=11)
    ring, oring = F.ScaleRing(4), O.ScaleRing(4)
    b = Bwd(G, x8, 2.0, w8, 0.5, ring)
    for step in range(2):
        b.run_two_stream(torch.cuda.Stream())
        og8, osg, oag = O.quantize_step(f32(G), O.E5M2, oring)
        assert np.array_equal(u8(b.g8), og8)
        assert f32_scalar(b.sg) == osg and f32_scalar(b.ag) == oag
        assert_ring_matches(ring, oring)
        check_gemm(bf16_bits(b.dx), O.linear_bwd_dx(og8, O.E5M2, w8, O.E4M3, osg, 0.5), "dx")
        check_gemm(bf16_bits(b.dw), O.linear_bwd_dw(og8, O.E5M2, x8, O.E4M3, osg, 2.0), "dw")
        check_gemm(bf16_bits(b.db), O.bias_grad(f32(G).astype(np.float64)), "db")


def test_two_stream_errors_enqueue_nothing():
    M, N, K = 64, 64, 64
    G, x8, w8, _ = _inputs(M, N, K, seed=2)
    ring = F.ScaleRing(4)
    b = Bwd(G, x8, 1.0, w8, 1.0, ring)
    with pytest.raises(F.Fp8Error) as e:  # db without its workspace
        F.fp8_linear_bwd(b.G, FG, b.x8q, b.w8q, b.dx, b.dw, b.db, None, ring, b.g8, b.sg, b.ag,
                         stream_dw=torch.cuda.Stream())
    assert e.value.status == F.FP8_ERR_NULL
    assert not ring.seeded

"""A training step of one FP8 linear captured as a HIP graph and replayed.

The step is the benchmark's: the paired X/W quantize, the forward GEMM with
a bf16 bias, the weight gradient (G quantized with its ring, db) and the
input gradient from G8.  Two copies of the same linear start from the same
inputs; after a seeding step run eagerly on both, one copy's step is
captured and replayed while the other runs eagerly.  Between replays the
program does its own eager work (it rescales X in both copies, so that the
rings see a changing amax) and synchronizes; every replay must give the
eager step's bytes exactly: codes, scales, amax, ring state and the bf16
outputs (the GEMMs are deterministic).  The calls record no memset nodes:
the library issues only kernels.  In the two-stream variant the backward is
fp8_linear_bwd with the dW GEMM on a second stream, which the capture takes
as a fork after the G quantize and a join at the end of the step.
"""

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from tests.gpu_util import DEV, ring_state

pytestmark = pytest.mark.gpu

FX, FG = F.FP8_E4M3, F.FP8_E5M2


class Linear:
    """Buffers, rings and the bound calls of one linear's step on a stream."""

    def __init__(self, X, W, b, G, stream, hist_len=4, side=None):
        M, K = X.shape
        N = W.shape[0]
        e = lambda *s, dt=torch.uint8: torch.empty(*s, dtype=dt, device=DEV)
        z = lambda: torch.zeros(1, dtype=torch.float32, device=DEV)
        self.X, self.W, self.b, self.G = (t.to(DEV).clone() for t in (X, W, b, G))
        self.x8, self.w8, self.g8 = e(M, K), e(N, K), e(M, N)
        self.y, self.dx, self.dw = e(M, N, dt=torch.bfloat16), e(M, K, dt=torch.bfloat16), \
            e(N, K, dt=torch.bfloat16)
        self.db = e(N, dt=torch.bfloat16)
        self.ws = e(max(1, F.fp8_db_workspace_bytes(M, N) // 4), dt=torch.float32)
        self.sx, self.sw, self.sg, self.ax, self.aw, self.ag = (z() for _ in range(6))
        self.rx, self.rw, self.rg = (F.ScaleRing(hist_len, stream=stream) for _ in range(3))
        x8q = F.Quantized(self.x8, FX, self.sx)
        w8q = F.Quantized(self.w8, FX, self.sw)
        g8q = F.Quantized(self.g8, FG, self.sg)
        self.calls = [
            F.bind_fp8_quantize_pair(self.X, self.x8, self.rx, self.sx, self.ax, self.W, self.w8,
                                     self.rw, self.sw, self.aw, FX, stream=stream),
            F.bind_fp8_linear_fwd(x8q, w8q, self.b, FX, self.y, stream=stream),
        ]
        if side is None:
            self.calls += [
                F.bind_fp8_linear_bwd_dw(self.G, FG, x8q, self.dw, self.db, self.ws, self.rg,
                                         self.g8, self.sg, self.ag, stream=stream),
                F.bind_fp8_linear_bwd_dx(g8q, FG, w8q, self.dx, stream=stream),
            ]
        else:
            # the two-stream backward: dW on side, joined back at the end
            self.calls += [
                F.bind_fp8_linear_bwd(self.G, FG, x8q, w8q, self.dx, self.dw, self.db, self.ws,
                                      self.rg, self.g8, self.sg, self.ag, stream=stream,
                                      stream_dw=side),
                lambda: stream.wait_stream(side),
            ]

    def step(self):
        for c in self.calls:
            c()

    def snapshot(self):
        out = {k: getattr(self, k).cpu().view(torch.uint8).numpy().copy()
               for k in ("x8", "w8", "g8", "y", "dx", "dw", "db", "sx", "sw", "sg", "ax", "aw",
                         "ag")}
        for name in ("rx", "rw", "rg"):
            for k, v in ring_state(getattr(self, name)).items():
                out[f"{name}.{k}"] = np.asarray(v).copy()
        return out


def _inputs(M, K, N, seed):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    return (bf(rng.standard_normal((M, K))), bf(rng.standard_normal((N, K)) * 0.02),
            bf(rng.standard_normal(N) * 0.01), bf(rng.standard_normal((M, N)) * 1e-3))


# (384, 320, 640): 128x128 tiles; (2048, 256, 4096): the 256x256 8-wave kernel.
# two_stream: the backward through fp8_linear_bwd with dW on a second stream
# (captured as a fork and a join of the graph).
@pytest.mark.parametrize("two_stream", [False, True])
@pytest.mark.parametrize("M,K,N", [(384, 320, 640), (2048, 256, 4096)])
def test_graph_replays_match_eager(M, K, N, two_stream):
    stream = torch.cuda.Stream()
    side = torch.cuda.Stream() if two_stream else None
    X0, W, b, G = _inputs(M, K, N, seed=M + N)
    eager = Linear(X0, W, b, G, stream, side=side)
    graphed = Linear(X0, W, b, G, stream, side=side)
    with torch.cuda.stream(stream):
        eager.step()  # seeding step: the first call through each ring
        graphed.step()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        graphed.step()
    torch.cuda.synchronize()

    x0 = X0.to(DEV).float()
    for i, f in enumerate((1.0, 3.0, 0.25, 8.0, 1.0)):
        with torch.cuda.stream(stream):
            xi = (x0 * f).to(torch.bfloat16)
            eager.X.copy_(xi)
            graphed.X.copy_(xi)
            eager.step()
            g.replay()
        torch.cuda.synchronize()
        a, r = eager.snapshot(), graphed.snapshot()
        for k in a:
            assert np.array_equal(a[k], r[k]), f"replay {i}: {k} differs from the eager step"


def test_unseeded_ring_refused_under_capture():
    """Whether a call seeds its ring is decided when it is issued; captured,
    the seeding pass would re-seed on every replay.  So a call that would
    seed a ring on a capturing stream fails with FP8_ERR_RING and enqueues
    nothing, and the same call succeeds eagerly afterwards."""
    x = torch.randn(256, 64, device=DEV).to(torch.bfloat16)
    q = torch.empty(256 * 64, dtype=torch.uint8, device=DEV)
    su = torch.zeros(1, dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()
    ring = F.ScaleRing(4, stream=stream)
    stream.synchronize()
    before = ring.buf.clone()
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g, stream=stream):
        q.zero_()  # the graph holds one node of its own
        try:
            F.fp8_quantize(x, FX, q, ring, su, stream=stream)
        except F.Fp8Error as exc:
            status = exc.status
    assert status == F.FP8_ERR_RING
    assert not ring.seeded
    torch.cuda.synchronize()
    assert torch.equal(ring.buf, before)
    F.fp8_quantize(x, FX, q, ring, su, stream=stream)  # eager: seeds
    stream.synchronize()
    assert ring.seeded and ring_state(ring)["idx"] == 1


def test_graph_fp8out_replays_match_eager():
    """The FP8-output GEMM in a graph: its steady state is the GEMM launch
    and the one-wave launch that folds the output ring.  Two copies of the
    call on the same codes, seeded eagerly; one captured and replayed while
    the other runs eagerly, with the operand scale changed between replays
    (so max |y| and the ring move); every replay must give the eager call's
    codes, scale, amax and ring state exactly."""
    M, K, N = 2048, 256, 4096  # the 256x256 8-wave kernel
    rng = np.random.default_rng(41)
    tab_ok = [c for c in range(256) if (c & 0x7F) != 0x7F]
    a8 = torch.from_numpy(rng.choice(tab_ok, size=(M, K)).astype(np.uint8)).to(DEV)
    b8 = torch.from_numpy(rng.choice(tab_ok, size=(N, K)).astype(np.uint8)).to(DEV)
    stream = torch.cuda.Stream()

    class Call:
        def __init__(self):
            self.sa = torch.full((1,), 3.0, dtype=torch.float32, device=DEV)
            self.sb = torch.full((1,), 5.0, dtype=torch.float32, device=DEV)
            self.c8 = torch.empty(M, N, dtype=torch.uint8, device=DEV)
            self.su = torch.zeros(1, dtype=torch.float32, device=DEV)
            self.am = torch.zeros(1, dtype=torch.float32, device=DEV)
            self.ring = F.ScaleRing(4, stream=stream)
            self.fn = F.bind_fp8_gemm_fp8out(F.Quantized(a8, FX, self.sa), F.Quantized(b8, FX, self.sb),
                                             self.c8, FX, self.ring, self.su, self.am, stream=stream)

        def snapshot(self):
            out = {k: getattr(self, k).cpu().view(torch.uint8).numpy().copy()
                   for k in ("c8", "su", "am")}
            for k, v in ring_state(self.ring).items():
                out[f"ring.{k}"] = np.asarray(v).copy()
            return out

    eager, graphed = Call(), Call()
    with torch.cuda.stream(stream):
        eager.fn()  # seeding call: the amax pass and the converting pass
        graphed.fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        graphed.fn()
    torch.cuda.synchronize()
    for i, sa in enumerate((3.0, 0.5, 12.0, 3.0)):
        with torch.cuda.stream(stream):
            eager.sa.fill_(sa)
            graphed.sa.fill_(sa)
            eager.fn()
            g.replay()
        torch.cuda.synchronize()
        a, r = eager.snapshot(), graphed.snapshot()
        for k in a:
            assert np.array_equal(a[k], r[k]), f"replay {i}: {k} differs from the eager call"


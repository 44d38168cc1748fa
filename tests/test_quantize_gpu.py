"""GPU parity of fp8_quantize against the oracle: bit-exact fp8 bytes,
scale_used, amax, and ring state (hist, idx, published scale)."""

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from oracle import fp8_oracle as O
from scaled_quantize_fp8_amd import workloads as WL
from tests.gpu_util import DEV, assert_ring_matches, f32, f32_scalar, ring_state, to_dev, u8

pytestmark = pytest.mark.gpu

FMTS = [O.E4M3, O.E5M2]


def _quant_gpu(x, fmt, ring=None):
    q = torch.empty(x.numel(), dtype=torch.uint8, device=DEV)
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    a = torch.empty(1, dtype=torch.float32, device=DEV)
    F.fp8_quantize(x, fmt, q, ring, s, a)
    torch.cuda.synchronize()
    return u8(q), f32_scalar(s), f32_scalar(a)


def _unit_ring(hist_len=16):
    """A ring whose current scale is 1.0 and that is marked seeded, so the
    quantize converts the raw values: q = enc(fl32(x * 1))."""
    r = F.ScaleRing(hist_len)
    r.c.seeded = 1
    return r


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_every_bf16_pattern(fmt):
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).to(DEV)
    q, s, _ = _quant_gpu(x, fmt, _unit_ring())
    assert s == 1.0
    assert np.array_equal(q, O.encode(f32(x), fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_every_f16_pattern(fmt):
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.float16).to(DEV)
    q, _, _ = _quant_gpu(x, fmt, _unit_ring())
    assert np.array_equal(q, O.encode(f32(x), fmt))


def _fp32_probe_values(fmt, seed=0):
    """Random bit patterns, every exponent with random mantissas, and the
    exact midpoints between adjacent codes with their fp32 neighbours."""
    g = np.random.default_rng(seed)
    parts = [g.integers(0, 2 ** 32, 3_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)]
    for e in range(256):
        m = g.integers(0, 2 ** 23, 4096, dtype=np.uint64).astype(np.uint32)
        for sgn in (0, 1):
            parts.append(((np.uint32(sgn) << 31) | (np.uint32(e) << 23) | m).view(np.float32))
    tab = O.decode_table(fmt)
    fin = np.sort(np.unique(np.abs(tab[np.isfinite(tab)])))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, [fin[-1] * (1 + 2 ** -4), fin[-1] * 1.125]]).astype(np.float32)
    near = [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))]
    near = np.concatenate(near)
    parts += [near, -near, np.array([0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)]
    return np.concatenate(parts).astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_fp32_patterns(fmt):
    xs = _fp32_probe_values(fmt)
    x = torch.from_numpy(xs).to(DEV)
    q, _, _ = _quant_gpu(x, fmt, _unit_ring())
    ref = O.encode(xs, fmt)
    bad = np.nonzero(q != ref)[0]
    assert bad.size == 0, [(float(xs[i]), hex(int(ref[i])), hex(int(q[i]))) for i in bad[:8]]


def _f32_bits(v: float) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_every_fp32_pattern_in_range(fmt):
    """Every fp32 bit pattern whose magnitude lies between half the smallest
    subnormal and twice the maximum of the format (both signs: 331M patterns
    for e4m3, 566M for e5m2), through the GPU encoder (scale 1, so the codes
    are enc(x) itself) against the oracle's encoder.  Outside that range
    every value encodes to a signed zero or saturates; those values, with
    NaN, infinities and fp32 subnormals, are covered by the seeded probes of
    test_encoder_fp32_patterns.  The oracle runs in spawned worker processes
    (numpy only) while the GPU encodes the same chunks."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import os

    from tests.encode_sweep_worker import encode_bits

    tab = O.decode_table(fmt)
    fin = np.abs(tab[np.isfinite(tab)])
    lo = _f32_bits(float(np.min(fin[fin > 0])) / 2)
    hi = _f32_bits(float(np.max(fin)) * 2)
    chunk = 1 << 24
    jobs = [(a, min(chunk, hi + 1 - a), neg) for neg in (False, True)
            for a in range(lo, hi + 1, chunk)]
    workers = max(1, min(16, os.cpu_count() or 1))
    with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as pool:
        futs = [pool.submit(encode_bits, a, n, neg, fmt) for a, n, neg in jobs]
        for (a, n, neg), fut in zip(jobs, futs):
            bits = torch.arange(a, a + n, dtype=torch.int64, device=DEV)
            if neg:
                bits -= 1 << 31  # int32 value whose bit pattern is that of a | 0x80000000
            x = bits.to(torch.int32).view(torch.float32)
            q, s, _ = _quant_gpu(x, fmt, _unit_ring())
            assert s == 1.0
            ref = fut.result()
            bad = np.nonzero(q != ref)[0]
            assert bad.size == 0, [(hex(a + int(i)), neg, hex(int(ref[i])), hex(int(q[i])))
                                   for i in bad[:8]]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 4095, 4096, 4097, 1_000_003, 9 * 2 ** 20])
def test_dynamic_quantize_matches_oracle(dtype, fmt, n):
    g = torch.Generator().manual_seed(n + 7)
    x = (torch.randn(n, generator=g) * 3.0).to(dtype).to(DEV)
    q, s, a = _quant_gpu(x, fmt, None)
    oq, os_, oa = O.quantize_step(f32(x), fmt, None)
    assert a.tobytes() == np.float32(oa).tobytes()
    assert s.tobytes() == np.float32(os_).tobytes()
    assert np.array_equal(q, oq)


def test_unaligned_input_and_output():
    base = (torch.randn(10_000, generator=torch.Generator().manual_seed(3)) * 5).to(torch.bfloat16)
    xd = base.to(DEV)[1:9_001]  # 2-byte offset: scalar path
    qbuf = torch.empty(9_003, dtype=torch.uint8, device=DEV)
    q = qbuf[3:9_003]
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    a = torch.empty(1, dtype=torch.float32, device=DEV)
    F.fp8_quantize(xd, O.E4M3, q, None, s, a)
    torch.cuda.synchronize()
    oq, os_, oa = O.quantize_step(f32(xd), O.E4M3, None)
    assert np.array_equal(u8(q), oq) and f32_scalar(s) == os_ and f32_scalar(a) == oa


def _ring_steps(factors, hist_len, fmt=O.E4M3, dtype=torch.bfloat16, shape=(128, 256)):
    x0 = WL.normal_bf16(shape, 1.0, WL.seed_for(0, "X")).to(dtype)
    ring = F.ScaleRing(hist_len)
    oring = O.ScaleRing(hist_len)
    for t, c in enumerate(factors):
        xt = (x0.float() * c).to(dtype).to(DEV)
        q, s, a = _quant_gpu(xt, fmt, ring)
        oq, os_, oa = O.quantize_step(f32(xt), fmt, oring)
        assert s.tobytes() == np.float32(os_).tobytes(), (t, s, os_)
        assert a.tobytes() == np.float32(oa).tobytes(), t
        assert np.array_equal(q, oq.reshape(-1)), t
        assert_ring_matches(ring, oring)
    return ring, oring


def test_ring_tiny_sequence():
    _ring_steps(WL.TINY_STEP_FACTORS, 16)


def test_ring_eviction_h2():
    _ring_steps((1.0, 4.0, 0.25, 16.0, 1.0, 1.0), 2)


@pytest.mark.parametrize("fmt", FMTS)
def test_ring_random_amax_large_window(fmt):
    g = np.random.default_rng(5)
    _ring_steps(list(10.0 ** g.uniform(-3, 3, 40)), 1024, fmt=fmt, dtype=torch.float32,
                shape=(300, 77))


def test_ring_many_blocks_single_fold():
    """Thousands of blocks take tickets; exactly one folds per launch."""
    _ring_steps((1.0, 2.0, 0.5), 16, shape=(4096, 6912))


def test_ring_repeat_runs_bit_identical():
    outs = []
    for _ in range(20):
        ring, _ = _ring_steps((1.0, 8.0), 4, shape=(1024, 1536))
        outs.append(ring.buf.cpu().numpy().tobytes())
    assert all(o == outs[0] for o in outs)


def test_ring_resume_from_byte_copy():
    x0 = WL.normal_bf16((512, 512), 1.0, 11)
    factors = (1.0, 3.0, 0.5, 7.0, 0.1)
    ring = F.ScaleRing(8)
    got = []
    snap = None
    for t, c in enumerate(factors):
        got.append(_quant_gpu((x0.float() * c).to(torch.bfloat16).to(DEV), O.E4M3, ring))
        if t == 1:
            snap = (ring.buf.clone(), ring.c.seeded)
    fresh = F.ScaleRing(8)
    fresh.buf.copy_(snap[0])
    fresh.c.seeded = snap[1]
    for t, c in enumerate(factors[2:], start=2):
        q, s, a = _quant_gpu((x0.float() * c).to(torch.bfloat16).to(DEV), O.E4M3, fresh)
        assert np.array_equal(q, got[t][0]) and s == got[t][1] and a == got[t][2]
    assert torch.equal(fresh.buf, ring.buf)


def test_ring_zero_size_folds_zero():
    ring = F.ScaleRing(4)
    oring = O.ScaleRing(4)
    x = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    for _ in range(2):
        _, s, a = _quant_gpu(x, O.E4M3, ring)
        _, os_, oa = O.quantize_step(np.zeros(0, np.float32), O.E4M3, oring)
        assert s == os_ and a == oa
        assert_ring_matches(ring, oring)


def test_nan_and_inf_inputs():
    x = torch.tensor([1.0, float("nan"), -float("nan"), float("inf"), -float("inf"), -0.0, 2.5e-9,
                      -3.0e-9, 500.0, -70000.0] * 7, dtype=torch.float32, device=DEV)
    for fmt in FMTS:
        q, _, _ = _quant_gpu(x, fmt, _unit_ring())
        assert np.array_equal(q, O.encode(f32(x), fmt))


@pytest.mark.parametrize("wl_name", ["dim1536_m2048", "generic_m4096"])
def test_full_size_layer_tensors(wl_name):
    """Every operand of the largest workloads, quantized by the GPU, equals
    the oracle byte for byte (delayed ring seeded on first use, then one
    steady-state step; or dynamic for the generic workload)."""
    wl = WL.WORKLOADS[wl_name]
    for li in range(len(wl.linears)):
        X, W, b, G = WL.layer_inputs(wl, li)
        for name, t, fmt in (("X", X, O.E4M3), ("W", W, O.E4M3), ("G", G, O.E5M2)):
            xd = t.to(DEV)
            ring = F.ScaleRing(wl.hist_len) if wl.delayed else None
            oring = O.ScaleRing(wl.hist_len) if wl.delayed else None
            for step in range(2 if wl.delayed else 1):
                q, s, a = _quant_gpu(xd, fmt, ring)
                oq, os_, oa = O.quantize_step(f32(xd), fmt, oring)
                assert s == os_ and a == oa, (wl_name, li, name, step)
                assert np.array_equal(q, oq.reshape(-1)), (wl_name, li, name, step)
            del xd


@pytest.mark.parametrize("dtypes", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("hist", [(16, 16), (16, 100)])
def test_quantize_pair_matches_two_rings(dtypes, hist):
    """fp8_quantize_pair over several delayed steps: step 0 seeds both rings
    (two launches); later steps with matching input types run as one launch.
    Every step matches the oracle for both tensors: bytes, scale_used, amax
    and ring state.  hist: the two windows; two of 16 fold in a one-wave
    launch after the paired launch, a 100-entry one makes both rings fold in
    the paired launch's last-block elections."""
    shapes = ((2048, 1536), (6912, 1536)) if dtypes[0] == dtypes[1] else ((333, 77), (4097, 3))
    x0 = WL.normal_bf16(shapes[0], 1.0, 21).float()
    x1 = WL.normal_bf16(shapes[1], 0.02, 22).float()
    rings = [F.ScaleRing(hist[0]), F.ScaleRing(hist[1])]
    orings = [O.ScaleRing(hist[0]), O.ScaleRing(hist[1])]
    for t, (c0, c1) in enumerate(((1.0, 1.0), (4.0, 0.5), (0.25, 2.0), (1.0, 1.0))):
        xs = [(x0 * c0).to(dtypes[0]), (x1 * c1).to(dtypes[1])]
        q = [torch.empty(x.numel(), dtype=torch.uint8, device=DEV) for x in xs]
        su = [torch.empty(1, dtype=torch.float32, device=DEV) for _ in xs]
        am = [torch.empty(1, dtype=torch.float32, device=DEV) for _ in xs]
        xd = [x.to(DEV) for x in xs]
        F.fp8_quantize_pair(xd[0], q[0], rings[0], su[0], am[0], xd[1], q[1], rings[1], su[1],
                            am[1], O.E4M3)
        torch.cuda.synchronize()
        for i in range(2):
            oq, os_, oa = O.quantize_step(f32(xs[i]), O.E4M3, orings[i])
            assert np.array_equal(u8(q[i]), oq.reshape(-1)), (t, i)
            assert f32_scalar(su[i]).tobytes() == np.float32(os_).tobytes(), (t, i)
            assert f32_scalar(am[i]).tobytes() == np.float32(oa).tobytes(), (t, i)
            assert_ring_matches(rings[i], orings[i])


def test_quantize_pair_rejects_one_ring_twice():
    ring = F.ScaleRing(16)
    x = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    q = [torch.empty(64, dtype=torch.uint8, device=DEV) for _ in range(2)]
    su = [torch.empty(1, dtype=torch.float32, device=DEV) for _ in range(2)]
    before = ring.buf.clone()
    with pytest.raises(F.Fp8Error):
        F.fp8_quantize_pair(x, q[0], ring, su[0], None, x, q[1], ring, su[1], None, O.E4M3)
    torch.cuda.synchronize()
    assert torch.equal(ring.buf, before)


# ---------------------------------------------------------------- fp8_quantize_2d
SHAPES_2D = [(2048, 1536), (333, 77), (64, 64), (1, 1000), (1000, 1), (130, 24), (96, 4104)]


@pytest.mark.parametrize("shape", SHAPES_2D)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_2d_dual_matches_oracle(shape, dtype):
    """Dual orientation over three delayed steps: q is the oracle's codes,
    qt their transpose, and scale, amax and ring match every step."""
    rows, cols = shape
    x0 = WL.normal_bf16(shape, 1.0, 31).float()
    ring, oring = F.ScaleRing(16), O.ScaleRing(16)
    for t, c in enumerate((1.0, 8.0, 0.5)):
        x = (x0 * c).to(dtype)
        q = torch.empty(rows, cols, dtype=torch.uint8, device=DEV)
        qt = torch.empty(cols, rows, dtype=torch.uint8, device=DEV)
        su = torch.empty(1, dtype=torch.float32, device=DEV)
        am = torch.empty(1, dtype=torch.float32, device=DEV)
        F.fp8_quantize_2d(x.to(DEV), O.E4M3, F.FP8_QUANT_DUAL, q, qt, ring, su, am)
        torch.cuda.synchronize()
        oq, os_, oa = O.quantize_step(f32(x), O.E4M3, oring)
        oq = oq.reshape(rows, cols)
        assert np.array_equal(u8(q), oq), t
        assert np.array_equal(u8(qt), oq.T), t
        assert f32_scalar(su).tobytes() == np.float32(os_).tobytes(), t
        assert f32_scalar(am).tobytes() == np.float32(oa).tobytes(), t
        assert_ring_matches(ring, oring)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_2d_transposed_only_dynamic(fmt):
    rows, cols = 517, 264
    x = (torch.randn(rows, cols, generator=torch.Generator().manual_seed(4)) * 3).to(torch.bfloat16)
    qt = torch.empty(cols, rows, dtype=torch.uint8, device=DEV)
    su = torch.empty(1, dtype=torch.float32, device=DEV)
    am = torch.empty(1, dtype=torch.float32, device=DEV)
    F.fp8_quantize_2d(x.to(DEV), fmt, F.FP8_QUANT_TRANSPOSED, None, qt, None, su, am)
    torch.cuda.synchronize()
    oq, os_, oa = O.quantize_step(f32(x), fmt, None)
    assert np.array_equal(u8(qt), oq.reshape(rows, cols).T)
    assert f32_scalar(su) == np.float32(os_) and f32_scalar(am) == np.float32(oa)


def test_quantize_2d_rows_equals_quantize():
    x = WL.normal_bf16((300, 200), 1.0, 41).to(DEV)
    q1, s1, a1 = _quant_gpu(x.reshape(-1), O.E5M2)
    q2 = torch.empty(300, 200, dtype=torch.uint8, device=DEV)
    su = torch.empty(1, dtype=torch.float32, device=DEV)
    am = torch.empty(1, dtype=torch.float32, device=DEV)
    F.fp8_quantize_2d(x, O.E5M2, F.FP8_QUANT_ROWS, q2, None, None, su, am)
    torch.cuda.synchronize()
    assert np.array_equal(u8(q2).reshape(-1), q1) and f32_scalar(su) == s1


def test_weight_gradient_from_transposed_operands():
    """dW = G8^T X8 run k-contiguous: quantize G and X transposed, then
    fp8_gemm with G8^T [N, M] and X8^T [K, M]; checked against the oracle
    and against the crosswise dW of fp8_linear_bwd_dw on the same codes."""
    from tests.gpu_util import check_gemm, bf16_bits
    M, N, K = 2048, 1536, 6912
    G = WL.normal_bf16((M, N), 1e-3, 51)
    X = WL.normal_bf16((M, K), 1.0, 52)
    g8t = torch.empty(N, M, dtype=torch.uint8, device=DEV)
    x8t = torch.empty(K, M, dtype=torch.uint8, device=DEV)
    sg, sx = (torch.empty(1, dtype=torch.float32, device=DEV) for _ in range(2))
    ag, ax = (torch.empty(1, dtype=torch.float32, device=DEV) for _ in range(2))
    F.fp8_quantize_2d(G.to(DEV), O.E5M2, F.FP8_QUANT_TRANSPOSED, None, g8t, None, sg, ag)
    F.fp8_quantize_2d(X.to(DEV), O.E4M3, F.FP8_QUANT_TRANSPOSED, None, x8t, None, sx, ax)
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm(F.Quantized(g8t, O.E5M2, sg), F.Quantized(x8t, O.E4M3, sx), dw)
    # the crosswise path on the same codes (transposed back)
    g8 = g8t.t().contiguous()
    x8 = x8t.t().contiguous()
    dw2 = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    F.fp8_linear_bwd_dw(F.Quantized(g8, O.E5M2, sg), O.E5M2, F.Quantized(x8, O.E4M3, sx), dw2)
    torch.cuda.synchronize()
    rows = np.random.default_rng(3).choice(N, 48, replace=False)
    ref = O.linear_bwd_dw(u8(g8)[:, rows], O.E5M2, u8(x8), O.E4M3, f32_scalar(sg), f32_scalar(sx))
    check_gemm(bf16_bits(dw)[rows], ref, "k-contiguous dW")
    check_gemm(bf16_bits(dw2)[rows], ref, "crosswise dW")

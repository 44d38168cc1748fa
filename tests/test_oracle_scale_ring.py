"""Pins of the oracle's amax, scale function and delayed-scaling ring (CPU).

Hand-worked sequences: the ring's behaviour follows from the pages'
description (seed from the first amax, quantize with the scale read before
the fold, fold amax into hist[idx], publish S(max(hist))).  With inputs
X_t = c_t * X0 for powers of two c_t, every scale is S(a0) times a power of
two, so the whole sequence is fixed in closed form.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as O
from scaled_quantize_fp8_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _x0(shape=(128, 256), seed=0):
    return WL.normal_bf16(shape, 1.0, WL.seed_for(seed, "X")).float().numpy()


# ---------------------------------------------------------------- amax / S

def test_amax_brute_force():
    x = _x0((7, 13))
    best = 0.0
    for v in x.ravel():
        best = max(best, abs(float(v)))
    assert O.amax(x) == np.float32(best)
    assert O.amax(np.zeros((0,), np.float32)) == 0.0
    assert O.amax(np.array([-3.0, 2.0], np.float32)) == 3.0


def test_amax_nan_propagates_like_torch():
    """A NaN among the inputs: the pages are silent; the reading taken is
    that it propagates (IEEE 754-2019 maximum returns NaN when an operand is
    NaN).  Pinned against torch's CPU amax, which propagates NaN, at every
    position of a small tensor and with either sign, and against the
    infinities, which are ordinary values of the max."""
    base = np.array([0.5, -3.0, 2.0, -0.0, 1e-30, 7.25], np.float32)
    for i in range(base.size):
        for nan in (np.float32(np.nan), np.float32(-np.nan)):
            x = base.copy()
            x[i] = nan
            ref = torch.from_numpy(np.abs(x)).amax().item()
            assert np.isnan(ref) and np.isnan(O.amax(x)), i
    for inf in (np.inf, -np.inf):
        x = base.copy()
        x[2] = inf
        assert O.amax(x) == np.float32(torch.from_numpy(np.abs(x)).amax().item()) == np.inf
    # and the scale of a NaN amax keeps the previous one, like any amax that
    # is not finite and positive
    assert O.scale_from_amax(np.float32(np.nan), O.E4M3, 5.0) == 5.0


def test_scale_closed_forms():
    assert O.scale_from_amax(1.0, O.E4M3, 7.0) == 448.0
    assert O.scale_from_amax(448.0, O.E4M3, 7.0) == 1.0
    assert O.scale_from_amax(57344.0, O.E5M2, 7.0) == 1.0
    assert O.scale_from_amax(2.0, O.E5M2, 7.0) == 28672.0
    # degenerate amax keeps the previous scale
    for bad in (0.0, np.inf, np.nan, -1.0):
        assert O.scale_from_amax(bad, O.E4M3, 7.0) == 7.0
    # quotient overflow keeps the previous scale
    assert O.scale_from_amax(np.float32(1e-45), O.E4M3, 3.0) == 3.0
    # IEEE fp32 division, correctly rounded
    a = np.float32(0.3)
    assert O.scale_from_amax(a, O.E4M3, 1.0) == np.float32(np.float64(448.0) / np.float64(a))
    # powers of two commute exactly
    g = np.random.default_rng(3)
    for a in g.uniform(0.01, 100, 200).astype(np.float32):
        s = O.scale_from_amax(a, O.E4M3, 1.0)
        assert O.scale_from_amax(a * np.float32(4), O.E4M3, 1.0) == s / np.float32(4)


def test_quantize_dequantize_within_half_step():
    x = _x0()
    for fmt in O.FORMATS:
        q, s, a = O.quantize_step(x, fmt, None)
        back = O.decode_array(q, fmt) / float(s)
        # relative rounding error of RNE with m mantissa bits, plus the
        # subnormal absolute step
        m = {O.E4M3: 3, O.E5M2: 2}[fmt]
        sub = {O.E4M3: 2.0 ** -9, O.E5M2: 2.0 ** -16}[fmt]
        err = np.abs(back - x)
        assert np.all(err <= np.abs(x) * 2.0 ** -(m + 1) + sub / 2 / float(s) * 1.0000001)
        assert np.abs(O.decode_array(q, fmt)).max() <= O.fmt_max(fmt)
        assert a == np.abs(x).max()


# ---------------------------------------------------------------- ring

def _run(factors, hist_len, fmt=O.E4M3):
    x0 = _x0()
    ring = O.ScaleRing(hist_len)
    out = []
    for c in factors:
        xt = (x0 * np.float32(c)).astype(np.float32)
        q, s, a = O.quantize_step(xt, fmt, ring)
        out.append((q, s, a, ring.copy()))
    return x0, out


def test_ring_tiny_sequence_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "ring_sequences.json")))["tiny_h16"]
    x0, out = _run(g["factors"], 16)
    a0 = O.amax(x0)
    S = O.scale_from_amax(a0, O.E4M3, 1.0)
    assert [o[1] for o in out] == [S * np.float32(f) for f in g["s_used_over_S"]]
    last = out[-1][3]
    assert last.scale == S * np.float32(g["published_over_S"])
    assert last.idx == g["idx"]
    exp_hist = [a0 * np.float32(h) for h in g["hist_over_a0"]] + [0.0] * (16 - len(g["hist_over_a0"]))
    assert np.array_equal(last.hist, np.array(exp_hist, np.float32))
    # 16x * S/4 == 4x * S exactly: step 3 reproduces step 1 byte for byte
    assert np.array_equal(out[3][0], out[1][0])


def test_ring_eviction_h2_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "ring_sequences.json")))["eviction_h2"]
    x0, out = _run(g["factors"], 2)
    S = O.scale_from_amax(O.amax(x0), O.E4M3, 1.0)
    assert [o[1] for o in out] == [S * np.float32(f) for f in g["s_used_over_S"]]
    assert out[-1][3].scale == S * np.float32(g["published_over_S"])


def test_ring_seed_uses_first_amax_not_one():
    x = _x0() * np.float32(0.01)
    ring = O.ScaleRing(16)
    _, s, a = O.quantize_step(x, O.E4M3, ring)
    assert s == O.scale_from_amax(a, O.E4M3, 1.0) and s != 1.0
    assert ring.seeded


def test_ring_snapshot_does_not_leak_next_scale():
    """The scale a step quantizes with is the one it read, not the one its
    fold publishes: dec(q)/s_used reproduces x, dec(q)/s_published does not
    (the non-leak regression invariant of the pages)."""
    x0, out = _run((1.0, 4.0, 0.25, 16.0), 16)
    leaks_detectable = 0
    for t, (q, s, a, ring_after) in enumerate(out):
        xt = x0 * np.float32((1.0, 4.0, 0.25, 16.0)[t])
        dec = O.decode_array(q, O.E4M3)
        # delayed scaling saturates the elements whose |x*s| passed the max
        sat = np.abs(xt.astype(np.float64) * float(s)) >= 448.0
        assert np.all(np.abs(dec[sat]) == 448.0)
        ok = ~sat & (np.abs(xt) > 2.0 ** -6 / float(s))  # normal range
        back = dec[ok] / float(s)
        assert np.all(np.abs(back - xt[ok]) <= np.abs(xt[ok]) * 2.0 ** -4)
        leaked = dec[ok] / float(ring_after.scale)
        if np.median(np.abs(leaked - xt[ok]) / np.abs(xt[ok])) > 0.5:
            leaks_detectable += 1
    assert leaks_detectable >= 2  # steps 1 and 3 publish a new scale


def test_ring_dynamic_matches_per_step_scale():
    x0 = _x0()
    for c in (1.0, 4.0, 1e-3):
        x = x0 * np.float32(c)
        q, s, a = O.quantize_step(x, O.E5M2, None)
        assert s == O.scale_from_amax(O.amax(x), O.E5M2, 1.0)


def test_ring_resume_from_copy_is_bit_exact():
    x0 = _x0()
    factors = (1.0, 3.0, 0.5, 7.0, 0.1)
    ring = O.ScaleRing(4)
    outs, snap = [], None
    for t, c in enumerate(factors):
        outs.append(O.quantize_step(x0 * np.float32(c), O.E4M3, ring))
        if t == 1:
            snap = ring.copy()
    for t, c in enumerate(factors[2:], start=2):
        q, s, a = O.quantize_step(x0 * np.float32(c), O.E4M3, snap)
        assert s == outs[t][1] and np.array_equal(q, outs[t][0])
    assert snap.scale == ring.scale and np.array_equal(snap.hist, ring.hist)


def test_quantize_torch_crosscheck():
    """q = enc(fl32(x*s)) agrees with torch's fp32 multiply + float8 cast
    wherever the product is in range (torch does not saturate)."""
    x = _x0()
    for fmt, tdt in ((O.E4M3, torch.float8_e4m3fn), (O.E5M2, torch.float8_e5m2)):
        s = O.scale_from_amax(O.amax(x), fmt, 1.0)
        q = O.quantize_with_scale(x, s, fmt)
        ref = (torch.from_numpy(x) * torch.tensor(s, dtype=torch.float32)).to(tdt)
        assert np.array_equal(ref.view(torch.uint8).numpy(), q)

"""GPU parity of the FP8-in / FP8-out GEMM (fp8_gemm_fp8out) against the
oracle's gemm_fp8out.

Exact cases (small-integer operands and bias, power-of-two scales: the fp32
accumulation is exact, so the GEMM output equals the oracle's value) compare
codes, scale, amax and ring state bit for bit over several steps of one
ring, the first of which seeds it through the extra amax pass.  Random cases
check what GEMM rounding leaves unique: amax within the GEMM tolerance of
the oracle's; the scale and ring update exactly as the oracle's rules give
them from the GPU's own amax; and each code within the codes that the
oracle's encoder gives at the two ends of the element's tolerance interval
(the encoder is monotone, so that interval bounds every correct code).
"""

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from oracle import fp8_oracle as O
from tests.gpu_util import (DEV, TIGHT_REL, assert_ring_matches, f32_scalar, ring_state,
                            scalar_dev, to_dev, u8)

pytestmark = pytest.mark.gpu

_INT_CODES = {  # value -> code of the small integers used by the exact cases
    O.E4M3: {0: 0x00, 1: 0x38, 2: 0x40, -1: 0xB8, -2: 0xC0},
    O.E5M2: {0: 0x00, 1: 0x3C, 2: 0x40, -1: 0xBC, -2: 0xC0},
}


def _int_codes(shape, fmt, rng):
    vals = rng.integers(-2, 3, size=shape)
    lut = _INT_CODES[fmt]
    return np.vectorize(lambda v: lut[int(v)], otypes=[np.uint8])(vals)


def _rand_codes(shape, fmt, rng):
    tab = O.decode_table(fmt)
    fin = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    return rng.choice(fin, size=shape)


def _bf16(vals):
    t = torch.from_numpy(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t, t.view(torch.int16).numpy().view(np.uint16)


def _run(a8, fa, b8, fb, sa, sb, bias_t, fmt_out, ring):
    M, N = a8.shape[0], b8.shape[0]
    c8 = torch.empty(M, N, dtype=torch.uint8, device=DEV)
    su = torch.zeros(1, dtype=torch.float32, device=DEV)
    am = torch.zeros(1, dtype=torch.float32, device=DEV)
    F.fp8_gemm_fp8out(F.Quantized(to_dev(a8), fa, scalar_dev(sa)),
                      F.Quantized(to_dev(b8), fb, scalar_dev(sb)), c8, fmt_out, ring, su, am,
                      bias=None if bias_t is None else bias_t.to(DEV))
    torch.cuda.synchronize()
    return u8(c8), f32_scalar(su), f32_scalar(am)


# (160, 384, 272): a ragged block row (160 = 128 + 32), three block columns;
# (1024, 256, 1536): 96 blocks, more than the 64 election groups;
# (2000, 256, 4096): 128 tiles of 256x256 (the 8-wave kernel), a ragged last
# tile row (2000 = 7 x 256 + 208).  H: a window of 4 (the steady state folds
# in a one-wave launch after the GEMM) and of 100 (longer than a wave: the
# GEMM's last block folds).
@pytest.mark.parametrize("fa,fb,M,K,N", [(O.E4M3, O.E4M3, 160, 384, 272),
                                         (O.E5M2, O.E4M3, 160, 384, 272),
                                         (O.E4M3, O.E4M3, 1024, 256, 1536),
                                         (O.E4M3, O.E5M2, 2000, 256, 4096)])
@pytest.mark.parametrize("fmt_out", [O.E4M3, O.E5M2])
@pytest.mark.parametrize("H", [4, 100])
def test_fp8out_exact_steps(fa, fb, M, K, N, fmt_out, H):
    rng = np.random.default_rng(7 + 3 * fa + fmt_out + M)
    b8 = _int_codes((N, K), fb, rng)
    ring, oring = F.ScaleRing(H), O.ScaleRing(H)
    for step in range(4):
        a8 = _int_codes((M, K), fa, rng)
        bias_t, bias_bits = _bf16(rng.integers(-8, 9, size=N) * 0.5)
        q, su, am = _run(a8, fa, b8, fb, 2.0, 4.0, bias_t, fmt_out, ring)
        oq, osu, oam, _ = O.gemm_fp8out(a8, fa, b8, fb, 2.0, 4.0,
                                        O.bias_values(bias_bits, "bf16"), fmt_out, oring)
        assert np.array_equal(q, oq), f"step {step}: codes differ"
        assert su == osu and am == oam, (step, su, osu, am, oam)
        assert_ring_matches(ring, oring)


# A NaN code in a row of A makes that row of y NaN: its codes are 0x7F with
# a sign (the sign of a NaN the GEMM makes is not fixed), every other code
# is exact; amax is NaN, the window then holds a NaN and the scale stays
# where it was.  (160, 384, 272): 128x128 blocks, ragged; (2000, 256, 4096):
# 256x256 blocks, inside tiles and a ragged tile row.
@pytest.mark.parametrize("M,K,N", [(160, 384, 272), (2000, 256, 4096)])
@pytest.mark.parametrize("fmt_out", [O.E4M3, O.E5M2])
def test_fp8out_nan_rows(M, K, N, fmt_out):
    fa = fb = O.E4M3
    rng = np.random.default_rng(29 + fmt_out + M)
    b8 = _int_codes((N, K), fb, rng)
    ring, oring = F.ScaleRing(4), O.ScaleRing(4)
    for step in range(4):
        a8 = _int_codes((M, K), fa, rng)
        if step in (1, 2):
            for r in (0, M // 2 + step, M - 1):
                a8[r, 3 + step] = 0x7F  # an e4m3 NaN code
        bias_t, bias_bits = _bf16(rng.integers(-8, 9, size=N) * 0.5)
        q, su, am = _run(a8, fa, b8, fb, 2.0, 4.0, bias_t, fmt_out, ring)
        oq, osu, oam, ref = O.gemm_fp8out(a8, fa, b8, fb, 2.0, 4.0,
                                          O.bias_values(bias_bits, "bf16"), fmt_out, oring)
        nan = np.isnan(ref.r)
        assert nan.any() == (step in (1, 2))
        assert np.all((q[nan] & 0x7F) == 0x7F), f"step {step}: NaN outputs not coded as NaN"
        assert np.array_equal(q[~nan], oq[~nan]), f"step {step}: codes differ"
        assert su == osu, (step, su, osu)
        assert (np.isnan(am) and np.isnan(oam)) or am == oam, (step, am, oam)
        st = ring_state(ring)
        assert st["scale"].tobytes() == np.float32(oring.scale).tobytes(), (step, st["scale"])
        assert st["idx"] == oring.idx
        oh = oring.hist.astype(np.float32)
        assert np.array_equal(np.isnan(st["hist"]), np.isnan(oh))
        assert st["hist"][~np.isnan(oh)].tobytes() == oh[~np.isnan(oh)].tobytes()
        assert st["top_amax"] == 0 and st["top_count"] == 0
        assert not st["group_count"].any() and not st["group_amax"].any()


# (200, 640, 528): 128x128 blocks (4 waves, two per CU), ragged rows;
# (2048, 1536, 6912): the up projection's forward, 216 tiles of 256x256 (the
# 8-wave kernel and its fp8 epilogue), every element compared
@pytest.mark.parametrize("M,K,N", [(200, 640, 528), (2048, 1536, 6912)])
@pytest.mark.parametrize("fmt_out", [O.E4M3, O.E5M2])
def test_fp8out_random_within_tolerance(fmt_out, M, K, N):
    rng = np.random.default_rng(11 + fmt_out + M)
    b8 = _rand_codes((N, K), O.E4M3, rng)
    bias_t, bias_bits = _bf16(rng.standard_normal(N))
    beta = O.bias_values(bias_bits, "bf16")
    ring = F.ScaleRing(4)
    for step in range(3):
        a8 = _rand_codes((M, K), O.E4M3, rng)
        before = ring_state(ring)
        q, su, am = _run(a8, O.E4M3, b8, O.E4M3, 3.0, 5.0, bias_t, fmt_out, ring)
        ref = O.linear_fwd(a8, b8, O.E4M3, 3.0, 5.0, beta)
        tol = O.gemm_tolerance(ref, TIGHT_REL)
        # amax: the max of values each within its tolerance of the reference
        amax_ref = np.max(np.abs(ref.r))
        assert abs(float(am) - amax_ref) <= float(np.max(tol)), (step, am, amax_ref)
        # the scale used and the ring update, exactly, from the GPU's amax
        if step == 0:
            assert su == O.scale_from_amax(am, fmt_out, np.float32(1.0))
        else:
            assert su == before["scale"]
        after = ring_state(ring)
        idx = before["idx"]
        hist = before["hist"].copy()
        hist[idx] = am
        assert after["hist"].tobytes() == hist.tobytes()
        assert after["idx"] == (idx + 1) % 4
        assert after["scale"] == O.scale_from_amax(np.max(hist), fmt_out, su)
        # codes: between the encodings of the tolerance interval's ends
        with np.errstate(over="ignore"):
            lo = O.encode(((ref.r - tol).astype(np.float32) * su).astype(np.float32), fmt_out)
            hi = O.encode(((ref.r + tol).astype(np.float32) * su).astype(np.float32), fmt_out)
        dv, dlo, dhi = (O.decode_array(c, fmt_out) for c in (q, lo, hi))
        bad = (dv < dlo) | (dv > dhi)
        assert not bad.any(), f"step {step}: {bad.sum()} codes outside their interval"


def test_fp8out_errors():
    M, K, N = 32, 64, 48
    a = F.Quantized(torch.zeros(M, K, dtype=torch.uint8, device=DEV), O.E4M3, scalar_dev(1.0))
    b = F.Quantized(torch.zeros(N, K, dtype=torch.uint8, device=DEV), O.E4M3, scalar_dev(1.0))
    su = torch.zeros(1, dtype=torch.float32, device=DEV)
    c8 = torch.zeros(M, N, dtype=torch.uint8, device=DEV)
    ring = F.ScaleRing(4)
    with pytest.raises(F.Fp8Error) as e:  # no ring
        F.fp8_gemm_fp8out(a, b, c8, O.E4M3, None, su)
    assert e.value.status == F.FP8_ERR_NULL
    bad_n = F.Quantized(torch.zeros(40, K, dtype=torch.uint8, device=DEV), O.E4M3,
                        scalar_dev(1.0))
    with pytest.raises(F.Fp8Error) as e:  # N not a multiple of 16
        F.fp8_gemm_fp8out(a, bad_n, torch.zeros(M, 40, dtype=torch.uint8, device=DEV), O.E4M3,
                          ring, su)
    assert e.value.status == F.FP8_ERR_SHAPE
    with pytest.raises(F.Fp8Error) as e:  # scale_used inside the ring header
        F.fp8_gemm_fp8out(a, b, c8, O.E4M3, ring, ring.buf[:4].view(torch.float32))
    assert e.value.status == F.FP8_ERR_RING
    assert not ring.seeded  # nothing ran

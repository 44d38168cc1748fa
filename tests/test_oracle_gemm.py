"""Pins of the oracle's three GEMMs, fused bias and bias gradient (CPU).

Checked against exact rational arithmetic (tiny shapes, every index written
out as a loop so a transposed operand or wrong index fails), torch's CPU
float64 matmul over torch-decoded float8 operands (an independent decoder
and product), closed forms (identity weight, constant gradient) and the
pages' statement that the fused bias is within one bf16 ulp of the split
path.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as O

TF8 = {O.E4M3: torch.float8_e4m3fn, O.E5M2: torch.float8_e5m2}


def _codes(shape, fmt, rng):
    """Random finite codes of the format."""
    tab = O.decode_table(fmt)
    finite = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    return rng.choice(finite, size=shape)


def _frac(code, fmt):
    return Fraction(O.decode(int(code), fmt))


def _bf16_of_fraction(fr: Fraction) -> int:
    """Exact RNE of a rational to bf16 bits (independent of O.bf16_bits)."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    sp = Fraction(2) ** (e - 7)
    q = a / sp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = np.array([float(fl * sp)], np.float32).view(np.uint32)[0]
    return sign | int(v >> 16)


# ---------------------------------------------------------------- exact

@pytest.mark.parametrize("fmt_a,fmt_b", [(O.E4M3, O.E4M3), (O.E5M2, O.E4M3)])
def test_three_gemms_exact_rational_tiny(fmt_a, fmt_b):
    rng = np.random.default_rng(11)
    M, N, K = 3, 5, 7
    sa, sb = np.float32(3.5), np.float32(0.625)
    # forward: Y[m,n] = sum_k x[m,k] w[n,k] / (sx sw) + b[n]   (both fmt_b)
    x8 = _codes((M, K), fmt_b, rng)
    w8 = _codes((N, K), fmt_b, rng)
    bias = rng.standard_normal(N).astype(np.float32)
    bias_bits = O.bf16_bits(bias.astype(np.float64))
    ref = O.linear_fwd(x8, w8, fmt_b, sa, sb, O.bias_values(bias_bits, "bf16"))
    for m in range(M):
        for n in range(N):
            acc = sum(_frac(x8[m, k], fmt_b) * _frac(w8[n, k], fmt_b) for k in range(K))
            exact = acc / (Fraction(float(sa)) * Fraction(float(sb))) + \
                Fraction(float(O.bf16_value(bias_bits[n])))
            assert ref.y_bits[m, n] == _bf16_of_fraction(exact)
            assert abs(Fraction(float(ref.r[m, n])) - exact) <= abs(exact) * Fraction(1, 2**50)
    # dX[m,k] = sum_n g[m,n] w[n,k] / (sg sw)
    g8 = _codes((M, N), fmt_a, rng)
    ref = O.linear_bwd_dx(g8, fmt_a, w8, fmt_b, sa, sb)
    for m in range(M):
        for k in range(K):
            acc = sum(_frac(g8[m, n], fmt_a) * _frac(w8[n, k], fmt_b) for n in range(N))
            exact = acc / (Fraction(float(sa)) * Fraction(float(sb)))
            assert ref.y_bits[m, k] == _bf16_of_fraction(exact)
    # dW[n,k] = sum_m g[m,n] x[m,k] / (sg sx)
    ref = O.linear_bwd_dw(g8, fmt_a, x8, fmt_b, sa, sb)
    for n in range(N):
        for k in range(K):
            acc = sum(_frac(g8[m, n], fmt_a) * _frac(x8[m, k], fmt_b) for m in range(M))
            exact = acc / (Fraction(float(sa)) * Fraction(float(sb)))
            assert ref.y_bits[n, k] == _bf16_of_fraction(exact)


def test_fp64_accumulation_exact_for_e4m3():
    """e4m3 values are multiples of 2^-9 below 2^9: with K = 4096 every partial
    sum fits 53 bits, so the fp64 matmul equals the exact integer sum."""
    rng = np.random.default_rng(5)
    x8 = _codes((4, 4096), O.E4M3, rng)
    w8 = _codes((3, 4096), O.E4M3, rng)
    X = O.decode_array(x8, O.E4M3)
    W = O.decode_array(w8, O.E4M3)
    Xi = (X * 2 ** 9).astype(np.int64)
    Wi = (W * 2 ** 9).astype(np.int64)
    exact = (Xi[:, None, :] * Wi[None, :, :]).sum(-1)
    ref = O.linear_fwd(x8, w8, O.E4M3, 1.0, 1.0)
    assert np.array_equal(ref.r * 2 ** 18, exact.astype(np.float64))


# ---------------------------------------------------------------- torch

@pytest.mark.parametrize("which", ["fwd", "dx", "dw"])
def test_gemms_match_torch_float64(which):
    rng = np.random.default_rng(21)
    M, N, K = 64, 48, 80
    x8 = _codes((M, K), O.E4M3, rng)
    w8 = _codes((N, K), O.E4M3, rng)
    g8 = _codes((M, N), O.E5M2, rng)
    sx, sw, sg = np.float32(20.0), np.float32(900.0), np.float32(3.0e4)

    def t(q, fmt):
        return torch.from_numpy(q).view(TF8[fmt]).to(torch.float64)

    if which == "fwd":
        ref = O.linear_fwd(x8, w8, O.E4M3, sx, sw)
        tr = (t(x8, O.E4M3) @ t(w8, O.E4M3).T) / (float(sx) * float(sw))
    elif which == "dx":
        ref = O.linear_bwd_dx(g8, O.E5M2, w8, O.E4M3, sg, sw)
        tr = (t(g8, O.E5M2) @ t(w8, O.E4M3)) / (float(sg) * float(sw))
    else:
        ref = O.linear_bwd_dw(g8, O.E5M2, x8, O.E4M3, sg, sx)
        tr = (t(g8, O.E5M2).T @ t(x8, O.E4M3)) / (float(sg) * float(sx))
    assert np.allclose(ref.r, tr.numpy(), rtol=1e-13, atol=0)
    assert np.array_equal(
        ref.y_bits, tr.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ) or np.abs(O.bf16_value(ref.y_bits) - tr.numpy()).max() <= O.bf16_ulp(tr.numpy()).max()


# ---------------------------------------------------------------- closed forms

def test_identity_weight():
    rng = np.random.default_rng(2)
    x8 = _codes((128, 256), O.E4M3, rng)
    w8 = np.where(np.eye(256, dtype=bool), 0x38, 0x00).astype(np.uint8)  # 1.0 on the diagonal
    sx, sw = np.float32(64.0), np.float32(2.0)
    beta = O.bf16_value(O.bf16_bits(rng.standard_normal(256) * 0.01))
    ref = O.linear_fwd(x8, w8, O.E4M3, sx, sw, beta)
    assert np.array_equal(ref.r, O.decode_array(x8, O.E4M3) / 128.0 + beta)


def test_fp8_bias_dequantized_after_operand_scaling():
    b8 = np.array([0x38, 0xB8, 0x7E, 0x01], np.uint8)  # 1, -1, 448, 2^-9
    vals = O.bias_values(b8, "e4m3", np.float32(8.0))
    assert list(vals) == [1 / 8, -1 / 8, 56.0, 2.0 ** -12]
    x8 = np.zeros((2, 4), np.uint8)
    w8 = np.zeros((4, 4), np.uint8)
    ref = O.linear_fwd(x8, w8, O.E4M3, 5.0, 7.0, vals)
    assert np.array_equal(ref.r, np.tile(vals, (2, 1)))


def test_fused_bias_within_one_ulp_of_split_path():
    rng = np.random.default_rng(9)
    x8 = _codes((96, 192), O.E4M3, rng)
    w8 = _codes((64, 192), O.E4M3, rng)
    beta = O.bf16_value(O.bf16_bits(rng.standard_normal(64) * 50.0))
    fused = O.linear_fwd(x8, w8, O.E4M3, 30.0, 500.0, beta)
    plain = O.linear_fwd(x8, w8, O.E4M3, 30.0, 500.0)
    split = O.bf16_value(O.bf16_bits(O.bf16_value(plain.y_bits) + beta))
    diff = np.abs(O.bf16_value(fused.y_bits) - split)
    # one ulp at the larger of the output and the pre-bias product (the
    # split path rounds once at the product's magnitude)
    assert np.all(diff <= np.maximum(O.bf16_ulp(fused.r), O.bf16_ulp(plain.r)))
    assert np.mean(diff == 0) > 0.5
    # and the fused result is at least as close to the exact value
    assert np.all(np.abs(O.bf16_value(fused.y_bits) - fused.r) <= np.abs(split - fused.r))


def test_bias_grad_closed_form_and_brute_force():
    M, N = 512, 24
    c = O.bf16_value(O.bf16_bits(np.full(N, 0.0078125)))
    g = np.tile(c, (M, 1))
    ref = O.bias_grad(g)
    assert np.array_equal(ref.r, M * c)
    rng = np.random.default_rng(4)
    g = O.bf16_value(O.bf16_bits(rng.standard_normal((37, 5)) * 1e-3))
    ref = O.bias_grad(g)
    for n in range(5):
        exact = sum(Fraction(float(v)) for v in g[:, n])
        assert ref.y_bits[n] == _bf16_of_fraction(exact)
    # pre-quantized gradient: dequantized before the sum
    g8 = _codes((37, 5), O.E5M2, rng)
    deq = O.dequantized(g8, O.E5M2, np.float32(4096.0))
    assert np.array_equal(deq, O.decode_array(g8, O.E5M2) / 4096.0)


# ---------------------------------------------------------------- bf16 spacing
# bfloat16 as a format (sign, 8 exponent bits with bias 127, 7 fraction
# bits; the fp32 exponent range): the value of every positive finite bit
# pattern written out from its fields with exact rationals, independent of
# the frexp/ldexp arithmetic of O.bf16_ulp.

def _bf16_field_value(p: int) -> Fraction:
    e, t = (p >> 7) & 0xFF, p & 0x7F
    if e == 0:
        return Fraction(t, 128) * Fraction(1, 2 ** 126)
    return (1 + Fraction(t, 128)) * Fraction(2) ** (e - 127)


_BF16_POS = None


def _bf16_table():
    """float64 values of the positive finite patterns 0x0000 .. 0x7F7F (each
    exact in float64), ascending."""
    global _BF16_POS
    if _BF16_POS is None:
        _BF16_POS = np.array([float(_bf16_field_value(p)) for p in range(0x7F80)], np.float64)
    return _BF16_POS


def _ulp_exact(r):
    """Spacing of bf16 at |r|: v(p+1) - v(p) for the pattern p with
    v(p) <= |r| < v(p+1); in the top binade (|r| >= v(0x7F7F)) the spacing
    of that binade."""
    tab = _bf16_table()
    a = np.abs(np.asarray(r, np.float64))
    p = np.searchsorted(tab, a, side="right") - 1
    p = np.clip(p, 0, len(tab) - 2)
    return tab[p + 1] - tab[p]


def test_bf16_ulp_matches_format_spacing():
    tab = _bf16_table()
    # every pattern's own value, the midpoint of its interval, the largest
    # float64 below the next pattern, and their negatives
    lo = tab[:-1]
    hi = tab[1:]
    pts = np.concatenate([lo, (lo + hi) / 2, np.nextafter(hi, 0.0), [tab[-1]]])
    pts = np.concatenate([pts, -pts])
    got = O.bf16_ulp(pts)
    want = _ulp_exact(pts)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(pts[i]), float(got[i]), float(want[i])) for i in bad[:6]]
    # closed values the format fixes: spacing 2^-7 on [1, 2), 2^-133 at and
    # near zero (the smallest subnormal), 2^120 in the top binade
    assert O.bf16_ulp(1.0) == 2.0 ** -7 and O.bf16_ulp(1.99) == 2.0 ** -7
    assert O.bf16_ulp(0.0) == 2.0 ** -133 and O.bf16_ulp(2.0 ** -140) == 2.0 ** -133
    assert O.bf16_ulp(2.0 ** -126) == 2.0 ** -133 and O.bf16_ulp(2.0 ** -125) == 2.0 ** -132
    assert O.bf16_ulp(3.0e38) == 2.0 ** 120


def test_tolerance_contract_exact():
    """gemm_tolerance = 2^-7 * sum_k |a_k b_k| / (sa sb) + ulp_bf16(r) (up to
    float64 rounding), with
    the sum of magnitudes written out term by term in exact rationals and the
    ulp from the format's bit fields; also for the tighter rel the GPU tests
    apply, and for dX / dW orientation (a transposed operand in the sum
    would fail)."""
    rng = np.random.default_rng(1)
    x8 = _codes((6, 16), O.E4M3, rng)
    w8 = _codes((4, 16), O.E4M3, rng)
    g8 = _codes((6, 4), O.E5M2, rng)
    sx, sw, sg = np.float32(2.0), np.float32(0.375), np.float32(1536.0)
    cases = [
        (O.linear_fwd(x8, w8, O.E4M3, sx, sw),
         lambda i, j: sum(abs(_frac(x8[i, k], O.E4M3) * _frac(w8[j, k], O.E4M3))
                          for k in range(16)), Fraction(1) / (Fraction(float(sx)) * Fraction(float(sw)))),
        (O.linear_bwd_dx(g8, O.E5M2, w8, O.E4M3, sg, sw),
         lambda i, j: sum(abs(_frac(g8[i, n], O.E5M2) * _frac(w8[n, j], O.E4M3))
                          for n in range(4)), Fraction(1) / (Fraction(float(sg)) * Fraction(float(sw)))),
        (O.linear_bwd_dw(g8, O.E5M2, x8, O.E4M3, sg, sx),
         lambda i, j: sum(abs(_frac(g8[m, i], O.E5M2) * _frac(x8[m, j], O.E4M3))
                          for m in range(6)), Fraction(1) / (Fraction(float(sg)) * Fraction(float(sx)))),
    ]
    for ref, abs_sum, dq in cases:
        for rel in (2.0 ** -7, 2.0 ** -10):
            tol = O.gemm_tolerance(ref, rel)
            ulp = _ulp_exact(ref.r)
            for i in range(ref.r.shape[0]):
                for j in range(ref.r.shape[1]):
                    want = Fraction(rel) * abs_sum(i, j) * dq + Fraction(float(ulp[i, j]))
                    # the oracle sums in float64: equal up to its rounding
                    err = abs(Fraction(float(tol[i, j])) - want)
                    assert err <= want * Fraction(1, 2 ** 40), (i, j, rel)


def test_quantized_gradient_direction_sanity():
    """The pages' regression signature of a wrong scale (the amax of already
    quantized values): the fp8 input gradient's direction collapsed to a
    cosine of about 0.05 with the bf16 one.  With the oracle's quantize and
    GEMM, the cosine of dX = G8 W8 / (sg sw) with the unquantized G W is
    close to 1, for the delayed scale of a first step and for a window that
    has seen 16x larger values; a scale that leaked the wrong ratio (G
    quantized with 2^-32 of its scale, most codes flushed to zero) is far
    from it."""
    rng = np.random.default_rng(5)
    M, N, K = 96, 64, 80
    W = O.bf16_value(O.bf16_bits(rng.standard_normal((N, K)) * 0.02))
    G = O.bf16_value(O.bf16_bits(rng.standard_normal((M, N)) * 1e-3))
    exact = G @ W
    cos = lambda a, b: float(np.sum(a * b) / np.sqrt(np.sum(a * a) * np.sum(b * b)))
    rw, rg = O.ScaleRing(16), O.ScaleRing(16)
    w8, sw, _ = O.quantize_step(W, O.E4M3, rw)
    g8, sg, _ = O.quantize_step(G, O.E5M2, rg)
    assert cos(O.linear_bwd_dx(g8, O.E5M2, w8, O.E4M3, sg, sw).r, exact) > 0.995
    O.quantize_step(G * 16.0, O.E5M2, rg)  # a larger step enters the window
    g8b, sgb, _ = O.quantize_step(G, O.E5M2, rg)
    assert sgb == sg / 16
    assert cos(O.linear_bwd_dx(g8b, O.E5M2, w8, O.E4M3, sgb, sw).r, exact) > 0.98
    bad_s = np.float32(sg * 2.0 ** -32)
    g8c = O.quantize_with_scale(G, bad_s, O.E5M2)
    assert cos(O.linear_bwd_dx(g8c, O.E5M2, w8, O.E4M3, bad_s, sw).r, exact) < 0.9


def test_fp8out_hand_worked_steps():
    """The FP8-output GEMM on a 2x2x2 case worked by hand: A = [[1, 2],
    [3, 1]], B = [[1, 0], [1, 1]] (e4m3 codes 0x38 = 1, 0x40 = 2, 0x44 = 3),
    sa = sb = 1, so A B^T = [[1, 3], [3, 4]].
      step 0, bias [0, 3]: y = [[1, 6], [3, 7]]; the fresh ring seeds
        s = 448 / 7 = 64; y s = 64, 384, 192, 448 -> 0x68, 0x7C, 0x74, 0x7E;
        hist [7, 0, 0], next scale 64.
      step 1, bias [0, 1]: y = [[1, 4], [3, 5]]; s = 64; y s = 64, 256,
        192, 320 -> 0x68, 0x78, 0x74, 0x7A; hist [7, 5, 0], scale 64.
      step 2, bias [0, 10]: y = [[1, 13], [3, 14]]; s = 64; 832 and 896
        saturate to 448 (0x7E); hist [7, 5, 14], next scale 448 / 14 = 32."""
    a8 = np.array([[0x38, 0x40], [0x44, 0x38]], dtype=np.uint8)
    b8 = np.array([[0x38, 0x00], [0x38, 0x38]], dtype=np.uint8)
    ring = O.ScaleRing(3)
    expect = [
        ([0.0, 3.0], [[0x68, 0x7C], [0x74, 0x7E]], 64.0, 7.0, [7, 0, 0], 64.0),
        ([0.0, 1.0], [[0x68, 0x78], [0x74, 0x7A]], 64.0, 5.0, [7, 5, 0], 64.0),
        ([0.0, 10.0], [[0x68, 0x7E], [0x74, 0x7E]], 64.0, 14.0, [7, 5, 14], 32.0),
    ]
    for bias, codes, s_used, a, hist, nxt in expect:
        q, s, am, _ = O.gemm_fp8out(a8, O.E4M3, b8, O.E4M3, 1.0, 1.0, np.array(bias),
                                     O.E4M3, ring)
        assert q.tolist() == codes
        assert float(s) == s_used and float(am) == a
        assert ring.hist.tolist() == hist and float(ring.scale) == nxt

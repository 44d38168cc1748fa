"""Plain CPU oracle for the FP8 linear-layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library; it is written to be read against the sources
below, not to be fast.

Sources (AstrAI commit-log pages; each cited by commit and page path):
  [P1] AstrAI commit 2eeac02d, page "tests/extension"
  [P2] AstrAI commit 2eeac02d, page "csrc"
  [P3] AstrAI commit 057c0d33, page "astrai/extension/ops"
  [P4] AstrAI commit 4019ddac, page "astrai"
  [P5] AstrAI commit 3e57cc80, page "astrai/extension/fp8.py"
  [OCP] OCP 8-bit Floating Point Specification (OFP8), rev 1.0 -- the bit
        layouts of E4M3 and E5M2; the pages name the formats and confirm only
        that the E4M3 maximum is about 448 ([P2], entry on the delayed-scale
        amax bug).

What the pages fix and what is a reading (every reading is listed with its
justification in the repository's design notes):
  * quantize: q = enc_fmt(fl32(x * s)), round-to-nearest-even, saturating
    to +-max; NaN -> 0x7F|sign; the sign of a value that rounds to zero is
    kept (reading: plainest RNE-saturate; the pages only name the formats).
  * amax is the max |x| over the *input* values, never over quantized values
    ([P3] entry on fp32-domain amax references; [P2]/[P5] entry on the amax
    bug that took the quantized max).
  * scale s = fmt_max / amax in IEEE fp32, kept at its previous value when
    amax is zero, non-finite or the quotient overflows (reading: margin 0).
  * delayed scaling ring: hist[H], idx, scale, seeded.  The first step seeds
    the scale from its own amax; every step quantizes with the scale it read,
    then folds its amax into hist[idx], advances idx and publishes
    scale = S(max(hist)) ([P1] entries on finalizing scale rings and on
    collapsing the tensor meta into three rings with seed/update; [P3] entry
    on snapshotting the scale before the finalize overwrites it).
  * GEMMs: Y = X8 W8^T / (sx sw) + bias, dX = G8 W8 / (sg sw),
    dW = G8^T X8 / (sg sx), accumulated here in fp64 and rounded once to
    bf16 ([P3] entries on bf16 output and on the forward's scale reaching the
    backward; [P1] entry on the fused bias and bias_scale; [P4] entry on the
    fused bias adding in fp32 before the single bf16 rounding).
  * db[n] = sum_m g[m, n] of the bf16 gradient, or of dec(g8)/sg when the
    gradient arrives pre-quantized ([P3] entry on bf16 grads and on a
    pre-quantized g dequantizing before the bias sum; [P4] entry on running
    the column sum only when the bias needs a gradient).

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, an independent library (torch CPU float8 casts and
float64 matmul), exact rational arithmetic on small cases, or hand-worked
sequences.  The amax of an input holding a NaN (the pages are silent; the
reading taken is that NaN propagates, as IEEE 754-2019 maximum does) is
pinned against torch's CPU amax.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------
# Formats  ([OCP]; [P3] entry validating the fmt enum)
# --------------------------------------------------------------------------

E4M3 = 0
E5M2 = 1
FORMATS = (E4M3, E5M2)

# exponent bits, mantissa bits, exponent bias of each format ([OCP] tables)
_LAYOUT = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}


def decode(code: int, fmt: int) -> float:
    """Exact value of one 8-bit code (Python float; NaN / +-inf where defined).

    E4M3 has no infinities and one NaN mantissa pattern (S.1111.111); E5M2
    follows IEEE-754 conventions (S.11111.00 = inf, S.11111.xx = NaN).
    """
    if fmt not in _LAYOUT:
        raise ValueError(f"unknown fp8 format {fmt}")
    e_bits, m_bits, bias = _LAYOUT[fmt]
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e_field = (code >> m_bits) & ((1 << e_bits) - 1)
    t_field = code & ((1 << m_bits) - 1)
    e_top = (1 << e_bits) - 1
    if fmt == E4M3 and e_field == e_top and t_field == (1 << m_bits) - 1:
        return math.copysign(math.nan, sign)
    if fmt == E5M2 and e_field == e_top:
        return sign * math.inf if t_field == 0 else math.copysign(math.nan, sign)
    if e_field == 0:  # subnormal: T * 2^(1 - bias - m_bits)
        return sign * t_field * 2.0 ** (1 - bias - m_bits)
    return sign * (1.0 + t_field / (1 << m_bits)) * 2.0 ** (e_field - bias)


def decode_table(fmt: int) -> np.ndarray:
    """float64[256]: value of every code."""
    return np.array([decode(c, fmt) for c in range(256)], dtype=np.float64)


def _positive_finite(fmt: int):
    """Sorted (values, codes) of the non-negative finite codes 0x00..max."""
    codes = [c for c in range(128) if math.isfinite(decode(c, fmt))]
    vals = np.array([decode(c, fmt) for c in codes], dtype=np.float64)
    assert np.all(np.diff(vals) > 0)
    return vals, np.array(codes, dtype=np.int64)


def fmt_max(fmt: int) -> float:
    """Largest finite magnitude of the format (448 for E4M3, 57344 for E5M2)."""
    return float(_positive_finite(fmt)[0][-1])


def encode(p, fmt: int) -> np.ndarray:
    """Encode fp32 values to codes: nearest finite code, ties to the even code,
    magnitudes at or beyond the maximum (and +-inf) saturate to +-max, NaN ->
    0x7F|sign, the sign of zero results is kept.

    Written as "nearest neighbour in the table of finite codes": |p| lies
    between two adjacent table values lo <= |p| < hi; their midpoint is exact
    in fp64, so the comparison with it is exact.
    """
    p = np.asarray(p, dtype=np.float32)
    vals, codes = _positive_finite(fmt)
    with np.errstate(invalid="ignore"):
        a = np.abs(p.astype(np.float64))
    neg = np.signbit(p).astype(np.int64)
    i = np.searchsorted(vals, a, side="right") - 1
    i = np.clip(i, 0, len(vals) - 2)
    lo, hi = vals[i], vals[i + 1]
    mid = (lo + hi) / 2.0
    even_hi = (codes[i + 1] & 1) == 0
    pick_hi = (a > mid) | ((a == mid) & even_hi)
    c = np.where(pick_hi, codes[i + 1], codes[i])
    c = np.where(a >= vals[-1], codes[-1], c)  # saturate (inf included)
    c = c | (neg << 7)
    c = np.where(np.isnan(p), 0x7F | (neg << 7), c)
    return c.astype(np.uint8)


def decode_array(q, fmt: int) -> np.ndarray:
    """float64 values of an array of codes."""
    return decode_table(fmt)[np.asarray(q, dtype=np.uint8).astype(np.int64)]


# --------------------------------------------------------------------------
# bf16 rounding (the single output rounding of the GEMMs and db)
# --------------------------------------------------------------------------

def bf16_bits(r) -> np.ndarray:
    """Round float64 values to bfloat16 (RNE, overflow -> inf); return bits.

    bf16 keeps 8 significant bits with the fp32 exponent range, so the
    spacing at |r| in [2^(e-1), 2^e) is 2^(e-8), never below the subnormal
    spacing 2^-133.  Scaling by that power of two is exact; rint is
    round-half-even.
    """
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    _, e = np.frexp(a)
    sp = np.maximum(e - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        v = np.ldexp(np.rint(np.ldexp(a, -sp)), sp)
        f = v.astype(np.float32)  # exact (or inf past the bf16 range)
    bits = (f.view(np.uint32) >> 16).astype(np.uint32)
    bits = bits | (np.signbit(r).astype(np.uint32) << 15)
    bits = np.where(np.isnan(r), 0x7FC0, bits)
    return bits.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """float64 value of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(r) -> np.ndarray:
    """Spacing of bf16 numbers at magnitude |r| (2^-133 at and near zero)."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    _, e = np.frexp(a)
    # frexp gives exponent 0 for zero; zero lies in the subnormal range,
    # whose spacing is the smallest subnormal 2^-133
    e = np.where(a == 0.0, -125, e)
    return np.ldexp(1.0, np.maximum(e - 8, -133))


# --------------------------------------------------------------------------
# Quantize, amax, scale  ([P3] two-primitive quantize; [P1] scale rings)
# --------------------------------------------------------------------------

def amax(x) -> np.float32:
    """max_i |x_i| over the input values in fp32 (0 for an empty tensor;
    NaN propagates)."""
    x = np.asarray(x, dtype=np.float32)
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def scale_from_amax(m, fmt: int, prev) -> np.float32:
    """S(m) = fmt_max / m in IEEE fp32; prev when m <= 0, m is not finite,
    or the quotient is not finite."""
    m = np.float32(m)
    if np.isfinite(m) and m > 0:
        with np.errstate(over="ignore"):
            r = np.float32(fmt_max(fmt)) / m
        if np.isfinite(r):
            return np.float32(r)
    return np.float32(prev)


def quantize_with_scale(x, s, fmt: int) -> np.ndarray:
    """q_i = enc(fl32(x_i * s)): one IEEE fp32 multiply, then the encoder."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        p = (x * np.float32(s)).astype(np.float32)
    return encode(p, fmt)


@dataclass
class ScaleRing:
    """Delayed-scaling state of one operand: hist[H], idx, scale, seeded."""

    hist_len: int
    hist: np.ndarray = field(init=False)
    idx: int = 0
    scale: np.float32 = np.float32(1.0)
    seeded: bool = False

    def __post_init__(self):
        if self.hist_len < 1:
            raise ValueError("hist_len must be >= 1")
        self.hist = np.zeros(self.hist_len, dtype=np.float32)

    def copy(self) -> "ScaleRing":
        r = ScaleRing(self.hist_len)
        r.hist = self.hist.copy()
        r.idx, r.scale, r.seeded = self.idx, np.float32(self.scale), self.seeded
        return r


def quantize_step(x, fmt: int, ring: ScaleRing | None = None):
    """One quantize of an operand.  Returns (q, s_used, a).

    ring is None: dynamic scaling, s_used = S(amax(x)) with prev = 1.
    Otherwise: seed on first use, quantize with the scale read *before*
    this step's fold, then fold amax into the window and publish the next
    scale (the window max includes never-written zero slots; amax >= 0).
    """
    x = np.asarray(x, dtype=np.float32)
    a = amax(x)
    if ring is None:
        s_used = scale_from_amax(a, fmt, np.float32(1.0))
        return quantize_with_scale(x, s_used, fmt), s_used, a
    if not ring.seeded:
        ring.scale = scale_from_amax(a, fmt, ring.scale)
        ring.seeded = True
    s_used = np.float32(ring.scale)
    q = quantize_with_scale(x, s_used, fmt)
    ring.hist[ring.idx] = a
    ring.idx = (ring.idx + 1) % ring.hist_len
    window = np.float32(np.max(ring.hist))
    ring.scale = scale_from_amax(window, fmt, ring.scale)
    return q, s_used, a


# --------------------------------------------------------------------------
# GEMMs ([P3] bf16 output, forward scale reused by backward; [P1] bias and
# bias_scale; [P4] bias added in fp32 before the single bf16 rounding)
# --------------------------------------------------------------------------

def _inv(s) -> float:
    return 1.0 / float(np.float32(s))


def bias_values(bias, bias_dtype: str, bias_scale=None) -> np.ndarray:
    """float64 bias: bf16 bits as values, or dec(b8) / bias_scale."""
    if bias_dtype == "bf16":
        return bf16_value(bias)
    fmt = {"e4m3": E4M3, "e5m2": E5M2}[bias_dtype]
    return decode_array(bias, fmt) / float(np.float32(bias_scale))


@dataclass
class GemmRef:
    r: np.ndarray       # unrounded float64 result
    y_bits: np.ndarray  # bf16 bits of RNE(r)
    abs_sum: np.ndarray  # sum |a*b| * dequant factor (tolerance base)


def _finish(acc, abs_acc, dq, add=None) -> GemmRef:
    r = acc * dq
    if add is not None:
        r = r + add
    return GemmRef(r=r, y_bits=bf16_bits(r), abs_sum=abs_acc * dq)


def linear_fwd(x8, w8, fmt: int, sx, sw, bias=None) -> GemmRef:
    """Y[m,n] = sum_k x8[m,k] w8[n,k] / (sx sw) + bias[n].

    bias: None or a float64 array of bias values (see bias_values)."""
    X = decode_array(x8, fmt)
    W = decode_array(w8, fmt)
    dq = _inv(sx) * _inv(sw)
    return _finish(X @ W.T, np.abs(X) @ np.abs(W).T, dq, bias)


def linear_bwd_dx(g8, fmt_g: int, w8, fmt_w: int, sg, sw) -> GemmRef:
    """dX[m,k] = sum_n g8[m,n] w8[n,k] / (sg sw)."""
    G = decode_array(g8, fmt_g)
    W = decode_array(w8, fmt_w)
    dq = _inv(sg) * _inv(sw)
    return _finish(G @ W, np.abs(G) @ np.abs(W), dq)


def linear_bwd_dw(g8, fmt_g: int, x8, fmt_x: int, sg, sx) -> GemmRef:
    """dW[n,k] = sum_m g8[m,n] x8[m,k] / (sg sx)."""
    G = decode_array(g8, fmt_g)
    X = decode_array(x8, fmt_x)
    dq = _inv(sg) * _inv(sx)
    return _finish(G.T @ X, np.abs(G).T @ np.abs(X), dq)


def bias_grad(g_values) -> GemmRef:
    """db[n] = sum_m g[m, n] (g given as float64 values: the bf16 gradient,
    or dec(g8)/sg for a pre-quantized one), rounded once to bf16."""
    g = np.asarray(g_values, dtype=np.float64)
    return GemmRef(r=g.sum(axis=0), y_bits=bf16_bits(g.sum(axis=0)),
                   abs_sum=np.abs(g).sum(axis=0))


def gemm_fp8out(a8, fmt_a: int, b8, fmt_b: int, sa, sb, bias, fmt_out: int,
                ring: ScaleRing):
    """FP8-in / FP8-out GEMM ([P1] entry on the custom op for an FP8-in /
    FP8-out GEMM; [P1] entry on the fp8 bias dequantized after the operand
    scaling and before any output quantization).

    y[m,n] = sum_k a8[m,k] b8[n,k] / (sa sb) + bias[n], as linear_fwd, and
    the output is one quantize step of fl32(y) with the output's ring.
    Reading: the pages name the op only; what is quantized is the fp32
    value the bf16-output GEMM would round, with the quantize's own scale
    and ring rules.  bias: None or float64 values (bias_values).  Returns
    (q, s_used, amax, ref)."""
    A = decode_array(a8, fmt_a)
    B = decode_array(b8, fmt_b)
    ref = _finish(A @ B.T, np.abs(A) @ np.abs(B).T, _inv(sa) * _inv(sb), bias)
    q, s_used, a = quantize_step(ref.r.astype(np.float32), fmt_out, ring)
    return q, s_used, a, ref


def dequantized(q, fmt: int, s) -> np.ndarray:
    """dec(q) / s in float64."""
    return decode_array(q, fmt) / float(np.float32(s))


# --------------------------------------------------------------------------
# Acceptance bound of a GEMM output against its reference
# --------------------------------------------------------------------------

def gemm_tolerance(ref: GemmRef, rel: float = 2.0 ** -7) -> np.ndarray:
    """|y - r| <= rel * sum|a b| * (dequant) + ulp_bf16(r).

    rel = 2^-7 is the acceptance contract; tests also apply a much tighter
    rel that fp32 accumulation meets, so a dropped or misplaced product
    cannot hide inside the contract's slack."""
    return rel * ref.abs_sum + bf16_ulp(ref.r)

"""GPU parity of the three FP8 GEMMs (through fp8_linear_fwd / bwd_dx /
bwd_dw with pre-quantized operands) against the oracle.

Two kinds of inputs: small-integer fp8 values, for which every partial sum
is exact and the bf16 output must equal the oracle bit for bit; and random
codes over the whole finite range, checked against the 2^-7 contract and
the 2^-10 diagnostic bound.
"""

import os

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from oracle import fp8_oracle as O
from tests.gpu_util import (DEV, bf16_bits, check_gemm, f32_scalar, scalar_dev, to_dev)

pytestmark = pytest.mark.gpu

TILES = ["auto", "256x256w8", "128x128w8", "256x256", "256x128", "128x128", "v1"]


@pytest.fixture(params=TILES)
def tile(request):
    """Force one GEMM tile configuration (the library reads FP8L_TILE at each
    launch); shapes the fast kernels cannot take fall back to v1 anyway."""
    old = os.environ.get("FP8L_TILE")
    if request.param == "auto":
        os.environ.pop("FP8L_TILE", None)
    else:
        os.environ["FP8L_TILE"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("FP8L_TILE", None)
    else:
        os.environ["FP8L_TILE"] = old

INT_CODES = {  # value -> code for 0, +-1, +-2
    O.E4M3: {0: 0x00, 1: 0x38, 2: 0x40, -1: 0xB8, -2: 0xC0},
    O.E5M2: {0: 0x00, 1: 0x3C, 2: 0x40, -1: 0xBC, -2: 0xC0},
}


def _int_codes(shape, fmt, rng):
    vals = rng.integers(-2, 3, size=shape)
    lut = INT_CODES[fmt]
    return np.vectorize(lambda v: lut[int(v)], otypes=[np.uint8])(vals)


def _rand_codes(shape, fmt, rng):
    tab = O.decode_table(fmt)
    fin = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    return rng.choice(fin, size=shape)


def _q(codes, fmt, s):
    return F.Quantized(to_dev(codes), fmt, scalar_dev(s))


def run_fwd(x8, w8, fmt, sx, sw, bias=None):
    M, K = x8.shape
    N = w8.shape[0]
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    F.fp8_linear_fwd(_q(x8, fmt, sx), _q(w8, fmt, sw), bias, fmt, y)
    torch.cuda.synchronize()
    return bf16_bits(y)


def run_dx(g8, fg, w8, fw, sg, sw):
    M, N = g8.shape
    K = w8.shape[1]
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    F.fp8_linear_bwd_dx(_q(g8, fg, sg), fg, _q(w8, fw, sw), dx)
    torch.cuda.synchronize()
    return bf16_bits(dx)


def run_dw(g8, fg, x8, fx, sg, sx, with_db=False):
    M, N = g8.shape
    K = x8.shape[1]
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    db = ws = None
    if with_db:
        db = torch.empty(N, dtype=torch.bfloat16, device=DEV)
        ws = torch.empty(max(1, F.fp8_db_workspace_bytes(M, N) // 4), dtype=torch.float32, device=DEV)
    F.fp8_linear_bwd_dw(_q(g8, fg, sg), fg, _q(x8, fx, sx), dw, db, ws)
    torch.cuda.synchronize()
    return bf16_bits(dw), (None if db is None else bf16_bits(db))


SHAPES = [(128, 128, 128), (256, 384, 512), (200, 136, 300), (1, 1, 1), (33, 17, 129),
          (130, 260, 1000), (272, 528, 400), (512, 256, 2064), (48, 80, 16)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_exact_small_integers_all_three(M, N, K, tile):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    x8 = _int_codes((M, K), O.E4M3, rng)
    w8 = _int_codes((N, K), O.E4M3, rng)
    g8 = _int_codes((M, N), O.E5M2, rng)
    y = run_fwd(x8, w8, O.E4M3, 1.0, 1.0)
    assert np.array_equal(y, O.linear_fwd(x8, w8, O.E4M3, 1.0, 1.0).y_bits)
    dx = run_dx(g8, O.E5M2, w8, O.E4M3, 1.0, 1.0)
    assert np.array_equal(dx, O.linear_bwd_dx(g8, O.E5M2, w8, O.E4M3, 1.0, 1.0).y_bits)
    dw, _ = run_dw(g8, O.E5M2, x8, O.E4M3, 1.0, 1.0)
    assert np.array_equal(dw, O.linear_bwd_dw(g8, O.E5M2, x8, O.E4M3, 1.0, 1.0).y_bits)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fa,fb", [(O.E4M3, O.E4M3), (O.E5M2, O.E4M3), (O.E5M2, O.E5M2),
                                   (O.E4M3, O.E5M2)])
def test_random_codes_tolerance(M, N, K, fa, fb, tile):
    rng = np.random.default_rng(M + N + K + 10 * fa + fb)
    sa, sb = np.float32(37.5), np.float32(0.0625)
    x8 = _rand_codes((M, K), fb, rng)
    w8 = _rand_codes((N, K), fb, rng)
    g8 = _rand_codes((M, N), fa, rng)
    check_gemm(run_fwd(x8, w8, fb, sb, sa), O.linear_fwd(x8, w8, fb, sb, sa), "fwd")
    check_gemm(run_dx(g8, fa, w8, fb, sa, sb), O.linear_bwd_dx(g8, fa, w8, fb, sa, sb), "dx")
    dw, _ = run_dw(g8, fa, x8, fb, sa, sb)
    check_gemm(dw, O.linear_bwd_dw(g8, fa, x8, fb, sa, sb), "dw")


@pytest.mark.parametrize("bias_kind", ["bf16", "e4m3", "e5m2"])
# 256 and 264: codes staged in LDS by the kernels (N times the code size a
# multiple of 16; 264 ends in a partial tile), 77: read from memory
@pytest.mark.parametrize("N", [256, 264, 77])
def test_fused_bias(bias_kind, N, tile):
    rng = np.random.default_rng(N)
    M, K = 160, 384
    x8 = _rand_codes((M, K), O.E4M3, rng)
    w8 = _rand_codes((N, K), O.E4M3, rng)
    if bias_kind == "bf16":
        bits = O.bf16_bits(rng.standard_normal(N) * 3.0)
        bias = to_dev(bits.view(np.int16)).view(torch.bfloat16)
        beta = O.bias_values(bits, "bf16")
    else:
        fmt = O.E4M3 if bias_kind == "e4m3" else O.E5M2
        b8 = _rand_codes((N,), fmt, rng)
        bs = np.float32(24.0)
        bias = F.Quantized(to_dev(b8), fmt, scalar_dev(bs))
        beta = O.bias_values(b8, bias_kind, bs)
    y = run_fwd(x8, w8, O.E4M3, 3.0, 5.0, bias)
    check_gemm(y, O.linear_fwd(x8, w8, O.E4M3, 3.0, 5.0, beta), "fwd+bias")
    # small-integer operands with a bf16-exact bias: bit-exact
    xi = _int_codes((M, K), O.E4M3, rng)
    wi = _int_codes((N, K), O.E4M3, rng)
    if bias_kind == "bf16":
        y = run_fwd(xi, wi, O.E4M3, 1.0, 1.0, bias)
        assert np.array_equal(y, O.linear_fwd(xi, wi, O.E4M3, 1.0, 1.0, beta).y_bits)


def test_identity_weight_special_case():
    rng = np.random.default_rng(2)
    x8 = _rand_codes((128, 256), O.E4M3, rng)
    w8 = np.where(np.eye(256, dtype=bool), 0x38, 0x00).astype(np.uint8)
    y = run_fwd(x8, w8, O.E4M3, 64.0, 2.0)
    ref = O.linear_fwd(x8, w8, O.E4M3, 64.0, 2.0)
    assert np.array_equal(y, ref.y_bits)
    # closed form dec(x)/(sx sw); a dot product of -0 with +0 terms is +0
    assert np.array_equal(y, O.bf16_bits(O.decode_array(x8, O.E4M3) / 128.0 + 0.0))


@pytest.mark.parametrize("M,N,K", [(64, 48, 0), (0, 48, 64), (48, 0, 64)])
def test_degenerate_sizes(M, N, K, tile):
    rng = np.random.default_rng(0)
    x8 = _rand_codes((M, K), O.E4M3, rng)
    w8 = _rand_codes((N, K), O.E4M3, rng)
    g8 = _rand_codes((M, N), O.E5M2, rng)
    assert np.array_equal(run_fwd(x8, w8, O.E4M3, 2.0, 2.0),
                          O.linear_fwd(x8, w8, O.E4M3, 2.0, 2.0).y_bits)
    assert np.array_equal(run_dx(g8, O.E5M2, w8, O.E4M3, 2.0, 2.0),
                          O.linear_bwd_dx(g8, O.E5M2, w8, O.E4M3, 2.0, 2.0).y_bits)
    dw, db = run_dw(g8, O.E5M2, x8, O.E4M3, 2.0, 2.0, with_db=True)
    assert np.array_equal(dw, O.linear_bwd_dw(g8, O.E5M2, x8, O.E4M3, 2.0, 2.0).y_bits)
    ref_db = O.bias_grad(O.dequantized(g8, O.E5M2, 2.0))
    assert np.array_equal(db, ref_db.y_bits)


@pytest.mark.parametrize("M,N", [(2048, 1536), (100, 40), (37, 300)])
def test_db_from_prequantized_gradient(M, N, tile):
    rng = np.random.default_rng(M)
    g8 = _rand_codes((M, N), O.E5M2, rng)
    x8 = _rand_codes((M, 64), O.E4M3, rng)
    sg = np.float32(2048.0)
    _, db = run_dw(g8, O.E5M2, x8, O.E4M3, sg, 1.0, with_db=True)
    check_gemm(db, O.bias_grad(O.dequantized(g8, O.E5M2, sg)), "db")


@pytest.mark.parametrize("M,N,K", [(2048, 1536, 1024), (520, 776, 1090)])
def test_repeat_runs_bit_identical(M, N, K, tile):
    """Every GEMM sums in a fixed order (the K halves of the 128x128 kernel
    meet in a fixed pairing, the bias gradient in a fixed xor tree), so two
    runs on the same operands give the same bytes."""
    rng = np.random.default_rng(M + N)
    x8 = _rand_codes((M, K), O.E4M3, rng)
    w8 = _rand_codes((N, K), O.E4M3, rng)
    g8 = _rand_codes((M, N), O.E5M2, rng)
    first = (run_fwd(x8, w8, O.E4M3, 4.0, 8.0), run_dx(g8, O.E5M2, w8, O.E4M3, 2.0, 8.0),
             *run_dw(g8, O.E5M2, x8, O.E4M3, 2.0, 4.0, with_db=True))
    second = (run_fwd(x8, w8, O.E4M3, 4.0, 8.0), run_dx(g8, O.E5M2, w8, O.E4M3, 2.0, 8.0),
              *run_dw(g8, O.E5M2, x8, O.E4M3, 2.0, 4.0, with_db=True))
    for name, a, b in zip(("y", "dx", "dw", "db"), first, second):
        assert np.array_equal(a, b), name


def test_full_size_sampled_rows(tile):
    """dim1536/ffn6912 shapes at M = 2048, random codes over the whole finite
    range.  Under the automatic tile choice (the configuration the step and
    the benchmark run) every output element is compared with the oracle;
    under each forced tile configuration a seeded sample of rows plus the
    first and last."""
    rng = np.random.default_rng(99)
    full = tile == "auto"
    for (K, N) in ((1536, 4608), (1536, 1536), (1536, 6912), (6912, 1536)):
        M = 2048
        x8 = _rand_codes((M, K), O.E4M3, rng)
        w8 = _rand_codes((N, K), O.E4M3, rng)
        g8 = _rand_codes((M, N), O.E5M2, rng)
        rows = np.arange(M) if full else \
            np.unique(np.concatenate([[0, M - 1], rng.choice(M, 48, replace=False)]))
        y = run_fwd(x8, w8, O.E4M3, 100.0, 3000.0)
        check_gemm(y[rows], O.linear_fwd(x8[rows], w8, O.E4M3, 100.0, 3000.0), f"fwd {K}x{N}")
        dx = run_dx(g8, O.E5M2, w8, O.E4M3, 7.0e3, 3000.0)
        check_gemm(dx[rows], O.linear_bwd_dx(g8[rows], O.E5M2, w8, O.E4M3, 7.0e3, 3000.0),
                   f"dx {K}x{N}")
        dw, _ = run_dw(g8, O.E5M2, x8, O.E4M3, 7.0e3, 100.0)
        nrows = np.arange(N) if full else \
            np.unique(np.concatenate([[0, N - 1], rng.choice(N, 48, replace=False)]))
        check_gemm(dw[nrows], O.linear_bwd_dw(g8[:, nrows], O.E5M2, x8, O.E4M3, 7.0e3, 100.0),
                   f"dw {K}x{N}")


# ---------------------------------------------------------------- fp8_gemm
# The general entry point: batch slices by stride, size-1 batches broadcast,
# and transposed views passed as a layout (no copy).  Each slice is compared
# with the oracle on the same codes arranged as [M, K] and [N, K].

def _stored(codes_rk, layout):
    """Device tensor holding [.., R, K] codes in the given layout: k-contiguous
    rows, or a [.., K, R] buffer seen through .mT."""
    if layout == F.FP8_K_CONTIG:
        return to_dev(np.ascontiguousarray(codes_rk))
    buf = to_dev(np.ascontiguousarray(np.swapaxes(codes_rk, -1, -2)))
    return buf.mT


@pytest.mark.parametrize("la", [F.FP8_K_CONTIG, F.FP8_K_STRIDED])
@pytest.mark.parametrize("lb", [F.FP8_K_CONTIG, F.FP8_K_STRIDED])
@pytest.mark.parametrize("shape", [(3, 256, 384, 512), (2, 200, 136, 300), (3, 208, 96, 64)])
def test_gemm_batched_layouts(tile, la, lb, shape):
    B, M, N, K = shape
    rng = np.random.default_rng(B * M + N + 7 * K + 2 * la + lb)
    a = _rand_codes((B, M, K), O.E4M3, rng)
    b = _rand_codes((B, N, K), O.E4M3, rng)
    bias = (rng.standard_normal(N) * 0.5).astype(np.float32)
    bias_t = torch.from_numpy(bias).to(torch.bfloat16)
    sa, sb = np.float32(3.0), np.float32(0.125)
    c = torch.empty(B, M, N, dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm(F.Quantized(_stored(a, la), O.E4M3, scalar_dev(sa)),
               F.Quantized(_stored(b, lb), O.E4M3, scalar_dev(sb)), c, bias=bias_t.to(DEV))
    torch.cuda.synchronize()
    beta = O.bias_values(bias_t.view(torch.int16).numpy().view(np.uint16), "bf16")
    got = bf16_bits(c)
    for z in range(B):
        check_gemm(got[z], O.linear_fwd(a[z], b[z], O.E4M3, sa, sb, beta), f"slice {z}")


@pytest.mark.parametrize("lb", [F.FP8_K_CONTIG, F.FP8_K_STRIDED])
def test_gemm_broadcast_and_mixed_formats_exact(tile, lb):
    """b given once (2-D) for 4 slices of a; e5m2 x e4m3 small integers, so
    every slice must equal the oracle bit for bit."""
    B, M, N, K = 4, 160, 272, 384
    rng = np.random.default_rng(11 + lb)
    a = _int_codes((B, M, K), O.E5M2, rng)
    b = _int_codes((N, K), O.E4M3, rng)
    c = torch.empty(B, M, N, dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm(F.Quantized(_stored(a, F.FP8_K_CONTIG), O.E5M2, scalar_dev(1.0)),
               F.Quantized(_stored(b, lb), O.E4M3, scalar_dev(2.0)), c)
    torch.cuda.synchronize()
    got = bf16_bits(c)
    for z in range(B):
        ref = O.linear_bwd_dx(a[z], O.E5M2, np.ascontiguousarray(b.T), O.E4M3, 1.0, 2.0)
        assert np.array_equal(got[z], ref.y_bits), f"slice {z}"


def test_gemm_batch_one_of_a_broadcasts(tile):
    """a with batch 1 against b with batch 3: a's slice is shared."""
    M, N, K = 128, 256, 192
    rng = np.random.default_rng(5)
    a = _rand_codes((1, M, K), O.E4M3, rng)
    b = _rand_codes((3, N, K), O.E4M3, rng)
    c = torch.empty(3, M, N, dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm(F.Quantized(to_dev(a), O.E4M3, scalar_dev(1.0)),
               F.Quantized(to_dev(b), O.E4M3, scalar_dev(1.0)), c)
    torch.cuda.synchronize()
    got = bf16_bits(c)
    for z in range(3):
        check_gemm(got[z], O.linear_fwd(a[0], b[z], O.E4M3, 1.0, 1.0), f"slice {z}")

"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/fp8linear.h declares, and rejects bad arguments with
the documented status before touching the device."""

import ctypes
import os
import re

import pytest

import scaled_quantize_fp8_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


HEADERS = {"fp8linear.h": "libfp8linear.so", "fp8probe.h": "libfp8probe.so"}


def _declared_functions(header="fp8linear.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(fp8[a-z_0-9]*_[a-z_0-9]+)\s*\(",
                      text, re.M)


def test_every_header_has_its_library():
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == \
        sorted(HEADERS)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.LIB_PATH):
        pytest.fail("libfp8linear.so is not built: run __graft_entry__.build()")
    return F.lib()


def test_header_declares_every_entry_point():
    names = set(_declared_functions())
    for must in ("fp8_quantize", "fp8_quantize_pair", "fp8_linear_fwd", "fp8_linear_bwd_dx",
                 "fp8_linear_bwd_dw"):
        assert must in names
    assert names == set(F.C_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_probe_library_exports_its_symbols():
    from scaled_quantize_fp8_amd import probe
    names = set(_declared_functions("fp8probe.h"))
    assert names == set(probe.C_SYMBOLS)
    L = probe.lib()
    for name in names:
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value
    # argument checks return before any launch
    assert L.fp8probe_mfma(0, 1, 1, 1, None) == 2
    assert L.fp8probe_mfma(4, 1, None, 1, None) == 1
    assert L.fp8probe_stream(1, 1, 17, 0, 1, 1, None) == 2
    assert L.fp8probe_stream(1, 1, 16, 3, 1, 1, None) == 2
    assert L.fp8probe_stream(None, 1, 16, 0, 1, 1, None) == 1


def test_version_and_status_strings(lib):
    assert F.fp8_abi_version() == 5
    for st in range(6):
        assert F.status_str(st)
    assert F.status_str(99) == "unknown status"


def test_library_built_from_tree_sources(lib):
    """The library carries the hash of the sources it was built from; the
    GPU tests refuse a library whose hash differs from the tree's."""
    from scaled_quantize_fp8_amd import _build
    h = F.fp8_source_hash()
    assert len(h) == 64 and h == _build.source_hash()


def test_sizes(lib):
    assert F.fp8_ring_bytes(16) == 8320 + 64
    assert F.fp8_ring_bytes(1024) == 8320 + 4096
    assert F.fp8_ring_bytes(0) == 0 and F.fp8_ring_bytes(1025) == 0
    assert F.fp8_db_workspace_bytes(2048, 6912) == 4 * 64 * 6912
    assert F.fp8_db_workspace_bytes(33, 10) == 4 * 2 * 10
    assert F.fp8_db_workspace_bytes(0, 10) == 0


P = ctypes.c_void_p(0x100000)  # a non-null "device" address never dereferenced


def test_quantize_validation(lib):
    q = lib.fp8_quantize
    ring = F._Ring(None, 16, 0)
    # NULL scale_used
    assert q(P, F.FP8_DT_BF16, 16, F.FP8_E4M3, P, None, None, P, None) == F.FP8_ERR_NULL
    # dynamic without amax_out
    assert q(P, F.FP8_DT_BF16, 16, F.FP8_E4M3, P, None, P, None, None) == F.FP8_ERR_NULL
    # bad format, bad dtype, negative size
    assert q(P, F.FP8_DT_BF16, 16, 7, P, None, P, P, None) == F.FP8_ERR_DTYPE
    assert q(P, F.FP8_DT_E4M3, 16, F.FP8_E4M3, P, None, P, P, None) == F.FP8_ERR_DTYPE
    assert q(P, F.FP8_DT_BF16, -1, F.FP8_E4M3, P, None, P, P, None) == F.FP8_ERR_SHAPE
    # ring with NULL dev, bad hist_len, misaligned dev
    assert q(P, F.FP8_DT_BF16, 16, F.FP8_E4M3, P, ctypes.byref(ring), P, None, None) == F.FP8_ERR_NULL
    ring = F._Ring(ctypes.c_void_p(0x100000), 0, 0)
    assert q(P, F.FP8_DT_BF16, 16, F.FP8_E4M3, P, ctypes.byref(ring), P, None, None) == F.FP8_ERR_RING
    ring = F._Ring(ctypes.c_void_p(0x100010), 16, 0)
    assert q(P, F.FP8_DT_BF16, 16, F.FP8_E4M3, P, ctypes.byref(ring), P, None, None) == F.FP8_ERR_RING
    # scale_used aliasing the ring's scale slot
    ring = F._Ring(ctypes.c_void_p(0x100000), 16, 1)
    assert q(P, F.FP8_DT_BF16, 16, F.FP8_E4M3, P, ctypes.byref(ring), P, None, None) == F.FP8_ERR_RING
    assert ring.seeded == 1


def test_quantize_pair_validation(lib):
    qp = lib.fp8_quantize_pair
    P2 = ctypes.c_void_p(0x200000)
    bf, e4 = F.FP8_DT_BF16, F.FP8_E4M3
    ring = F._Ring(ctypes.c_void_p(0x100000), 16, 1)
    r = ctypes.byref(ring)
    # one ring for both tensors
    assert qp(P, bf, 16, P, r, P2, None, P, bf, 16, P, r, P2, None, e4, None) == F.FP8_ERR_RING
    # second tensor: fp8 input type, NULL scale_used, dynamic without amax_out
    assert qp(P, bf, 16, P, None, P2, P, P, F.FP8_DT_E5M2, 16, P, None, P2, P, e4,
              None) == F.FP8_ERR_DTYPE
    assert qp(P, bf, 16, P, None, P2, P, P, bf, 16, P, None, None, P, e4, None) == F.FP8_ERR_NULL
    assert qp(P, bf, 16, P, None, P2, P, P, bf, 16, P, None, P2, None, e4, None) == F.FP8_ERR_NULL
    # bad format, negative size
    assert qp(P, bf, 16, P, None, P2, P, P, bf, 16, P, None, P2, P, 5, None) == F.FP8_ERR_DTYPE
    assert qp(P, bf, -3, P, None, P2, P, P, bf, 16, P, None, P2, P, e4, None) == F.FP8_ERR_SHAPE


def test_linear_validation(lib):
    hp = F._Operand(P, F.FP8_DT_BF16, None)
    f8 = F._Operand(P, F.FP8_DT_E4M3, P)
    f8_noscale = F._Operand(P, F.FP8_DT_E4M3, None)
    f8_wrong = F._Operand(P, F.FP8_DT_E5M2, P)
    none = F._Operand(None, F.FP8_DT_BF16, None)
    fwd = lib.fp8_linear_fwd
    args = lambda x, w, b=none, fmt=F.FP8_E4M3, y=P: (8, 8, 8, x, w, b, fmt, None, None, y, P, P, P, P,
                                                       P, P, None)
    assert fwd(*args(hp, f8_noscale)) == F.FP8_ERR_NULL
    assert fwd(*args(hp, f8_wrong)) == F.FP8_ERR_DTYPE
    assert fwd(*args(hp, f8, fmt=3)) == F.FP8_ERR_DTYPE
    assert fwd(*args(hp, f8, b=F._Operand(P, F.FP8_DT_F32, None))) == F.FP8_ERR_DTYPE
    assert fwd(*args(hp, f8, b=F._Operand(P, F.FP8_DT_E4M3, None))) == F.FP8_ERR_NULL
    assert fwd(*args(hp, f8, y=None)) == F.FP8_ERR_NULL
    assert fwd(-1, 8, 8, hp, f8, none, 0, None, None, P, P, P, P, P, P, P, None) == F.FP8_ERR_SHAPE
    assert fwd(2**40, 2**40, 8, hp, f8, none, 0, None, None, P, P, P, P, P, P, P, None) == F.FP8_ERR_SHAPE
    # x8_out missing for a high-precision x
    assert fwd(8, 8, 8, hp, f8, none, 0, None, None, P, None, P, P, P, P, P, None) == F.FP8_ERR_NULL
    dx = lib.fp8_linear_bwd_dx
    assert dx(8, 8, 8, hp, F.FP8_E5M2, None, hp, P, P, P, P, None) == F.FP8_ERR_DTYPE
    assert dx(8, 8, 8, hp, F.FP8_E5M2, None, f8, None, P, P, P, None) == F.FP8_ERR_NULL
    assert dx(8, 8, 8, f8, F.FP8_E5M2, None, f8, P, P, P, P, None) == F.FP8_ERR_DTYPE
    dw = lib.fp8_linear_bwd_dw
    assert dw(8, 8, 8, hp, F.FP8_E5M2, None, f8, P, P, None, P, P, P, None) == F.FP8_ERR_NULL
    assert dw(8, 8, 8, hp, 9, None, f8, P, None, None, P, P, P, None) == F.FP8_ERR_DTYPE


def test_two_stream_backward_validation(lib):
    """fp8_linear_bwd checks the union of the dX and dW arguments before it
    enqueues anything (or records its fork event)."""
    hp = F._Operand(P, F.FP8_DT_BF16, None)
    f8 = F._Operand(P, F.FP8_DT_E4M3, P)
    g8 = F._Operand(P, F.FP8_DT_E5M2, P)
    S2 = ctypes.c_void_p(0x300000)
    bwd = lib.fp8_linear_bwd

    def call(M=8, N=8, K=8, g=hp, fmt=F.FP8_E5M2, x8=f8, w8=f8, dx=P, dw=P, db=None, ws=None,
             g8_out=P, su=P, am=P):
        return bwd(M, N, K, g, fmt, None, x8, w8, dx, dw, db, ws, g8_out, su, am, None, S2)

    assert call(M=-1) == F.FP8_ERR_SHAPE
    assert call(M=2**40, N=2**40) == F.FP8_ERR_SHAPE
    assert call(fmt=7) == F.FP8_ERR_DTYPE
    assert call(g=F._Operand(P, F.FP8_DT_E4M3, P)) == F.FP8_ERR_DTYPE  # fp8 g of the other format
    assert call(g=F._Operand(P, F.FP8_DT_E5M2, None)) == F.FP8_ERR_NULL  # pre-quantized, no scale
    assert call(g8_out=None) == F.FP8_ERR_NULL                         # hp g needs g8_out
    assert call(su=None) == F.FP8_ERR_NULL
    assert call(am=None) == F.FP8_ERR_NULL                             # dynamic: amax required
    assert call(w8=hp) == F.FP8_ERR_DTYPE                              # dX operand
    assert call(w8=F._Operand(P, F.FP8_DT_E4M3, None)) == F.FP8_ERR_NULL
    assert call(dx=None) == F.FP8_ERR_NULL
    assert call(x8=hp) == F.FP8_ERR_DTYPE                              # dW operand
    assert call(x8=F._Operand(None, F.FP8_DT_E4M3, P)) == F.FP8_ERR_NULL
    assert call(dw=None) == F.FP8_ERR_NULL
    assert call(db=P, ws=None) == F.FP8_ERR_NULL                       # db needs its workspace
    assert call(g=g8, g8_out=None, su=None, am=None, dx=None) == F.FP8_ERR_NULL


def test_ring_init_validation(lib):
    r = F._Ring()
    assert lib.fp8_ring_init(None, P, 16, None) == F.FP8_ERR_NULL
    assert lib.fp8_ring_init(ctypes.byref(r), None, 16, None) == F.FP8_ERR_NULL
    assert lib.fp8_ring_init(ctypes.byref(r), P, 0, None) == F.FP8_ERR_RING
    assert lib.fp8_ring_init(ctypes.byref(r), ctypes.c_void_p(0x100040), 16, None) == F.FP8_ERR_RING


def test_gemm_validation(lib):
    gm = lib.fp8_gemm
    f8 = F._Operand(P, F.FP8_DT_E4M3, P)
    f8b = F._Operand(P, F.FP8_DT_E5M2, P)
    none = F._Operand(None, F.FP8_DT_BF16, None)
    KC, KS = F.FP8_K_CONTIG, F.FP8_K_STRIDED

    def call(batch=2, M=8, N=16, K=32, a=f8, la=KC, lda=32, sa=256, b=f8b, lb=KC, ldb=32, sb=512,
             bias=none, c=P, ldc=16, sc=128):
        return gm(batch, M, N, K, a, la, lda, sa, b, lb, ldb, sb, bias, c, ldc, sc, None)

    assert call(a=F._Operand(P, F.FP8_DT_BF16, None)) == F.FP8_ERR_DTYPE  # not fp8
    assert call(la=2) == F.FP8_ERR_DTYPE
    assert call(a=F._Operand(P, F.FP8_DT_E4M3, None)) == F.FP8_ERR_NULL  # no scale
    assert call(bias=F._Operand(P, F.FP8_DT_F16, None)) == F.FP8_ERR_DTYPE
    assert call(bias=F._Operand(P, F.FP8_DT_E5M2, None)) == F.FP8_ERR_NULL
    assert call(lda=31) == F.FP8_ERR_SHAPE                 # k-contiguous A needs lda >= K
    assert call(la=KS, lda=7) == F.FP8_ERR_SHAPE           # strided A needs lda >= M
    assert call(lb=KS, ldb=15) == F.FP8_ERR_SHAPE          # strided B needs ldb >= N
    assert call(ldc=15) == F.FP8_ERR_SHAPE
    assert call(sc=16 * 7 + 15) == F.FP8_ERR_SHAPE         # output slices would overlap
    assert call(batch=-1) == F.FP8_ERR_SHAPE and call(sa=-1) == F.FP8_ERR_SHAPE
    assert call(batch=65536) == F.FP8_ERR_SHAPE
    assert call(c=None) == F.FP8_ERR_NULL
    # empty problems enqueue nothing and succeed
    assert call(batch=0) == F.FP8_OK and call(M=0) == F.FP8_OK



def test_quantize_2d_validation(lib):
    q2 = lib.fp8_quantize_2d
    bf, e4 = F.FP8_DT_BF16, F.FP8_E4M3
    P2 = ctypes.c_void_p(0x200000)
    assert q2(P, bf, 8, 8, e4, 3, P, P, None, P2, P, None) == F.FP8_ERR_DTYPE   # layout
    assert q2(P, bf, 8, 8, e4, F.FP8_QUANT_ROWS, None, P, None, P2, P, None) == F.FP8_ERR_NULL
    assert q2(P, bf, 8, 8, e4, F.FP8_QUANT_TRANSPOSED, P, None, None, P2, P, None) == F.FP8_ERR_NULL
    assert q2(P, bf, 8, 8, e4, F.FP8_QUANT_DUAL, P, None, None, P2, P, None) == F.FP8_ERR_NULL
    assert q2(P, bf, -1, 8, e4, F.FP8_QUANT_DUAL, P, P, None, P2, P, None) == F.FP8_ERR_SHAPE
    assert q2(P, F.FP8_DT_E5M2, 8, 8, e4, F.FP8_QUANT_DUAL, P, P, None, P2, P, None) == F.FP8_ERR_DTYPE
    assert q2(P, bf, 8, 8, e4, F.FP8_QUANT_DUAL, P, P, None, None, P, None) == F.FP8_ERR_NULL

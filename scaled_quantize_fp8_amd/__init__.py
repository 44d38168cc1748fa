"""Python binding of libfp8linear.so: argument marshalling only.

Every function here has the name of the C entry point it calls and maps
torch tensors (device memory) to the pointers and sizes of the C ABI
declared in include/fp8linear.h.  No step of the computation runs in
Python; without the built library every call raises.

Conventions: fmt / dtype values are the C enums below; pre-quantized
operands are passed as ``Quantized(codes_uint8, fmt, scale_f32)``; rings are
``ScaleRing`` objects that own their device buffer and the C struct.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from ._build import LIB_PATH

FP8_E4M3, FP8_E5M2 = 0, 1
FP8_DT_F32, FP8_DT_F16, FP8_DT_BF16, FP8_DT_E4M3, FP8_DT_E5M2 = 0, 1, 2, 3, 4
FP8_OK, FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_DTYPE, FP8_ERR_RING, FP8_ERR_HIP = range(6)
FP8_K_CONTIG, FP8_K_STRIDED = 0, 1
FP8_QUANT_ROWS, FP8_QUANT_TRANSPOSED, FP8_QUANT_DUAL = 0, 1, 2

_TORCH_DT = {torch.float32: FP8_DT_F32, torch.float16: FP8_DT_F16, torch.bfloat16: FP8_DT_BF16}
_FMT_DT = {FP8_E4M3: FP8_DT_E4M3, FP8_E5M2: FP8_DT_E5M2}

C_SYMBOLS = (
    "fp8_abi_version", "fp8_source_hash", "fp8_status_str", "fp8_ring_bytes", "fp8_ring_init", "fp8_quantize",
    "fp8_quantize_pair", "fp8_linear_fwd", "fp8_linear_bwd_dx", "fp8_db_workspace_bytes",
    "fp8_linear_bwd_dw", "fp8_gemm", "fp8_quantize_2d", "fp8_gemm_fp8out", "fp8_linear_bwd",
    "fp8_linear_bwd_dw_noalloc",
)


class Fp8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class _Operand(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("scale", ctypes.c_void_p)]


class _Ring(ctypes.Structure):
    _fields_ = [("dev", ctypes.c_void_p), ("hist_len", ctypes.c_int32), ("seeded", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        op, rp = _Operand, ctypes.POINTER(_Ring)
        L.fp8_abi_version.restype = ctypes.c_int
        L.fp8_source_hash.restype = ctypes.c_char_p
        L.fp8_source_hash.argtypes = []
        L.fp8_status_str.restype = ctypes.c_char_p
        L.fp8_status_str.argtypes = [ctypes.c_int]
        L.fp8_ring_bytes.restype = sz
        L.fp8_ring_bytes.argtypes = [i32]
        L.fp8_db_workspace_bytes.restype = sz
        L.fp8_db_workspace_bytes.argtypes = [i64, i64]
        L.fp8_ring_init.argtypes = [rp, vp, i32, vp]
        L.fp8_quantize.argtypes = [vp, i32, i64, i32, vp, rp, vp, vp, vp]
        L.fp8_quantize_pair.argtypes = [vp, i32, i64, vp, rp, vp, vp, vp, i32, i64, vp, rp, vp, vp,
                                        i32, vp]
        L.fp8_linear_fwd.argtypes = [i64, i64, i64, op, op, op, i32, rp, rp, vp, vp, vp, vp, vp, vp,
                                     vp, vp]
        L.fp8_linear_bwd_dx.argtypes = [i64, i64, i64, op, i32, rp, op, vp, vp, vp, vp, vp]
        L.fp8_linear_bwd_dw.argtypes = [i64, i64, i64, op, i32, rp, op, vp, vp, vp, vp, vp, vp, vp]
        L.fp8_linear_bwd_dw_noalloc.argtypes = [i64, i64, i64, op, i32, rp, op, vp, vp, vp, vp, vp,
                                                vp]
        L.fp8_linear_bwd.argtypes = [i64, i64, i64, op, i32, rp, op, op, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp]
        L.fp8_quantize_2d.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, rp, vp, vp, vp]
        L.fp8_gemm.argtypes = [i64, i64, i64, i64, op, i32, i64, i64, op, i32, i64, i64, op, vp,
                               i64, i64, vp]
        L.fp8_gemm_fp8out.argtypes = [i64, i64, i64, op, op, op, i32, rp, vp, vp, vp, vp]
        for name in ("fp8_ring_init", "fp8_quantize", "fp8_quantize_pair", "fp8_quantize_2d",
                     "fp8_linear_fwd", "fp8_gemm", "fp8_linear_bwd_dx",
                     "fp8_linear_bwd_dw", "fp8_gemm_fp8out", "fp8_linear_bwd",
                     "fp8_linear_bwd_dw_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().fp8_status_str(status).decode()


def fp8_abi_version() -> int:
    return lib().fp8_abi_version()


def fp8_source_hash() -> str:
    return lib().fp8_source_hash().decode()


def fp8_ring_bytes(hist_len: int) -> int:
    return lib().fp8_ring_bytes(hist_len)


def fp8_db_workspace_bytes(M: int, N: int) -> int:
    return lib().fp8_db_workspace_bytes(M, N)


# ---------------------------------------------------------------- marshalling

def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != FP8_OK:
        raise Fp8Error(status, where)


_HP = (torch.float32, torch.float16, torch.bfloat16)


def _need(t, what, dtypes=None, shape=None, numel=None, optional=True):
    """Validate a tensor argument before its pointer crosses the boundary:
    contiguous (the C ABI takes dense row-major buffers: a transposed or
    strided view would be read as the wrong elements), of an allowed dtype,
    of the expected shape or element count, on the GPU.  None passes when
    the argument is optional (the library decides whether it is needed)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{what} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous (shape {tuple(t.shape)}, "
                         f"strides {t.stride()}); pass .contiguous()")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype} not in {[str(d) for d in dtypes]}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, at least {numel} needed")


def _on_gpu(**named):
    """Second phase of the checks, after every argument's structure: each
    tensor (or Quantized operand) given lives on the GPU."""
    for what, t in named.items():
        for name, x in ((what, t.codes), (what + ".scale", t.scale)) if isinstance(t, Quantized) \
                else ((what, t),):
            if isinstance(x, torch.Tensor) and x.device.type != "cuda":
                raise ValueError(f"{name}: must be a GPU tensor (got {x.device})")


def _need_scalar(t, what, optional=True):
    _need(t, what, (torch.float32,), numel=1, optional=optional)


def _need_operand(t, what, shape, hp_ok=True):
    """A high-precision tensor or a Quantized (uint8 codes + float32 scale)."""
    if isinstance(t, Quantized):
        _need(t.codes, f"{what}.codes", (torch.uint8,), shape=shape, optional=False)
        _need_scalar(t.scale, f"{what}.scale", optional=False)
        if t.fmt not in _FMT_DT:
            raise ValueError(f"{what}: unknown fp8 format {t.fmt}")
    elif hp_ok:
        _need(t, what, _HP, shape=shape, optional=False)
    else:
        raise TypeError(f"{what}: expected a Quantized operand")


def _dims2(t, what):
    d = t.codes if isinstance(t, Quantized) else t
    if not isinstance(d, torch.Tensor) or d.dim() != 2:
        raise ValueError(f"{what}: expected a 2-D matrix")
    return d.shape


@dataclass
class Quantized:
    """Pre-quantized operand: uint8 codes, format, device float32 scale [1]."""
    codes: torch.Tensor
    fmt: int
    scale: torch.Tensor


def _operand(t) -> _Operand:
    if t is None:
        return _Operand(None, FP8_DT_BF16, None)
    if isinstance(t, Quantized):
        return _Operand(_ptr(t.codes), _FMT_DT[t.fmt], _ptr(t.scale))
    return _Operand(_ptr(t), _TORCH_DT[t.dtype], None)


class ScaleRing:
    """Delayed-scaling ring: device buffer plus the C struct (seeded mirror)."""

    def __init__(self, hist_len: int, device="cuda", stream=None):
        nbytes = fp8_ring_bytes(hist_len)
        if nbytes == 0:
            raise Fp8Error(FP8_ERR_RING, "ScaleRing")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = _Ring()
        _check(lib().fp8_ring_init(ctypes.byref(self.c), self.buf.data_ptr(), hist_len,
                                   _stream(stream)), "fp8_ring_init")

    @property
    def seeded(self) -> bool:
        return bool(self.c.seeded)

    def ref(self):
        return ctypes.byref(self.c)


def _ring(r):
    return None if r is None else r.ref()


# ---------------------------------------------------------------- entry points
# Each entry point has a *_args helper that turns tensors into the C argument
# tuple (marshalling), the call itself, and a bind_* variant that marshals
# once and returns a zero-argument callable (for launch-bound loops and graph
# capture: the pointers, sizes and stream are fixed at bind time).

def _vp(t):
    return ctypes.c_void_p(_ptr(t))


def _quantize_args(x, fmt, q, ring, scale_used, amax_out, stream):
    _need(x, "x", _HP, optional=False)
    _need(q, "q", (torch.uint8,), numel=x.numel(), optional=x.numel() == 0)
    _need_scalar(scale_used, "scale_used")
    _need_scalar(amax_out, "amax_out")
    _on_gpu(x=x, q=q, scale_used=scale_used, amax_out=amax_out)
    return (_vp(x), ctypes.c_int32(_TORCH_DT[x.dtype]), ctypes.c_int64(x.numel()),
            ctypes.c_int32(fmt), _vp(q), _ring(ring), _vp(scale_used), _vp(amax_out),
            ctypes.c_void_p(_stream(stream)))


def _quantize_pair_args(x0, q0, ring0, su0, am0, x1, q1, ring1, su1, am1, fmt, stream):
    for i, (x, q, su, am) in enumerate(((x0, q0, su0, am0), (x1, q1, su1, am1))):
        _need(x, f"x{i}", _HP, optional=False)
        _need(q, f"q{i}", (torch.uint8,), numel=x.numel(), optional=x.numel() == 0)
        _need_scalar(su, f"scale_used{i}")
        _need_scalar(am, f"amax_out{i}")
    _on_gpu(x0=x0, q0=q0, su0=su0, am0=am0, x1=x1, q1=q1, su1=su1, am1=am1)
    return (_vp(x0), ctypes.c_int32(_TORCH_DT[x0.dtype]), ctypes.c_int64(x0.numel()), _vp(q0),
            _ring(ring0), _vp(su0), _vp(am0), _vp(x1), ctypes.c_int32(_TORCH_DT[x1.dtype]),
            ctypes.c_int64(x1.numel()), _vp(q1), _ring(ring1), _vp(su1), _vp(am1),
            ctypes.c_int32(fmt), ctypes.c_void_p(_stream(stream)))


def _fwd_args(x, w, bias, fmt, y, ring_x, ring_w, x8_out, w8_out, sx_used, sw_used, amax_x,
              amax_w, stream):
    M, K = _dims2(x, "x")
    N = _dims2(w, "w")[0]
    _need_operand(x, "x", (M, K))
    _need_operand(w, "w", (N, K))
    if bias is not None:
        if isinstance(bias, Quantized):
            _need_operand(bias, "bias", (N,), hp_ok=False)
        else:
            _need(bias, "bias", (torch.bfloat16,), shape=(N,))
    _need(y, "y", (torch.bfloat16,), shape=(M, N), optional=M * N == 0)
    _need(x8_out, "x8_out", (torch.uint8,), shape=(M, K))
    _need(w8_out, "w8_out", (torch.uint8,), shape=(N, K))
    for t, n in ((sx_used, "sx_used"), (sw_used, "sw_used"), (amax_x, "amax_x"),
                 (amax_w, "amax_w")):
        _need_scalar(t, n)
    _on_gpu(x=x, w=w, bias=bias, y=y, x8_out=x8_out, w8_out=w8_out, sx_used=sx_used,
            sw_used=sw_used, amax_x=amax_x, amax_w=amax_w)
    return (ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K), _operand(x), _operand(w),
            _operand(bias), ctypes.c_int32(fmt), _ring(ring_x), _ring(ring_w), _vp(y), _vp(x8_out),
            _vp(w8_out), _vp(sx_used), _vp(sw_used), _vp(amax_x), _vp(amax_w),
            ctypes.c_void_p(_stream(stream)))


def _dx_args(g, fmt_g, w8, dx, ring_g, g8_out, sg_used, amax_g, stream):
    M, N = _dims2(g, "g")
    K = _dims2(w8, "w8")[1]
    _need_operand(g, "g", (M, N))
    _need_operand(w8, "w8", (N, K), hp_ok=False)
    _need(dx, "dx", (torch.bfloat16,), shape=(M, K), optional=M * K == 0)
    _need(g8_out, "g8_out", (torch.uint8,), shape=(M, N))
    _need_scalar(sg_used, "sg_used")
    _need_scalar(amax_g, "amax_g")
    _on_gpu(g=g, w8=w8, dx=dx, g8_out=g8_out, sg_used=sg_used, amax_g=amax_g)
    return (ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K), _operand(g),
            ctypes.c_int32(fmt_g), _ring(ring_g), _operand(w8), _vp(dx), _vp(g8_out),
            _vp(sg_used), _vp(amax_g), ctypes.c_void_p(_stream(stream)))


def _dw_args(g, fmt_g, x8, dw, db, db_ws, ring_g, g8_out, sg_used, amax_g, stream):
    M, N = _dims2(g, "g")
    K = _dims2(x8, "x8")[1]
    _need_operand(g, "g", (M, N))
    _need_operand(x8, "x8", (M, K), hp_ok=False)
    _need(dw, "dw", (torch.bfloat16,), shape=(N, K), optional=N * K == 0)
    _need(db, "db", (torch.bfloat16,), shape=(N,))
    _need(db_ws, "db_ws", (torch.float32,), numel=fp8_db_workspace_bytes(M, N) // 4)
    _need(g8_out, "g8_out", (torch.uint8,), shape=(M, N))
    _need_scalar(sg_used, "sg_used")
    _need_scalar(amax_g, "amax_g")
    _on_gpu(g=g, x8=x8, dw=dw, db=db, db_ws=db_ws, g8_out=g8_out, sg_used=sg_used, amax_g=amax_g)
    return (ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K), _operand(g),
            ctypes.c_int32(fmt_g), _ring(ring_g), _operand(x8), _vp(dw), _vp(db), _vp(db_ws),
            _vp(g8_out), _vp(sg_used), _vp(amax_g), ctypes.c_void_p(_stream(stream)))


def _bind(name, args):
    fn = getattr(lib(), name)

    def call():
        st = fn(*args)
        if st != FP8_OK:
            raise Fp8Error(st, name)
    return call


def fp8_quantize(x, fmt, q, ring=None, scale_used=None, amax_out=None, stream=None):
    _check(lib().fp8_quantize(*_quantize_args(x, fmt, q, ring, scale_used, amax_out, stream)),
           "fp8_quantize")


def bind_fp8_quantize(x, fmt, q, ring=None, scale_used=None, amax_out=None, stream=None):
    return _bind("fp8_quantize", _quantize_args(x, fmt, q, ring, scale_used, amax_out, stream))


def _quantize_2d_args(x, fmt, layout, q, qt, ring, scale_used, amax_out, stream):
    _need(x, "x", _HP, optional=False)
    if x.dim() != 2:
        raise ValueError("x: expected a 2-D matrix")
    rows, cols = x.shape
    _need(q, "q", (torch.uint8,), shape=(rows, cols))
    _need(qt, "qt", (torch.uint8,), shape=(cols, rows))
    _need_scalar(scale_used, "scale_used")
    _need_scalar(amax_out, "amax_out")
    _on_gpu(x=x, q=q, qt=qt, scale_used=scale_used, amax_out=amax_out)
    return (_vp(x), ctypes.c_int32(_TORCH_DT[x.dtype]), ctypes.c_int64(rows), ctypes.c_int64(cols),
            ctypes.c_int32(fmt), ctypes.c_int32(layout), _vp(q), _vp(qt), _ring(ring),
            _vp(scale_used), _vp(amax_out), ctypes.c_void_p(_stream(stream)))


def fp8_quantize_2d(x, fmt, layout, q=None, qt=None, ring=None, scale_used=None, amax_out=None,
                    stream=None):
    """x [rows, cols] -> q [rows, cols] and/or qt [cols, rows] (layout:
    FP8_QUANT_ROWS / _TRANSPOSED / _DUAL)."""
    _check(lib().fp8_quantize_2d(*_quantize_2d_args(x, fmt, layout, q, qt, ring, scale_used,
                                                    amax_out, stream)), "fp8_quantize_2d")


def bind_fp8_quantize_2d(x, fmt, layout, q=None, qt=None, ring=None, scale_used=None,
                         amax_out=None, stream=None):
    return _bind("fp8_quantize_2d", _quantize_2d_args(x, fmt, layout, q, qt, ring, scale_used,
                                                      amax_out, stream))


def fp8_quantize_pair(x0, q0, ring0, su0, am0, x1, q1, ring1, su1, am1, fmt, stream=None):
    """Two quantizes (x0 -> q0 with ring0, x1 -> q1 with ring1) in one call."""
    _check(lib().fp8_quantize_pair(*_quantize_pair_args(x0, q0, ring0, su0, am0, x1, q1, ring1,
                                                        su1, am1, fmt, stream)),
           "fp8_quantize_pair")


def bind_fp8_quantize_pair(x0, q0, ring0, su0, am0, x1, q1, ring1, su1, am1, fmt, stream=None):
    return _bind("fp8_quantize_pair", _quantize_pair_args(x0, q0, ring0, su0, am0, x1, q1, ring1,
                                                          su1, am1, fmt, stream))


def fp8_linear_fwd(x, w, bias, fmt, y, ring_x=None, ring_w=None, x8_out=None, w8_out=None,
                   sx_used=None, sw_used=None, amax_x=None, amax_w=None, stream=None):
    """x: [M,K] tensor or Quantized; w: [N,K] tensor or Quantized; bias: None,
    a bf16 [N] tensor or Quantized (fp8 codes with bias_scale)."""
    _check(lib().fp8_linear_fwd(*_fwd_args(x, w, bias, fmt, y, ring_x, ring_w, x8_out, w8_out,
                                           sx_used, sw_used, amax_x, amax_w, stream)),
           "fp8_linear_fwd")


def bind_fp8_linear_fwd(x, w, bias, fmt, y, ring_x=None, ring_w=None, x8_out=None, w8_out=None,
                        sx_used=None, sw_used=None, amax_x=None, amax_w=None, stream=None):
    return _bind("fp8_linear_fwd", _fwd_args(x, w, bias, fmt, y, ring_x, ring_w, x8_out, w8_out,
                                             sx_used, sw_used, amax_x, amax_w, stream))


def fp8_linear_bwd_dx(g, fmt_g, w8, dx, ring_g=None, g8_out=None, sg_used=None, amax_g=None,
                      stream=None):
    _check(lib().fp8_linear_bwd_dx(*_dx_args(g, fmt_g, w8, dx, ring_g, g8_out, sg_used, amax_g,
                                             stream)), "fp8_linear_bwd_dx")


def bind_fp8_linear_bwd_dx(g, fmt_g, w8, dx, ring_g=None, g8_out=None, sg_used=None, amax_g=None,
                           stream=None):
    return _bind("fp8_linear_bwd_dx", _dx_args(g, fmt_g, w8, dx, ring_g, g8_out, sg_used, amax_g,
                                               stream))


def fp8_linear_bwd_dw(g, fmt_g, x8, dw, db=None, db_ws=None, ring_g=None, g8_out=None,
                      sg_used=None, amax_g=None, stream=None):
    _check(lib().fp8_linear_bwd_dw(*_dw_args(g, fmt_g, x8, dw, db, db_ws, ring_g, g8_out,
                                             sg_used, amax_g, stream)), "fp8_linear_bwd_dw")


def bind_fp8_linear_bwd_dw(g, fmt_g, x8, dw, db=None, db_ws=None, ring_g=None, g8_out=None,
                           sg_used=None, amax_g=None, stream=None):
    return _bind("fp8_linear_bwd_dw", _dw_args(g, fmt_g, x8, dw, db, db_ws, ring_g, g8_out,
                                               sg_used, amax_g, stream))


def _dw_noalloc_args(g, fmt_g, x8, dw, db, ring_g, g8_out, sg_used, amax_g, stream):
    args = _dw_args(g, fmt_g, x8, dw, db, None, ring_g, g8_out, sg_used, amax_g, stream)
    return args[:9] + args[10:]  # the same arguments without db_ws


def fp8_linear_bwd_dw_noalloc(g, fmt_g, x8, dw, db=None, ring_g=None, g8_out=None, sg_used=None,
                              amax_g=None, stream=None):
    """fp8_linear_bwd_dw without a workspace: the db partials live in the
    library's static per-GPU array (no allocation; calls that overlap on one
    GPU race on it)."""
    _check(lib().fp8_linear_bwd_dw_noalloc(*_dw_noalloc_args(g, fmt_g, x8, dw, db, ring_g, g8_out,
                                                             sg_used, amax_g, stream)),
           "fp8_linear_bwd_dw_noalloc")


def bind_fp8_linear_bwd_dw_noalloc(g, fmt_g, x8, dw, db=None, ring_g=None, g8_out=None,
                                   sg_used=None, amax_g=None, stream=None):
    return _bind("fp8_linear_bwd_dw_noalloc", _dw_noalloc_args(g, fmt_g, x8, dw, db, ring_g,
                                                               g8_out, sg_used, amax_g, stream))


def _bwd_args(g, fmt_g, x8, w8, dx, dw, db, db_ws, ring_g, g8_out, sg_used, amax_g, stream,
              stream_dw):
    M, N = _dims2(g, "g")
    K = _dims2(x8, "x8")[1]
    _need_operand(g, "g", (M, N))
    _need_operand(x8, "x8", (M, K), hp_ok=False)
    _need_operand(w8, "w8", (N, K), hp_ok=False)
    _need(dx, "dx", (torch.bfloat16,), shape=(M, K), optional=M * K == 0)
    _need(dw, "dw", (torch.bfloat16,), shape=(N, K), optional=N * K == 0)
    _need(db, "db", (torch.bfloat16,), shape=(N,))
    _need(db_ws, "db_ws", (torch.float32,), numel=fp8_db_workspace_bytes(M, N) // 4)
    _need(g8_out, "g8_out", (torch.uint8,), shape=(M, N))
    _need_scalar(sg_used, "sg_used")
    _need_scalar(amax_g, "amax_g")
    _on_gpu(g=g, x8=x8, w8=w8, dx=dx, dw=dw, db=db, db_ws=db_ws, g8_out=g8_out, sg_used=sg_used,
            amax_g=amax_g)
    st = _stream(stream)
    st_dw = st if stream_dw is None else stream_dw.cuda_stream
    return (ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K), _operand(g),
            ctypes.c_int32(fmt_g), _ring(ring_g), _operand(x8), _operand(w8), _vp(dx), _vp(dw),
            _vp(db), _vp(db_ws), _vp(g8_out), _vp(sg_used), _vp(amax_g), ctypes.c_void_p(st),
            ctypes.c_void_p(st_dw))


def fp8_linear_bwd(g, fmt_g, x8, w8, dx, dw, db=None, db_ws=None, ring_g=None, g8_out=None,
                   sg_used=None, amax_g=None, stream=None, stream_dw=None):
    """Both gradients from one quantize of g: dX on stream, dW (and db) on
    stream_dw after the quantize (stream_dw None: the same stream)."""
    _check(lib().fp8_linear_bwd(*_bwd_args(g, fmt_g, x8, w8, dx, dw, db, db_ws, ring_g, g8_out,
                                           sg_used, amax_g, stream, stream_dw)), "fp8_linear_bwd")


def bind_fp8_linear_bwd(g, fmt_g, x8, w8, dx, dw, db=None, db_ws=None, ring_g=None, g8_out=None,
                        sg_used=None, amax_g=None, stream=None, stream_dw=None):
    return _bind("fp8_linear_bwd", _bwd_args(g, fmt_g, x8, w8, dx, dw, db, db_ws, ring_g, g8_out,
                                             sg_used, amax_g, stream, stream_dw))


def _matrix_view(t, what):
    """(batch, rows, cols, batch_stride, layout, ld) of a 2-D or 3-D tensor
    whose last two dims are (rows, k): k-contiguous rows, or the transposed
    view of such rows (k strided).  A batch dim of size 1 or stride 0 is
    broadcast."""
    if t.dim() == 2:
        t3, bstride = t.unsqueeze(0), 0
    elif t.dim() == 3:
        t3, bstride = t, (0 if t.shape[0] == 1 else t.stride(0))
    else:
        raise ValueError(f"{what}: expected a 2-D or 3-D tensor")
    B, R, Kd = t3.shape
    if t3.stride(2) == 1 or Kd <= 1:
        return B, R, Kd, bstride, FP8_K_CONTIG, max(t3.stride(1), Kd, 1)
    if t3.stride(1) == 1 or R <= 1:
        return B, R, Kd, bstride, FP8_K_STRIDED, max(t3.stride(2), R, 1)
    raise ValueError(f"{what}: neither dim of the matrix is contiguous")


def _gemm_args(a, b, c, bias, stream):
    Ba, M, K, sa, la, lda = _matrix_view(a.codes, "a")
    Bb, N, Kb, sb, lb, ldb = _matrix_view(b.codes, "b")
    if K != Kb:
        raise ValueError("a and b disagree on K")
    batch = max(Ba, Bb)
    if Ba not in (1, batch) or Bb not in (1, batch):
        raise ValueError("batch sizes do not broadcast")
    c3 = c if c.dim() == 3 else c.unsqueeze(0)
    if tuple(c3.shape) != (batch, M, N) or c3.stride(2) != 1:
        raise ValueError("c must be [batch, M, N] (or [M, N]) with contiguous rows")
    return (ctypes.c_int64(batch), ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K),
            _operand(a), ctypes.c_int32(la), ctypes.c_int64(lda), ctypes.c_int64(sa),
            _operand(b), ctypes.c_int32(lb), ctypes.c_int64(ldb), ctypes.c_int64(sb),
            _operand(bias), _vp(c), ctypes.c_int64(max(c3.stride(1), N)),
            ctypes.c_int64(c3.stride(0) if batch > 1 else 0), ctypes.c_void_p(_stream(stream)))


def fp8_gemm(a, b, c, bias=None, stream=None):
    """c[z] = a[z] b[z]^T / (sa sb) (+ bias), bf16.  a: Quantized with codes
    [.., M, K]; b: Quantized with codes [.., N, K]; either may be a transposed
    view (.mT of a [.., K, M] buffer) and either may be 2-D or have batch 1
    (broadcast).  c: bf16 [.., M, N]."""
    _check(lib().fp8_gemm(*_gemm_args(a, b, c, bias, stream)), "fp8_gemm")


def bind_fp8_gemm(a, b, c, bias=None, stream=None):
    return _bind("fp8_gemm", _gemm_args(a, b, c, bias, stream))



def _gemm_fp8out_args(a, b, c8, fmt_out, ring_out, scale_used, amax_out, bias, stream):
    M, K = _dims2(a, "a")
    N = _dims2(b, "b")[0]
    _need_operand(a, "a", (M, K), hp_ok=False)
    _need_operand(b, "b", (N, K), hp_ok=False)
    _need(c8, "c8", (torch.uint8,), shape=(M, N), optional=False)
    _need_scalar(scale_used, "scale_used")
    _need_scalar(amax_out, "amax_out")
    if bias is not None:
        if isinstance(bias, Quantized):
            _need_operand(bias, "bias", (N,), hp_ok=False)
        else:
            _need(bias, "bias", (torch.bfloat16,), shape=(N,))
    _on_gpu(a=a, b=b, c8=c8, scale_used=scale_used, amax_out=amax_out, bias=bias)
    return (ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K), _operand(a), _operand(b),
            _operand(bias), ctypes.c_int32(fmt_out), _ring(ring_out), _vp(c8), _vp(scale_used),
            _vp(amax_out), ctypes.c_void_p(_stream(stream)))


def fp8_gemm_fp8out(a, b, c8, fmt_out, ring_out, scale_used, amax_out=None, bias=None,
                    stream=None):
    """c8 = enc_fmt_out(fl32(y * s_out)), y = a b^T / (sa sb) (+ bias) in fp32,
    s_out from ring_out (delayed scaling; folded with max |y|).  a, b:
    Quantized with contiguous codes [M, K] and [N, K]; c8: uint8 [M, N]."""
    _check(lib().fp8_gemm_fp8out(*_gemm_fp8out_args(a, b, c8, fmt_out, ring_out, scale_used,
                                                    amax_out, bias, stream)), "fp8_gemm_fp8out")


def bind_fp8_gemm_fp8out(a, b, c8, fmt_out, ring_out, scale_used, amax_out=None, bias=None,
                         stream=None):
    return _bind("fp8_gemm_fp8out", _gemm_fp8out_args(a, b, c8, fmt_out, ring_out, scale_used,
                                                      amax_out, bias, stream))

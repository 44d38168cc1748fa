"""Python binding of libfp8probe.so, the measurement kernels (an MFMA-only
ceiling and a plain HBM stream; include/fp8probe.h).  Used by bench.py to
measure the machine's own ceilings beside the published peaks; not part of
the FP8 linear path."""

from __future__ import annotations

import ctypes
import os

import torch

from ._build import PROBE_LIB_PATH

C_SYMBOLS = ("fp8probe_mfma", "fp8probe_stream")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.fp8probe_mfma.argtypes = [i32, i32, vp, vp, vp]
        L.fp8probe_stream.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        L.fp8probe_mfma.restype = L.fp8probe_stream.restype = ctypes.c_int
        _lib = L
    return _lib


def _stream(stream):
    return (stream or torch.cuda.current_stream()).cuda_stream


def mfma_codes(random: bool, device="cuda", seed=0) -> torch.Tensor:
    """512 * 64 words of e4m3 operand codes: random finite codes (bytes other
    than 0x7F / 0xFF, the NaN codes), or zeros."""
    if not random:
        return torch.zeros(512 * 64, dtype=torch.int32, device=device)
    g = torch.Generator().manual_seed(seed)
    b = torch.randint(0, 254, (512 * 64 * 4,), generator=g, dtype=torch.int32)
    b = torch.where(b >= 0x7F, b + 1, b).to(torch.uint8)  # skip 0x7F; 0xFF is never drawn
    return b.view(torch.int32).to(device)


def mfma(blocks: int, iters: int, codes: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    st = lib().fp8probe_mfma(blocks, iters, codes.data_ptr(), out.data_ptr(), _stream(stream))
    if st:
        raise RuntimeError(f"fp8probe_mfma: status {st}")


def mfma_flops(blocks: int, iters: int) -> float:
    return float(blocks) * 8 * iters * 4 * 2 * 32 * 32 * 64


def stream(src, dst, nbytes: int, mode: int, blocks_per_cu: int, sink, stream=None) -> None:
    st = lib().fp8probe_stream(None if src is None else src.data_ptr(),
                               None if dst is None else dst.data_ptr(), nbytes, mode,
                               blocks_per_cu, sink.data_ptr(), _stream(stream))
    if st:
        raise RuntimeError(f"fp8probe_stream: status {st}")

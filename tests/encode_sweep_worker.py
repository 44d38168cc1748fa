"""Worker of the exhaustive encoder sweep (tests/test_quantize_gpu.py): the
oracle's encoding of one contiguous range of fp32 bit patterns.  Imported by
spawned processes, so it imports numpy and the oracle only (no torch, no
GPU)."""

import numpy as np

from oracle import fp8_oracle as O


def encode_bits(first: int, count: int, negative: bool, fmt: int) -> np.ndarray:
    """Codes of the fp32 values whose bit patterns are first .. first+count-1
    (with the sign bit set when negative)."""
    bits = np.arange(first, first + count, dtype=np.uint64).astype(np.uint32)
    if negative:
        bits |= np.uint32(0x80000000)
    return O.encode(bits.view(np.float32), fmt)

"""CPU checks of the Python binding's argument validation: every tensor is
checked (contiguous, dtype, shape, on the GPU) before a pointer crosses the
C ABI, so a transposed view or a host tensor raises instead of being read as
the wrong bytes.  No kernel runs: each call fails in the marshalling."""

import pytest
import torch

import scaled_quantize_fp8_amd as F


def _fwd(x, w, y, **kw):
    F.fp8_linear_fwd(x, w, None, F.FP8_E4M3, y, **kw)


def test_transposed_view_raises():
    x = torch.zeros(64, 32, dtype=torch.bfloat16).mT  # [32, 64], strides (1, 32)
    w = torch.zeros(16, 64, dtype=torch.bfloat16)
    y = torch.zeros(32, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        _fwd(x, w, y)
    q8 = F.Quantized(torch.zeros(64, 32, dtype=torch.uint8).mT, F.FP8_E4M3,
                     torch.ones(1))
    with pytest.raises(ValueError, match="contiguous"):
        F.fp8_linear_bwd_dx(torch.zeros(16, 32, dtype=torch.bfloat16).mT, F.FP8_E5M2,
                            F.Quantized(torch.zeros(16, 64, dtype=torch.uint8), F.FP8_E4M3,
                                        torch.ones(1)), torch.zeros(32, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="contiguous"):
        F.fp8_linear_bwd_dw(torch.zeros(32, 16, dtype=torch.bfloat16), F.FP8_E5M2, q8,
                            torch.zeros(16, 64, dtype=torch.bfloat16))


def test_host_tensor_raises():
    x = torch.zeros(32, 64, dtype=torch.bfloat16)
    w = torch.zeros(16, 64, dtype=torch.bfloat16)
    y = torch.zeros(32, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        _fwd(x, w, y)
    with pytest.raises(ValueError, match="GPU tensor"):
        F.fp8_quantize(x, F.FP8_E4M3, torch.zeros(32 * 64, dtype=torch.uint8))


def test_wrong_dtype_and_shape_raise():
    x = torch.zeros(32, 64, dtype=torch.bfloat16)
    w = torch.zeros(16, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="dtype"):
        _fwd(x, w, torch.zeros(32, 16, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        _fwd(x, w, torch.zeros(16, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        _fwd(x, torch.zeros(16, 48, dtype=torch.bfloat16), torch.zeros(32, 16, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="dtype"):
        F.fp8_quantize(torch.zeros(8, dtype=torch.int32), F.FP8_E4M3,
                       torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="at least"):
        F.fp8_linear_bwd_dw(torch.zeros(64, 16, dtype=torch.bfloat16), F.FP8_E5M2,
                            F.Quantized(torch.zeros(64, 32, dtype=torch.uint8), F.FP8_E4M3,
                                        torch.ones(1)),
                            torch.zeros(16, 32, dtype=torch.bfloat16),
                            db=torch.zeros(16, dtype=torch.bfloat16),
                            db_ws=torch.zeros(1, dtype=torch.float32))

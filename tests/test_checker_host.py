"""CPU checks of the GPU tests' acceptance helper (tests/gpu_util.check_gemm):
an output planted with NaN, infinity, or an error just past either bound
must fail; the exact rounded reference must pass."""

import numpy as np
import pytest

from oracle import fp8_oracle as O
from tests.gpu_util import check_gemm


def _ref():
    rng = np.random.default_rng(3)
    tab = O.decode_table(O.E4M3)
    fin = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    x8 = rng.choice(fin, size=(16, 64))
    w8 = rng.choice(fin, size=(8, 64))
    return O.linear_fwd(x8, w8, O.E4M3, 2.0, 4.0)


def test_rounded_reference_passes():
    ref = _ref()
    check_gemm(ref.y_bits, ref, "exact")


@pytest.mark.parametrize("bits", [0x7FC0, 0xFFC0, 0x7F80, 0xFF80])
def test_nan_or_inf_output_fails(bits):
    ref = _ref()
    y = ref.y_bits.copy()
    y[3, 5] = bits
    with pytest.raises(AssertionError, match="non-finite"):
        check_gemm(y, ref, "planted")


def test_error_past_the_diagnostic_bound_fails():
    ref = _ref()
    # the element whose bf16 spacing is smallest against its sum |ab| (most
    # cancellation), moved by 2^-9 of that sum plus two spacings: inside the
    # 2^-7 contract, outside the 2^-10 diagnostic bound
    i, j = np.unravel_index(np.argmin(O.bf16_ulp(ref.r) / ref.abs_sum), ref.r.shape)
    r = ref.r.copy()
    r[i, j] += 2.0 ** -9 * ref.abs_sum[i, j] + 2 * O.bf16_ulp(ref.r[i, j])
    with pytest.raises(AssertionError, match="2\\^-10"):
        check_gemm(O.bf16_bits(r), ref, "planted")
    r = ref.r.copy()
    r[i, j] += 2.0 ** -6 * ref.abs_sum[i, j]
    with pytest.raises(AssertionError, match="2\\^-7"):
        check_gemm(O.bf16_bits(r), ref, "planted")

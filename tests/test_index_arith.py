"""Exhaustive host check of the integer-division shortcut the small-M kernels
use while staging x: for 0 <= i < 2^13 and every divisor d >= 1 a kernel can
pass, truncating the FP32 product (i + 1/2) * RN(1/d) gives exactly i // d.
The kernels compute RN(1/d) with a correctly rounded division and the
product in one rounding; numpy's float32 arithmetic does the same."""
import numpy as np


def test_row_index_by_reciprocal_product_is_exact():
    i = np.arange(1 << 13, dtype=np.int64)
    fi = i.astype(np.float32) + np.float32(0.5)
    for d in range(1, (1 << 13) + 1):
        inv = np.float32(1.0) / np.float32(d)
        got = (fi * inv).astype(np.int64)  # truncation toward zero, as int(float)
        np.testing.assert_array_equal(got, i // d, err_msg=f"d = {d}")


def test_float32_operations_round_to_nearest():
    # the check above relies on one rounding per operation: a product whose
    # exact value needs more than 24 bits must round to nearest
    a = np.float32(1 + 2 ** -12)
    assert a * a == np.float32(1 + 2 ** -11)  # exact 1 + 2^-11 + 2^-24: the 2^-24 rounds off

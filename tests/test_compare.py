"""CPU checks of the comparator itself: the 16-bit bar accepts a correctly
rounded result and a one-ulp slip at a near-tie, and rejects a result
rounded the wrong way (truncation) away from a tie."""
import numpy as np
import pytest

import oracle
from smx_compare import check


def _rows(dtype):
    rng = np.random.default_rng(5)
    p = rng.uniform(0.0, 1.0, (4, 512))
    p /= p.sum(1, keepdims=True)
    cls = np.zeros(p.shape, dtype=np.uint8)
    st = np.zeros(p.shape[0], dtype=np.int32)
    return p, cls, st


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_correct_rounding_passes(dtype):
    p, cls, st = _rows(dtype)
    y = oracle.encode(p, dtype)
    out = check(y, dtype, p, cls, st, "rne")
    assert out["max_ulp"] == 0 and out["exact_lanes"] > 0.9 * p.size


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_truncation_fails(dtype):
    p, cls, st = _rows(dtype)
    y = oracle.encode(p, dtype).astype(np.int64)
    # truncation: step down wherever the correctly rounded value lies above p
    up = np.array([oracle.decode(np.array([b], dtype=np.uint16), dtype)[0] for b in y.ravel()]).reshape(p.shape) > p
    y_trunc = np.where(up, y - 1, y).astype(np.uint16)
    with pytest.raises(AssertionError, match="clear of a rounding midpoint"):
        check(y_trunc, dtype, p, cls, st, "truncated")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_near_tie_slip_passes(dtype):
    # a value within 2^-20 (relative) of a midpoint may round either way
    p, cls, st = _rows(dtype)
    y = oracle.encode(p, dtype).astype(np.int64)
    lo = np.array([oracle.decode(np.array([b], dtype=np.uint16), dtype)[0] for b in y[0, :8]])
    hi = np.array([oracle.decode(np.array([b + 1], dtype=np.uint16), dtype)[0] for b in y[0, :8]])
    mid = 0.5 * (lo + hi)
    p[0, :8] = mid * (1 + 2.0 ** -22)  # just above the tie: rounds up
    y = oracle.encode(p, dtype).astype(np.int64)
    y[0, :8] -= 1  # the kernel's fp32 error put them just below the tie
    check(y.astype(np.uint16), dtype, p, cls, st, "near tie")

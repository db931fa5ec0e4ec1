"""Comparison of library outputs against the oracle, to the stated bars.

* f32 output: per element |y - r| / max(|r|, FLT_MIN) <= 1e-6 (FLT_MIN =
  2^-126, so a subnormal reference is held to about 8 subnormal ulps), and
  for every row that is not a policy row |sum(y) - 1| <= 1e-5 (summed in
  double).
* f16 / bf16 output: within 1 ulp of the oracle's value rounded once to the
  format (bit patterns compared as integers; outputs are >= 0 so the order is
  monotone).
* policy lanes (masked, -inf, empty row, NaN row): bit-exact +0.0 or the
  canonical quiet NaN.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

F32_REL_TOL = 1e-6
F32_SUM_TOL = 1e-5
ULP_TOL = 1
FLT_MIN = np.float64(2.0 ** -126)
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(x_raw: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x_raw, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(x_raw).view(np.int16)).to(device)
    return t.view(TORCH_DTYPE[dtype])


def to_host(y: torch.Tensor, dtype: str) -> np.ndarray:
    """Raw storage on the host: float32, or uint16 bit patterns."""
    if dtype == "f32":
        return y.detach().cpu().numpy()
    return y.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_of(y_raw: np.ndarray, dtype: str) -> np.ndarray:
    return y_raw.view(np.uint32).astype(np.int64) if dtype == "f32" else y_raw.astype(np.int64)


def check(y_raw: np.ndarray, dtype: str, p: np.ndarray, cls: np.ndarray, st: np.ndarray, what: str = ""):
    """Assert y matches the oracle's (p, lane class, row status); return stats."""
    assert y_raw.shape == p.shape, (y_raw.shape, p.shape)
    bits = bits_of(y_raw, dtype)
    zero = cls == oracle.LANE_ZERO
    nan = cls == oracle.LANE_NAN
    num = cls == oracle.LANE_NUMERIC
    bad_zero = np.count_nonzero(bits[zero] != 0)
    bad_nan = np.count_nonzero(bits[nan] != NAN_BITS[dtype])
    assert bad_zero == 0, f"{what}: {bad_zero} policy-zero lanes are not +0.0"
    assert bad_nan == 0, f"{what}: {bad_nan} policy-NaN lanes are not the canonical NaN"
    out = {"numeric_lanes": int(num.sum())}
    if dtype == "f32":
        y = y_raw.astype(np.float64)
        rel = np.zeros_like(p)
        rel[num] = np.abs(y[num] - p[num]) / np.maximum(np.abs(p[num]), FLT_MIN)
        worst = float(rel.max()) if rel.size else 0.0
        if worst > F32_REL_TOL:
            i = np.unravel_index(np.argmax(rel), rel.shape)
            raise AssertionError(f"{what}: f32 relative error {worst:.3e} at {i}: got {y[i]!r} want {p[i]!r}")
        ok_rows = st == oracle.ROW_OK
        if ok_rows.any():
            sums = np.where(num, y, 0.0)[ok_rows].sum(axis=1)
            dev = float(np.abs(sums - 1.0).max())
            assert dev <= F32_SUM_TOL, f"{what}: |sum - 1| = {dev:.3e}"
            out["max_sum_dev"] = dev
        out["max_rel"] = worst
    else:
        want = oracle.encode(np.where(num, p, 0.0), dtype).astype(np.int64)
        d = np.abs(bits - want)
        d[~num] = 0
        worst = int(d.max()) if d.size else 0
        if worst > ULP_TOL:
            i = np.unravel_index(np.argmax(d), d.shape)
            raise AssertionError(f"{what}: {worst} ulp at {i}: got {bits[i]:#06x} want {want[i]:#06x} (ref {p[i]!r})")
        out["max_ulp"] = worst
        out["frac_off_by_one"] = float(np.count_nonzero(d[num])) / max(1, int(num.sum()))
    return out

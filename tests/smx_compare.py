"""Comparison of library outputs against the oracle, to the stated bars.

* f32 output: per element |y - r| / max(|r|, FLT_MIN) <= 1e-6 (FLT_MIN =
  2^-126, so a subnormal reference is held to about 8 subnormal ulps), and
  for every row that is not a policy row |sum(y) - 1| <= 1e-5 (summed in
  double).
* f16 / bf16 output: within 1 ulp of the oracle's value rounded once to the
  format (bit patterns compared as integers; outputs are >= 0 so the order is
  monotone), and exactly that rounded value wherever the oracle's value is
  clear of a rounding midpoint by more than the kernel's fp32 error (2^-16
  relative): the 1-ulp allowance covers near-ties only, so a kernel that
  truncated, or rounded ties the wrong way far from a tie, fails.
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


CLEAR_REL = 2.0 ** -16


def exact_where_clear(bits, ref, dtype, sel, margin, what):
    """16-bit lanes in sel whose reference rounds to the same pattern at
    ref - margin and ref + margin must hold exactly that pattern."""
    if not sel.any():
        return 0
    r = ref[sel]
    m = np.broadcast_to(margin, ref.shape)[sel]
    want = oracle.encode(r, dtype).astype(np.int64)
    lo = oracle.encode(r - m, dtype).astype(np.int64)
    hi = oracle.encode(r + m, dtype).astype(np.int64)
    clear = (lo == want) & (hi == want)
    got = bits[sel]
    bad = clear & (got != want)
    if bad.any():
        i = int(np.argmax(bad))
        idx = tuple(np.argwhere(sel)[i])
        raise AssertionError(f"{what}: lane {idx} is clear of a rounding midpoint but got {got[i]:#06x}, "
                             f"the correctly rounded value is {want[i]:#06x} (ref {r[i]!r})")
    return int(clear.sum())


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
        out["exact_lanes"] = exact_where_clear(bits, p, dtype, num, CLEAR_REL * np.abs(p), what)
    return out


# ---------------------------------------------------------------------------
# Log-domain outputs (log-softmax and the per-row log-sum-exp)
# ---------------------------------------------------------------------------
#
# The references are the oracle's double-precision x - LSE and LSE. The GPU
# forms LSE = m + log(l) and x - LSE in fp32, so near-cancelling lanes carry
# the fp32 resolution of the operands:
#   f32     : |y - r| <= 1e-6 * max(1, |x|, |LSE|)
#   f16/bf16: within 1 ulp of the rounded reference, or
#             |y - r| <= 2^-22 * max(1, |x|, |LSE|)
#   LSE     : |lse - LSE| <= 1e-6 * max(1, |LSE|)
# Policy lanes are bit-exact: masked / -inf lanes and empty rows -inf, NaN
# rows the canonical NaN (and NaN / -inf in lse).

LOG_F32_TOL = 1e-6
LOG_16_ABS = 2.0 ** -22
NEG_INF_BITS = {"f32": 0xFF800000, "f16": 0xFC00, "bf16": 0xFF80}


def check_log(y_raw, dtype, logp, lse_ref, lse_got, cls, st, x_float, what=""):
    out = {}
    if lse_got is not None:
        ok_rows = st == oracle.ROW_OK
        g = lse_got.astype(np.float64)
        assert np.array_equal(np.isnan(g), st == oracle.ROW_POISON), f"{what}: lse NaN rows differ"
        assert (lse_got[st == oracle.ROW_POISON].view(np.uint32) == 0x7FC00000).all(), f"{what}: lse NaN bits"
        assert (g[st == oracle.ROW_EMPTY] == -np.inf).all(), f"{what}: empty rows need lse = -inf"
        if ok_rows.any():
            err = np.abs(g[ok_rows] - lse_ref[ok_rows]) / np.maximum(1.0, np.abs(lse_ref[ok_rows]))
            assert err.max() <= LOG_F32_TOL, f"{what}: lse error {err.max():.3e}"
            out["lse_max_err"] = float(err.max())
    if y_raw is None:
        return out
    bits = bits_of(y_raw, dtype)
    zero = cls == oracle.LANE_ZERO
    nan = cls == oracle.LANE_NAN
    num = cls == oracle.LANE_NUMERIC
    assert (bits[zero] == NEG_INF_BITS[dtype]).all(), f"{what}: masked lanes must be -inf"
    assert (bits[nan] == NAN_BITS[dtype]).all(), f"{what}: NaN rows must be the canonical NaN"
    lse_b = np.broadcast_to(np.where(st == oracle.ROW_OK, lse_ref, 0.0)[:, None], logp.shape)
    with np.errstate(invalid="ignore"):  # NaN lanes of policy rows; only numeric lanes use the scale
        scale = np.maximum(1.0, np.maximum(np.abs(x_float.astype(np.float64)), np.abs(lse_b)))
    y = y_raw.astype(np.float64) if dtype == "f32" else \
        (y_raw.view(np.float16).astype(np.float64) if dtype == "f16"
         else (y_raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    err = np.zeros_like(logp)
    err[num] = np.abs(y[num] - logp[num]) / scale[num]
    if dtype == "f32":
        worst = float(err.max()) if err.size else 0.0
        if worst > LOG_F32_TOL:
            i = np.unravel_index(np.argmax(err), err.shape)
            raise AssertionError(f"{what}: log error {worst:.3e} at {i}: got {y[i]!r} want {logp[i]!r}")
        out["max_err"] = worst
    else:
        want = oracle.encode(np.where(num, logp, 0.0), dtype).astype(np.int64)
        d = np.abs(bits - want)
        bad = num & (d > ULP_TOL) & (err > LOG_16_ABS)
        if bad.any():
            i = np.argwhere(bad)[0]
            i = tuple(i)
            raise AssertionError(f"{what}: {d[i]} ulp at {i}: got {bits[i]:#06x} want {want[i]:#06x} (ref {logp[i]!r})")
        out["max_ulp"] = int(d[num].max()) if num.any() else 0
        big = num & (np.abs(logp) >= 2.0 ** -8)
        out["max_ulp_away_from_0"] = int(d[big].max()) if big.any() else 0
        out["exact_lanes"] = exact_where_clear(bits, logp, dtype, num, 2.0 ** -20 * scale, what)
    return out


# ---------------------------------------------------------------------------
# Softmax backward (dx = p * (g - g.p))
# ---------------------------------------------------------------------------
#
# The forward error of p_j * (g_j - s) scales with p_j * (|g_j| + sum|g_k p_k|),
# so the bars are relative to that scale:
#   f32      : |dx - r| <= 1e-6  * max(p_j (|g_j| + sum_k |g_k p_k|), 2^-126)
#              (the floor is the forward's: a subnormal result is held to
#              about 8 subnormal steps)
#   f16/bf16 : within 1 ulp of the rounded reference, or
#              |dx - r| <= 2^-20 * p_j (|g_j| + sum_k |g_k p_k|)
# Rows holding a NaN in p or g must be the canonical NaN in every lane.

BWD_F32_TOL = 1e-6
BWD_16_TOL = 2.0 ** -20


def check_bwd(dx_raw, dtype, ref, p_f64, g_f64, what=""):
    nan_rows = np.isnan(p_f64).any(1) | np.isnan(g_f64).any(1)
    bits = bits_of(dx_raw, dtype)
    assert (bits[nan_rows] == NAN_BITS[dtype]).all(), f"{what}: NaN rows must be the canonical NaN"
    ok = ~nan_rows
    p, g, r = p_f64[ok], g_f64[ok], ref[ok]
    scale = np.abs(p) * (np.abs(g) + np.abs(g * p).sum(1, keepdims=True))
    if dtype == "f32":
        y = dx_raw[ok].astype(np.float64)
        err = np.abs(y - r)
        scale = np.maximum(scale, FLT_MIN)
        bad = err > BWD_F32_TOL * scale
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"{what}: dx error {err[i]:.3e} > {BWD_F32_TOL * scale[i]:.3e} at {i}")
        return {"max_err_over_scale": float((err / np.maximum(scale, 1e-300)).max()) if err.size else 0.0}
    y = (dx_raw[ok].view(np.float16).astype(np.float64) if dtype == "f16"
         else (dx_raw[ok].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    want = oracle.encode(r, dtype).astype(np.int64)
    d = np.abs(bits[ok] - want)
    err = np.abs(y - r)
    bad = (d > ULP_TOL) & (err > BWD_16_TOL * scale)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {d[i]} ulp and error {err[i]:.3e} at {i} (ref {r[i]!r})")
    far = np.abs(r) >= 2.0 ** -8 * scale
    full = np.zeros(bits.shape, dtype=bool)
    full[ok] = True
    ref_full = np.zeros(bits.shape)
    ref_full[ok] = r
    scale_full = np.zeros(bits.shape)
    scale_full[ok] = scale
    return {"max_ulp": int(d.max()) if d.size else 0,
            "max_ulp_without_cancellation": int(d[far].max()) if far.any() else 0,
            "exact_lanes": exact_where_clear(bits, ref_full, dtype, full, CLEAR_REL * scale_full, what)}


# ---------------------------------------------------------------------------
# Cross-entropy with logits (loss_r = LSE - x_t, dx = p - onehot(t))
# ---------------------------------------------------------------------------
#
# loss (fp32): |loss - r| <= 1e-6 * max(|r|, a, 2^-126), with a = 0 when the
#   target holds the row maximum (the log1p form keeps full relative
#   precision) and a = 1 otherwise (the fp32 resolution of m - x_t + log l);
#   the 2^-126 floor is the fp32 output's, as for dx: a loss below the
#   smallest normal fp32 number is held to about 8 subnormal steps, and one
#   below the smallest subnormal rounds to 0, which is then its value;
# dx: the softmax bars (f32 relative 1e-6 with the 2^-126 floor, f16/bf16
#   1 ulp), the target lane included (its value -(others / l) is accurate);
# policy: ignored rows loss 0 and dx +0.0; poisoned rows NaN; an empty row or
#   a masked / -inf target gives loss +inf; policy lanes of dx bit-exact
#   (+0.0, or -1.0 at the target of an empty row).

XENT_TOL = 1e-6


def check_xent(loss_got, dx_raw, dtype, loss_ref, dx_ref, x_float, target, what=""):
    rows, cols = x_float.shape
    t = target.astype(np.int64)
    ignored = (t < 0) | (t >= cols)
    lr = loss_ref
    assert (loss_got[ignored] == 0).all(), f"{what}: ignored rows need loss 0"
    nanr = np.isnan(lr)
    assert (loss_got[nanr].view(np.uint32) == 0x7FC00000).all(), f"{what}: poisoned rows need the canonical NaN"
    infr = lr == np.inf
    assert (loss_got[infr] == np.inf).all(), f"{what}: rows with an unreachable target need +inf"
    num = ~(ignored | nanr | infr)
    out = {}
    if num.any():
        rows_i = np.nonzero(num)[0]
        xt = x_float[rows_i, t[rows_i]].astype(np.float64)
        rowmax = np.nanmax(np.where(np.isfinite(x_float[rows_i]), x_float[rows_i], -np.inf), axis=1)
        a = np.where(xt == rowmax, 0.0, 1.0)
        err = np.abs(loss_got[rows_i].astype(np.float64) - lr[rows_i])
        bound = XENT_TOL * np.maximum(np.maximum(np.abs(lr[rows_i]), a), FLT_MIN)
        bad = err > bound
        if bad.any():
            i = rows_i[np.argmax(bad)]
            raise AssertionError(f"{what}: loss row {i}: got {loss_got[i]!r} want {lr[i]!r}")
        out["loss_max_err_ratio"] = float((err / np.maximum(bound, 1e-300)).max())
    if dx_raw is None:
        return out
    bits = bits_of(dx_raw, dtype)
    zero_bits = 0
    assert (bits[ignored] == zero_bits).all(), f"{what}: ignored rows need dx = +0.0"
    assert (bits[nanr] == NAN_BITS[dtype]).all(), f"{what}: poisoned rows need NaN dx"
    live = ~(ignored | nanr)
    # lanes whose reference is exactly 0 or -1 (masked lanes, empty rows) are
    # policy values and must match bit for bit
    exact = live[:, None] & ((dx_ref == 0) | (dx_ref == -1)) & (np.abs(dx_ref) >= 0)
    want_bits = bits_of(oracle.encode(np.where(exact, dx_ref, 0.0), dtype), dtype)
    mism = exact & (bits != want_bits)
    # a numeric lane may round to exactly 0 or -1 legitimately; only lanes the
    # oracle puts at exactly 0 / -1 are held to bits, and those are policy
    # lanes or exact results (one valid lane: dx_t = 0)
    if mism.any():
        i = tuple(np.argwhere(mism)[0])
        raise AssertionError(f"{what}: policy lane {i} got {bits[i]:#x} want {want_bits[i]:#x}")
    numl = live[:, None] & ~exact
    if dtype == "f32":
        y = dx_raw.astype(np.float64)
        rel = np.zeros_like(dx_ref)
        rel[numl] = np.abs(y[numl] - dx_ref[numl]) / np.maximum(np.abs(dx_ref[numl]), FLT_MIN)
        worst = float(rel.max()) if rel.size else 0.0
        if worst > F32_REL_TOL:
            i = np.unravel_index(np.argmax(rel), rel.shape)
            raise AssertionError(f"{what}: dx relative error {worst:.3e} at {i}: got {y[i]!r} want {dx_ref[i]!r}")
        out["dx_max_rel"] = worst
    else:
        want = oracle.encode(np.where(numl, dx_ref, 0.0), dtype).astype(np.int64)
        d = np.abs(bits - want)
        d[~numl] = 0
        worst = int(d.max()) if d.size else 0
        if worst > ULP_TOL:
            i = np.unravel_index(np.argmax(d), d.shape)
            raise AssertionError(f"{what}: dx {worst} ulp at {i}: got {bits[i]:#06x} want {want[i]:#06x} (ref {dx_ref[i]!r})")
        out["dx_max_ulp"] = worst
        out["dx_exact_lanes"] = exact_where_clear(bits, dx_ref, dtype, numl, CLEAR_REL * np.abs(dx_ref), what)
    return out


# ---------------------------------------------------------------------------
# Softmax-weighted value sums (out = softmax(s) @ V)
# ---------------------------------------------------------------------------
#
# The kernel's error in fp32, before the final rounding, is bounded by
# 2^-14 * sum_j p_j |V_jk| + 2^-30 (the weights enter as 16-bit hi + lo
# pairs, about 2^-17 relative down to 2^-39; fp32 accumulation over up to
# 2 * cols / 16 matrix-core steps adds at most a few 2^-24 each, which keeps
# the worst case inside 2^-14 for rows up to about 2,000 columns; longer rows
# stay inside it in practice because those rounding errors do not all share
# one sign, as the tests on rows of 165,000 and 8,388,616 columns show; the absolute
# term covers the weights below 2^-39 that fp16 cannot carry), so an output
# component must be within 1 ulp of the correctly rounded oracle value or
# within that bound, and exactly the rounded value wherever the reference is
# clear of a rounding midpoint by more than the bound. Policy: poisoned rows
# are the canonical NaN in every component, empty rows +0.0.

WEIGHTED_TOL = 2.0 ** -14
WEIGHTED_FLOOR = 2.0 ** -30


def _ordered16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)


def check_weighted(out_raw, dtype, ref, st, scale, what=""):
    """out_raw: uint16 [rows, d]; ref, scale: float64 [rows, d] (scale =
    sum_j p_j |V_jk|); st: row status."""
    bits = bits_of(out_raw, dtype)
    pois = st == oracle.ROW_POISON
    empty = st == oracle.ROW_EMPTY
    assert (bits[pois] == NAN_BITS[dtype]).all(), f"{what}: poisoned rows must be the canonical NaN"
    assert (bits[empty] == 0).all(), f"{what}: empty rows must be +0.0"
    ok = st == oracle.ROW_OK
    if not ok.any():
        return {}
    y = oracle.decode(out_raw[ok], dtype) if out_raw[ok].size < 4096 else (
        (out_raw[ok].astype(np.uint32) << 16).view(np.float32).astype(np.float64) if dtype == "bf16"
        else out_raw[ok].view(np.float16).astype(np.float64))
    r = ref[ok]
    sc = scale[ok]
    want = oracle.encode(r, dtype).astype(np.int64)
    ulps = np.abs(_ordered16(bits[ok]) - _ordered16(want))
    err = np.abs(y - r)
    bound = WEIGHTED_TOL * sc + WEIGHTED_FLOOR
    bad = (ulps > ULP_TOL) & (err > bound)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {ulps[i]} ulp and error {err[i]:.3e} > {bound[i]:.3e} at {i} "
                             f"(got {y[i]!r}, ref {r[i]!r})")
    sel = np.ones(r.shape, dtype=bool)
    exact = exact_where_clear(bits[ok], r, dtype, sel, bound, what)
    return {"max_ulp": int(ulps.max()), "max_err_over_scale": float((err / np.maximum(sc, 1e-300)).max()),
            "exact_lanes": exact, "lanes": int(r.size)}

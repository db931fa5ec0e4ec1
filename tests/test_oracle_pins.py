"""Pins for the CPU oracle: values the pages print, closed forms, library
routines, invariants and brute force. None of these retypes the oracle's own
formula; each is chosen so that a dropped term, a wrong sign, an off-by-one
mask index or a swapped operand in oracle.c fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from conftest import golden, golden_dict


# ---------------------------------------------------------------------------
# Printed worked examples
# ---------------------------------------------------------------------------

def test_worked_fp16_example_stable_values():
    g = golden_dict("worked_fp16_example.txt")
    x = np.array([g["x"][0]], dtype=np.float32)
    p, cls, st = oracle.softmax_rows(x, "f32")
    assert st[0] == oracle.ROW_OK and (cls == oracle.LANE_NUMERIC).all()
    printed, tol = g["p"]
    for i in range(3):
        assert abs(p[0, i] - printed[i]) <= tol[i]
    assert abs(p[0, 3] - g["p3_true"][0][0]) <= g["p3_true"][1][0]
    m, l = oracle.chunk_stats(x, "f32", 4)
    assert m[0, 0] == 20.0
    assert abs(l[0, 0] - g["sum"][0][0]) <= g["sum"][1][0]
    # the printed exponentials are p * sum
    ex, tol = g["exp"]
    for i in range(4):
        assert abs(p[0, i] * l[0, 0] - ex[i]) <= tol[i]


def test_worked_fp16_example_naive_overflows():
    """The unshifted formula (a failure mode, not part of the oracle) turns the
    row into NaN in fp16, as printed; the oracle stays finite."""
    g = golden_dict("worked_fp16_example.txt")
    x16 = np.array(g["x"][0], dtype=np.float16)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x16)
        naive = e / e.sum(dtype=np.float16)
    # every logit that overflows becomes inf/inf = NaN; the page prints NaN for
    # all four lanes, while IEEE gives exp(-5)/inf = 0 for the last one
    assert np.isinf(e[:3]).all() and np.isnan(naive[:3]).all() and naive[3] == 0
    assert abs(math.exp(20.0) - g["naive_exp20"][0][0]) <= g["naive_exp20"][1][0]
    assert float(np.finfo(np.float16).max) == g["fp16_max"][0][0]
    bits = W.f64_to_f16_bits(np.array(g["x"][0]))
    p, _, st = oracle.softmax_rows(bits[None, :], "f16")
    assert st[0] == oracle.ROW_OK and np.isfinite(p).all()


def test_merge_worked_example():
    g = golden_dict("merge_worked_example.txt")
    ma, la, mb, lb = (g[k][0][0] for k in ("m_a", "l_a", "m_b", "l_b"))
    m, l = oracle.merge(ma, la, mb, lb)
    assert m == g["m_merged"][0][0]
    assert abs(l - g["l_merged"][0][0]) <= g["l_merged"][1][0]
    assert abs((l - lb) - g["a_rescaled"][0][0]) <= g["a_rescaled"][1][0]
    assert abs(l - g["l_direct_wrong"][0][0]) > 1.0  # the direct add is caught
    # mb < m: the larger side keeps its sum unchanged (factor exactly 1)
    m2, l2 = oracle.merge(mb, lb, ma, la)
    assert m2 == mb and l2 == l
    m3, l3 = oracle.merge(12.0, 1.3, 12.0 - 1e9, 5.0)
    assert m3 == 12.0 and l3 == 1.3


def test_binary_lab_family():
    for x, w, printed, tol in golden("binary_lab.txt"):
        z = float(w) * float(x) - 0.5
        p, _, _ = oracle.softmax_rows(np.array([[0.0, z]], dtype=np.float32), "f32")
        sigma = 1.0 / (1.0 + math.exp(-np.float32(z)))  # logistic closed form
        assert abs(p[0, 1] - sigma) <= 1e-15
        assert abs(p[0, 0] - (1.0 - sigma)) <= 1e-15
        assert abs(p[0, 1] - float(printed)) <= float(tol)


def test_large_logits_row_finite_and_shift_exact():
    rows = {r[0]: [float(v) for v in r[1].split(",")] for r in golden("large_logits_row.txt")}
    big = np.array([rows["row"]], dtype=np.float32)
    small = np.array([rows["shifted"]], dtype=np.float32)
    pb, _, st = oracle.softmax_rows(big, "f32")
    ps, _, _ = oracle.softmax_rows(small, "f32")
    assert st[0] == oracle.ROW_OK and np.isfinite(pb).all()
    assert (pb == ps).all()  # an integer shift is exact in double
    ref = torch.softmax(torch.tensor(rows["row"], dtype=torch.float32), 0).double().numpy()
    assert np.allclose(pb[0], ref, rtol=2e-7, atol=0)
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float32(1000.0)))


def test_trace_row_matches_prefix_definition():
    meta = {r[0]: r[1] for r in golden("trace_row.txt")}
    x = [float(v) for v in meta["row"].split(",")]
    m, d = oracle.online_elementwise(x)
    for i in range(len(x)):
        mi = max(x[: i + 1])
        di = math.fsum(math.exp(v - mi) for v in x[: i + 1])
        assert m[i] == mi
        assert abs(d[i] - di) <= 1e-15 * di
    # the wrong version agrees until the maximum first moves, and is far off
    # once 12 arrives
    k = int(meta["max_change_index"])
    mw, dw = oracle.online_no_rescale(x)
    assert dw[0] == d[0] and dw[1] != d[1]
    assert abs(dw[k] - d[k]) > 1.0


def test_visualization_row_tiled_equals_three_pass():
    """The row drawn in "Kernel visualization: online softmax" (tile of 4)."""
    x = [3.0, 1.0, 4.0, 2.0, 8.0, 5.0, 7.0, 6.0]
    m, d = oracle.online_tiled(x, 4)
    assert list(m) == [4.0, 8.0]
    assert abs(d[0] - math.fsum(math.exp(v - 4.0) for v in x[:4])) <= 1e-15
    full = math.fsum(math.exp(v - 8.0) for v in x)
    assert abs(d[1] - full) <= 2e-15 * full
    ms, ls = oracle.chunk_stats(np.array([x], dtype=np.float32), "f32", 8)
    assert ms[0, 0] == 8.0 and abs(ls[0, 0] - d[1]) <= 2e-15 * full


# ---------------------------------------------------------------------------
# Library routines and closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", W.DTYPES)
def test_matches_torch_softmax_float64(dtype):
    rng = np.random.default_rng(11)
    for rows, cols, scale in ((7, 33, 3.0), (5, 300, 20.0), (3, 1025, 40.0)):
        x = W.to_format(scale * rng.standard_normal((rows, cols)), dtype)
        p, cls, st = oracle.softmax_rows(x, dtype)
        ref = torch.softmax(torch.from_numpy(W.to_float(x, dtype).astype(np.float64)), dim=1).numpy()
        assert (st == 0).all()
        assert np.allclose(p, ref, rtol=1e-13, atol=1e-300)


def test_matches_high_precision_on_sampled_rows():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 40
    rng = np.random.default_rng(12)
    for scale in (1.0, 30.0):
        x = (scale * rng.standard_normal(200)).astype(np.float32)
        p, _, _ = oracle.softmax_rows(x[None, :], "f32")
        xs = [mpmath.mpf(float(v)) for v in x]
        den = mpmath.fsum(mpmath.exp(v) for v in xs)
        for j in range(0, 200, 7):
            ref = float(mpmath.exp(xs[j]) / den)
            assert abs(p[0, j] - ref) <= 4 * np.spacing(ref) + 1e-300


def test_log_softmax_matches_library():
    from scipy.special import logsumexp

    rng = np.random.default_rng(13)
    x = (10 * rng.standard_normal((6, 77))).astype(np.float32)
    lse, logp = oracle.log_softmax_rows(x, "f32")
    assert np.allclose(lse, logsumexp(x.astype(np.float64), axis=1), rtol=1e-14)
    ref = torch.log_softmax(torch.from_numpy(x.astype(np.float64)), 1).numpy()
    assert np.allclose(logp, ref, rtol=1e-13, atol=1e-13)
    # constant row of n: LSE = c + log n
    c = np.full((1, 64), 3.0, dtype=np.float32)
    lse, _ = oracle.log_softmax_rows(c, "f32")
    assert abs(lse[0] - (3.0 + math.log(64))) <= 1e-15 * 8


def test_softmax_backward_matches_library():
    rng = np.random.default_rng(14)
    x = torch.from_numpy(3 * rng.standard_normal((5, 40)))
    p64 = torch.softmax(x, 1)
    p = W.to_format(p64.numpy(), "f32")
    g = W.to_format(rng.standard_normal((5, 40)), "f32")
    dx = oracle.softmax_backward_rows(p, g, "f32")
    pt = torch.from_numpy(p.astype(np.float64))
    gt = torch.from_numpy(g.astype(np.float64))
    ref = torch.ops.aten._softmax_backward_data(gt, pt, 1, torch.float64).numpy()
    assert np.allclose(dx, ref, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# Encoding / decoding of the element formats
# ---------------------------------------------------------------------------

def test_decode_every_f16_and_bf16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    d16 = oracle.decode(bits, "f16")
    ref16 = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(d16), np.isnan(ref16))
    ok = ~np.isnan(ref16)
    assert np.array_equal(d16[ok], ref16[ok])
    db = oracle.decode(bits, "bf16")
    with np.errstate(invalid="ignore"):
        refb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(db), np.isnan(refb))
    ok = ~np.isnan(refb)
    assert np.array_equal(db[ok], refb[ok])


def _round_cases(rng, lo_exp, hi_exp, table):
    """Random doubles, the exact table values, and exact midpoints between
    neighbours (ties), across normal and subnormal ranges."""
    r = np.exp2(rng.uniform(lo_exp, hi_exp, 4000)) * rng.uniform(1, 2, 4000)
    mids = (table[:-1] + table[1:]) / 2.0  # exact in double
    pick = rng.choice(len(mids), 4000)
    return np.concatenate([r, table[rng.choice(len(table), 2000)], mids[pick],
                           np.nextafter(mids[pick], 0), np.nextafter(mids[pick], np.inf)])


def _nearest_even(v, table, table_bits):
    """Brute force: the nearest table entry, ties to the even bit pattern."""
    i = np.searchsorted(table, v)
    out = np.empty(len(v), dtype=np.int64)
    for k, (vi, ii) in enumerate(zip(v, i)):
        cands = [c for c in (ii - 1, ii) if 0 <= c < len(table)]
        dist = [abs(table[c] - vi) for c in cands]
        best = min(dist)
        tied = [c for c, dd in zip(cands, dist) if dd == best]
        c = tied[0] if len(tied) == 1 else [c for c in tied if table_bits[c] % 2 == 0][0]
        out[k] = table_bits[c]
    return out


def test_round_f16_matches_numpy_and_brute_force():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. max finite
    table = bits.view(np.float16).astype(np.float64)
    rng = np.random.default_rng(15)
    v = _round_cases(rng, -26, 15.9, table)
    v = v[v <= 65504.0]
    got = np.array([oracle.round_f16_bits(t) for t in v])
    assert np.array_equal(got, v.astype(np.float16).view(np.uint16))
    assert np.array_equal(got[:600], _nearest_even(v[:600], table, bits.astype(np.int64)))
    assert oracle.round_f16_bits(65519.99) == 0x7BFF and oracle.round_f16_bits(65520.0) == 0x7C00
    assert oracle.round_f16_bits(float("nan")) == 0x7E00
    assert oracle.round_f16_bits(-2.0 ** -25) == 0x8000  # tie to even zero, sign kept
    assert oracle.round_f16_bits(2.0 ** -25 * 1.0000001) == 0x0001


def test_round_bf16_brute_force():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    table = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(16)
    v = _round_cases(rng, -135, 127.5, table)
    v = v[v <= table[-1]]
    got = np.array([oracle.round_bf16_bits(t) for t in v])
    sel = rng.choice(len(v), 3000, replace=False)
    assert np.array_equal(got[sel], _nearest_even(v[sel], table, bits.astype(np.int64)))
    assert oracle.round_bf16_bits(float("nan")) == 0x7FC0
    mid = (2.0 - 2.0 ** -8) * 2.0 ** 127  # halfway between the largest finite and 2^128
    assert oracle.round_bf16_bits(mid) == 0x7F80  # tie goes to the even pattern: inf
    assert oracle.round_bf16_bits(np.nextafter(mid, 0)) == 0x7F7F
    assert oracle.round_bf16_bits(2.0 ** -134) == 0x0000  # tie to even zero
    assert oracle.round_bf16_bits(2.0 ** -134 * 1.5) == 0x0001


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(17)
    v = np.concatenate([np.exp2(rng.uniform(-152, 127, 5000)), rng.standard_normal(1000)])
    got = np.array([oracle.round_f32_bits(t) for t in v], dtype=np.uint32)
    assert np.array_equal(got, v.astype(np.float32).view(np.uint32))


def test_worked_example_encodings():
    """The stable row rounded once into fp16 and bf16 (nearest-even of the
    double value); numpy's double->half conversion is the library check."""
    x = np.array([[20.0, 18.0, 17.0, -5.0]], dtype=np.float32)
    p, _, _ = oracle.softmax_rows(x, "f32")
    assert np.array_equal(oracle.encode(p, "f16").ravel(), p.ravel().astype(np.float16).view(np.uint16))
    assert list(oracle.encode(p, "f16").ravel()) == [0x3AC0, 0x2F4F, 0x2961, 0x0000]


# ---------------------------------------------------------------------------
# Invariants and exact special cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", W.DTYPES)
def test_invariants_random_rows(dtype):
    rng = np.random.default_rng(18)
    x = W.to_format(25 * rng.standard_normal((40, 129)), dtype)
    valid = rng.integers(0, 130, 40).astype(np.int32)
    mask = W.MaskSpec("valid_len", valid_len=valid)
    p, cls, st = oracle.softmax_rows(x, dtype, mask)
    m, l = oracle.chunk_stats(x, dtype, 129, mask)
    for r in range(40):
        n = int(valid[r])
        if n == 0:
            assert st[r] == oracle.ROW_EMPTY and (p[r] == 0).all()
            continue
        assert 1.0 <= l[r, 0] <= n
        assert (p[r] >= 0).all() and (p[r] <= 1).all()
        assert abs(p[r].sum() - 1.0) <= 1e-14 * n
        assert p[r, :n].max() >= 1.0 / n
        assert (p[r, n:] == 0).all() and (cls[r, n:] == oracle.LANE_ZERO).all()
        assert m[r, 0] == W.to_float(x, dtype)[r, :n].max()


def test_exact_special_cases():
    for dtype in W.DTYPES:
        # one valid lane -> exactly 1
        x = W.to_format(np.array([[5.0, -3.0, 2.0]]), dtype)
        p, _, _ = oracle.softmax_rows(x, dtype, W.MaskSpec("valid_len", valid_len=np.array([1], np.int32)))
        assert p[0, 0] == 1.0 and (p[0, 1:] == 0).all()
        # constant row of 2^k -> exactly 2^-k, in every format after rounding
        for k in (0, 3, 8, 12):
            x = W.to_format(np.full((1, 1 << k), 1.5), dtype)
            p, _, _ = oracle.softmax_rows(x, dtype)
            assert (p == 2.0 ** -k).all()
            enc = oracle.encode(p, dtype)
            assert (W.to_float(enc, dtype) == np.float32(2.0 ** -k)).all()
        # two equal maxima, the rest -inf -> 0.5, 0.5
        x = W.to_format(np.array([[-np.inf, 7.0, -np.inf, 7.0]]), dtype)
        p, cls, _ = oracle.softmax_rows(x, dtype)
        assert list(p[0]) == [0.0, 0.5, 0.0, 0.5]
        assert list(cls[0]) == [oracle.LANE_ZERO, 0, oracle.LANE_ZERO, 0]


def test_bf16_accumulator_would_stagnate():
    """"Softmax numerics architecture", section on the fp32 accumulator: in
    bf16 a running sum stalls at 256. The oracle's sum does not: a constant
    row of 4096 gives exactly 2^-12, where a stalled sum would give 2^-8."""
    acc = np.float32(0)
    for _ in range(4096):
        acc = W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.array([acc + np.float32(1.0)])))[0]
    assert acc == 256.0
    x = W.to_format(np.zeros((1, 4096)), "bf16")
    p, _, _ = oracle.softmax_rows(x, "bf16")
    assert (p == 2.0 ** -12).all()


def test_shift_invariance():
    rng = np.random.default_rng(19)
    xi = rng.integers(-20, 20, (6, 50)).astype(np.float32)
    p0, _, _ = oracle.softmax_rows(xi, "f32")
    for c in (-7.0, 13.0, 100.0):
        p1, _, _ = oracle.softmax_rows(xi + np.float32(c), "f32")
        assert np.array_equal(p0, p1)
    # non-integer logits on a 2^-10 grid, shifted by a non-integer on the
    # same grid: every shifted value is exact, so the output is bit-identical
    xf = (np.round(5 * rng.standard_normal((6, 50)) * 1024) / 1024).astype(np.float32)
    p0, _, _ = oracle.softmax_rows(xf, "f32")
    for c in (307 / 1024, -4099 / 1024):
        p1, _, _ = oracle.softmax_rows((xf.astype(np.float64) + c).astype(np.float32), "f32")
        assert np.array_equal(p0, p1)
    # and against a shifted row the library computes: same values to 1e-15
    ref = torch.softmax(torch.from_numpy(xf.astype(np.float64) + 1e3), 1).numpy()
    assert np.allclose(p0, ref, rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# Mask contract and policy
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", W.DTYPES)
def test_masks_agree_with_explicit_keep(dtype):
    rng = np.random.default_rng(20)
    rows, cols = 24, 21
    x = W.to_format(6 * rng.standard_normal((rows, cols)), dtype)
    period, off = 8, 2
    causal = W.MaskSpec("causal", causal_period=period, causal_offset=off)
    tri = np.tril(np.ones((period, cols), dtype=np.uint8), k=off)  # row i keeps 0..i+off
    keep = np.tile(tri, (rows // period, 1))
    pc, cc, _ = oracle.softmax_rows(x, dtype, causal)
    pk, ck, _ = oracle.softmax_rows(x, dtype, W.MaskSpec("keep", keep=keep))
    assert np.array_equal(pc, pk) and np.array_equal(cc, ck)
    valid = rng.integers(-3, cols + 4, rows).astype(np.int32)  # out of range clamps
    keep2 = (np.arange(cols)[None, :] < valid[:, None]).astype(np.uint8)
    pv, cv, _ = oracle.softmax_rows(x, dtype, W.MaskSpec("valid_len", valid_len=valid))
    pk2, ck2, _ = oracle.softmax_rows(x, dtype, W.MaskSpec("keep", keep=keep2))
    assert np.array_equal(pv, pk2) and np.array_equal(cv, ck2)


def test_masked_row_equals_truncated_row():
    rng = np.random.default_rng(21)
    x = (4 * rng.standard_normal((1, 30))).astype(np.float32)
    for n in (1, 7, 29, 30):
        pm, _, _ = oracle.softmax_rows(x, "f32", W.MaskSpec("valid_len", valid_len=np.array([n], np.int32)))
        pt, _, _ = oracle.softmax_rows(np.ascontiguousarray(x[:, :n]), "f32")
        assert np.array_equal(pm[0, :n], pt[0]) and (pm[0, n:] == 0).all()


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_policy_rows(dtype):
    cols = 9
    base = W.to_format(np.linspace(-3, 3, cols)[None, :].repeat(6, 0), dtype)
    x = base.copy()
    W.set_bits(x, 0, 4, dtype, W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype])
    W.set_bits(x, 1, 2, dtype, W.NEG_SNAN[dtype])
    W.set_bits(x, 2, 8, dtype, W.QNAN[dtype])  # masked lane below
    W.set_bits(x, 3, 8, dtype, W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype])
    for j in range(5):
        W.set_bits(x, 4, j, dtype, W.NEG_INF[dtype].view(np.uint32) if dtype == "f32" else W.NEG_INF[dtype])
    valid = np.array([9, 9, 8, 8, 5, 0], dtype=np.int32)
    p, cls, st = oracle.softmax_rows(x, dtype, W.MaskSpec("valid_len", valid_len=valid))
    assert list(st) == [oracle.ROW_POISON, oracle.ROW_POISON, 0, 0, oracle.ROW_EMPTY, oracle.ROW_EMPTY]
    assert np.isnan(p[:2]).all() and (cls[:2] == oracle.LANE_NAN).all()
    ref, _, _ = oracle.softmax_rows(base, dtype, W.MaskSpec("valid_len", valid_len=valid))
    assert np.array_equal(p[2:4], ref[2:4])  # masked NaN / +inf are ignored
    assert (p[4:] == 0).all() and (cls[4:] == oracle.LANE_ZERO).all()
    enc = oracle.encode(p, dtype)
    nanbits = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}[dtype]
    raw = enc.view(np.uint32) if dtype == "f32" else enc
    assert (raw[:2] == nanbits).all() and (raw[4:] == 0).all()
    # torch agrees on a row holding +inf (NaN row) once masks are -inf fills
    t = torch.softmax(torch.tensor([1.0, float("inf"), 2.0]), 0)
    assert torch.isnan(t).all()


def test_neg_inf_lane_equals_masked_lane():
    rng = np.random.default_rng(22)
    x = (3 * rng.standard_normal((1, 12))).astype(np.float32)
    x2 = x.copy()
    x2[0, 5] = -np.inf
    keep = np.ones((1, 12), np.uint8)
    keep[0, 5] = 0
    a, ca, _ = oracle.softmax_rows(x2, "f32")
    b, cb, _ = oracle.softmax_rows(x, "f32", W.MaskSpec("keep", keep=keep))
    assert np.array_equal(a, b) and np.array_equal(ca, cb)


def test_empty_shapes():
    p, cls, st = oracle.softmax_rows(np.zeros((3, 0), np.float32), "f32")
    assert p.shape == (3, 0) and list(st) == [oracle.ROW_EMPTY] * 3
    p, cls, st = oracle.softmax_rows(np.zeros((0, 5), np.float32), "f32")
    assert p.shape == (0, 5)


# ---------------------------------------------------------------------------
# Online recurrences and merges against the three-pass definition
# ---------------------------------------------------------------------------

VALUE_SET = (-np.inf, -30.0, -1.0, 0.0, 0.5, 3.0, 88.0, 1000.0)


# The oracle's summaries and merges are pure functions of their inputs, and
# the brute force below evaluates the same segments and the same merges over
# and over (rows are drawn from a set of eight values), so both are cached:
# each distinct call reaches the oracle once, and the exhaustive tiers fit
# the default run. Keys are the exact float bit patterns (NaN included).
_SEG_CACHE = {}
_MERGE_CACHE = {}


def _segment_stats(row, lo, hi):
    key = tuple(row[lo:hi])
    r = _SEG_CACHE.get(key)
    if r is None:
        seg = np.ascontiguousarray(np.array([row[lo:hi]], dtype=np.float32))
        m, l = oracle.chunk_stats(seg, "f32", hi - lo)
        r = _SEG_CACHE[key] = (m[0, 0], l[0, 0])
    return r


def _merge(ma, la, mb, lb):
    key = np.array([ma, la, mb, lb], dtype=np.float64).tobytes()
    r = _MERGE_CACHE.get(key)
    if r is None:
        r = _MERGE_CACHE[key] = oracle.merge(ma, la, mb, lb)
    return r


def _fold(stats):
    m, l = -np.inf, 0.0
    for sm, sl in stats:
        m, l = _merge(m, l, sm, sl)
    return m, l


def _tree_shapes(items):
    """All binary bracketings of an ordered list of summaries."""
    if len(items) == 1:
        yield items[0]
        return
    for k in range(1, len(items)):
        for a in _tree_shapes(items[:k]):
            for b in _tree_shapes(items[k:]):
                yield _merge(*a, *b)


def _brute_force_rows(n, rows):
    """For every row: the chunk summary of the whole row against the
    definition, then every contiguous split, every merge order of up to four
    chunks as a left fold (one order beyond), and every bracketing of the
    chunks, each held to the three-pass summary. Returns the folds checked."""
    checked = 0
    for row in rows:
        x = np.array([row], dtype=np.float32)
        M, L = oracle.chunk_stats(x, "f32", n)
        M, L = M[0, 0], L[0, 0]
        finite = [v for v in row if v != -np.inf]
        if not finite:
            assert (M, L) == (-np.inf, 0.0)
        else:
            assert M == max(finite) and 1.0 <= L <= len(finite)
        for cuts in itertools.product((0, 1), repeat=n - 1):
            bounds = [0] + [i + 1 for i, c in enumerate(cuts) if c] + [n]
            stats = [_segment_stats(row, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
            orders = itertools.permutations(stats) if len(stats) <= 4 else [stats]
            for perm in orders:
                m, l = _fold(perm)
                assert m == M
                assert abs(l - L) <= 8 * n * 2.0 ** -53 * max(L, 1.0)
                checked += 1
            for m, l in _tree_shapes(stats):
                assert m == M and abs(l - L) <= 8 * n * 2.0 ** -53 * max(L, 1.0)
    return checked


def test_brute_force_every_split_and_merge_order():
    checked = 0
    for n in range(1, 5):
        checked += _brute_force_rows(n, itertools.product(VALUE_SET, repeat=n))
    assert checked > 100000


def test_brute_force_rows_of_five_exhaustive():
    """Every row of five values from the set (32768 rows, every contiguous
    split, every merge order and bracketing: over a million folds)."""
    assert _brute_force_rows(5, itertools.product(VALUE_SET, repeat=5)) > 1000000


@pytest.mark.slow
def test_brute_force_rows_of_six_exhaustive():
    """The slow tier (--runslow): every row of six values from the set
    (262144 rows, every contiguous split, every merge order of up to four
    chunks and every bracketing)."""
    assert _brute_force_rows(6, itertools.product(VALUE_SET, repeat=6)) > 10000000


def test_split_path_oracle_equals_three_pass():
    rng = np.random.default_rng(23)
    for dtype in W.DTYPES:
        x = W.to_format(10 * rng.standard_normal((9, 1000)), dtype)
        valid = rng.integers(0, 1001, 9).astype(np.int32)
        mask = W.MaskSpec("valid_len", valid_len=valid)
        p, cls, st = oracle.softmax_rows(x, dtype, mask)
        for chunk in (1, 37, 128, 999, 1000, 4096):
            m, l = oracle.chunk_stats(x, dtype, chunk, mask)
            q, cq, sq = oracle.merge_normalize(x, dtype, m, l, mask)
            assert np.array_equal(cls, cq) and np.array_equal(st, sq)
            assert np.allclose(q, p, rtol=1e-13, atol=0)


def test_stress_online_vs_three_pass_and_negative_control():
    """1,000 random rows with occasional logits in [50, 100] ("Online stable
    softmax", trace exercise)."""
    rng = np.random.default_rng(24)
    wrong = 0
    max_rel = 0.0
    for _ in range(1000):
        n = int(rng.integers(2, 64))
        x = rng.standard_normal(n) * 3
        hot = rng.random(n) < 0.1
        x[hot] = rng.uniform(50, 100, hot.sum())
        x32 = x.astype(np.float32)
        M, L = oracle.chunk_stats(x32[None, :], "f32", n)
        m, d = oracle.online_elementwise(x32.astype(np.float64))
        mt, dt = oracle.online_tiled(x32.astype(np.float64), 5)
        assert m[-1] == M[0, 0] and mt[-1] == M[0, 0]
        max_rel = max(max_rel, abs(d[-1] - L[0, 0]) / L[0, 0], abs(dt[-1] - L[0, 0]) / L[0, 0])
        _, dw = oracle.online_no_rescale(x32.astype(np.float64))
        if abs(dw[-1] - L[0, 0]) > 1e-6 * L[0, 0]:
            wrong += 1
    assert max_rel <= 1e-13
    assert wrong > 500  # the no-rescale version is caught on most rows


def test_workload_generators_shapes():
    w = W.small_rows()
    assert (w.rows, w.cols, w.dtype) == (64, 1024, "f32")
    w = W.masked_rows(rows=64)
    assert w.mask.kind == "valid_len" and w.mask.valid_len.min() >= 0 and w.mask.valid_len.max() <= 512
    w = W.causal_scores(groups=2, n=64, head_dim=16)
    assert w.rows == 128 and all(len(v) == 2 for v in w.special_rows.values())
    p, cls, st = oracle.softmax_rows(w.x, "bf16", w.mask)
    for name in ("pos_inf_valid", "nan_valid"):
        assert (st[w.special_rows[name]] == oracle.ROW_POISON).all()
    assert (st[w.special_rows["all_neg_inf"]] == oracle.ROW_EMPTY).all()
    for name in ("nan_masked", "pos_inf_masked"):
        assert (st[w.special_rows[name]] == oracle.ROW_OK).all()


def test_softmax_backward_closed_forms():
    """"Softmax numerics architecture", Jacobian section: J = diag(p) - p p^T.
    A one-hot g picks a column of J in closed form, and a constant g (the
    gradient of a shift) gives zero, since the rows of J sum to 0."""
    rng = np.random.default_rng(25)
    x = (4 * rng.standard_normal((3, 17))).astype(np.float64)
    p = np.exp(x - x.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    p32 = p.astype(np.float32)
    pd = p32.astype(np.float64)
    for t in (0, 5, 16):
        g = np.zeros((3, 17), dtype=np.float32)
        g[:, t] = 1.0
        dx = oracle.softmax_backward_rows(p32, g, "f32")
        col = -pd * pd[:, t:t + 1]
        col[:, t] += pd[:, t]
        assert np.allclose(dx, col, rtol=1e-15, atol=1e-18)
    g = np.full((3, 17), 2.5, dtype=np.float32)
    dx = oracle.softmax_backward_rows(p32, g, "f32")
    assert np.abs(dx).max() <= 2.5 * 17 * 2.0 ** -23  # sum(p) is 1 to fp32 rounding


def test_cross_entropy_closed_forms_and_library():
    """CE = LSE - x_t ("Softmax numerics architecture", log-sum-exp section).
    The two-logit family of the network lab gives CE([0, z], 1) = -log sigma(z)
    = log(1 + e^-z), and the fused gradient is p - onehot ("Jacobian" section);
    torch's cross_entropy in float64 is the library check."""
    for z in (0.5, 2.5, -7.0, 30.0):
        x = np.array([[0.0, z]], dtype=np.float32)
        loss, dx = oracle.cross_entropy_rows(x, "f32", np.array([1], np.int32))
        zz = float(np.float32(z))
        assert abs(loss[0] - math.log1p(math.exp(-zz))) <= 1e-15 * max(1.0, loss[0])
        s = 1.0 / (1.0 + math.exp(-zz))
        assert abs(dx[0, 0] - (1.0 - s)) <= 1e-15
        # the target lane, sigma(z) - 1 = -1 / (1 + e^z), to full relative precision
        exact = -1.0 / (1.0 + math.exp(zz))
        assert abs(dx[0, 1] - exact) <= 4e-16 * abs(exact)
    rng = np.random.default_rng(26)
    x = (6 * rng.standard_normal((20, 50))).astype(np.float32)
    t = rng.integers(0, 50, 20).astype(np.int32)
    loss, dx = oracle.cross_entropy_rows(x, "f32", t)
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
    ref = torch.nn.functional.cross_entropy(xt, torch.from_numpy(t.astype(np.int64)), reduction="none")
    ref.sum().backward()
    assert np.allclose(loss, ref.detach().numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_cross_entropy_policy():
    x = np.array([[1.0, 2.0, 3.0, 4.0]] * 5, dtype=np.float32)
    x[2, 1] = np.nan
    valid = np.array([4, 4, 4, 2, 0], dtype=np.int32)
    t = np.array([-1, 9, 0, 3, 1], dtype=np.int32)
    loss, dx = oracle.cross_entropy_rows(x, "f32", t, W.MaskSpec("valid_len", valid_len=valid))
    assert loss[0] == 0 and (dx[0] == 0).all() and loss[1] == 0 and (dx[1] == 0).all()  # ignored
    assert np.isnan(loss[2]) and np.isnan(dx[2]).all()  # poisoned
    assert loss[3] == np.inf and dx[3, 3] == -1.0 and abs(dx[3].sum() + 0.0) <= 1e-15  # masked target
    assert loss[4] == np.inf and list(dx[4]) == [0.0, -1.0, 0.0, 0.0]  # empty row


# ---------------------------------------------------------------------------
# The CPU-baseline routine: the same rows, encoded, over host threads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", W.DTYPES)
def test_cpu_baseline_routine_equals_rows_then_encode(dtype):
    """oracle_softmax_rows_encode_mt (what the benchmark's CPU baseline times)
    must write exactly the bytes of the three-pass rows rounded by
    oracle_encode, whatever the thread count (including counts that do not
    divide the rows, one thread per row, and more threads than rows), under
    every mask kind and with policy rows present. The output buffer starts
    filled with a byte pattern that is no encoding of any result, so a row
    the routine skipped, or wrote at another row's offset, cannot match."""
    rng = np.random.default_rng(78)
    rows, cols = 37, 203
    x = W.to_format(12.0 * rng.standard_normal((rows, cols)), dtype)
    inf = W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype]
    W.set_bits(x, 3, 10, dtype, inf)                   # +inf in a (mostly) valid lane
    W.set_bits(x, 11, 0, dtype, W.NEG_SNAN[dtype])     # NaN in lane 0 (valid under every mask)
    x[20] = W.to_format(np.full(cols, -np.inf), dtype)  # every lane -inf
    valid = rng.integers(0, cols + 1, rows).astype(np.int32)
    valid[5] = 0
    keep = (rng.random((rows, cols)) < 0.3).astype(np.uint8)
    keep[7] = 0
    keep[3, 10] = keep[11, 0] = 1  # the poisoned lanes stay valid
    masks = [W.MaskSpec(), W.MaskSpec("valid_len", valid_len=valid),
             W.MaskSpec("causal", causal_period=13, causal_offset=-2), W.MaskSpec("keep", keep=keep)]
    for mask in masks:
        p, cls, st = oracle.softmax_rows(x, dtype, mask)
        want = oracle.encode(p, dtype).view(np.uint8)
        assert (st == oracle.ROW_POISON).any() and (st == oracle.ROW_EMPTY).any(), mask.kind
        for threads in (1, 2, 3, 16, rows, rows + 5):
            out = np.empty_like(x)
            out.view(np.uint8)[...] = 0xA5
            y, dt = oracle.softmax_rows_encode_mt(x, dtype, mask, threads, out=out)
            assert y is out and dt >= 0.0
            assert np.array_equal(y.view(np.uint8), want), (mask.kind, threads)

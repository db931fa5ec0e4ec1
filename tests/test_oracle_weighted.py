"""Pins for the oracle's softmax-weighted value sums and their online states
("Online stable softmax", sections on the weighted-value numerator, the
worked merge and the reference summary; "Softmax numerics architecture",
tiled attention). CPU only. None of these checks restates the oracle's own
formula: each compares it with a value the pages print, a special case that
reduces to an already pinned routine or a closed form, a library routine,
or brute force over every split and merge order."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from conftest import golden, golden_dict


def _sv(rng, rows, cols, d, groups, dtype, scale=3.0):
    s = W.to_format(scale * rng.standard_normal((rows, cols)), dtype)
    v = W.to_format(rng.standard_normal((groups, cols, d)), dtype)
    return s, v


def test_binary_lab_family_as_expected_value():
    # V = [0, 1] turns the weighted sum into the second probability, sigma(z)
    for x, w, printed, tol in golden("binary_lab.txt"):
        z = float(w) * float(x) - 0.5
        s = np.array([[0.0, z]], dtype=np.float32)
        v = np.array([[[0.0], [1.0]]], dtype=np.float32)
        out, st = oracle.softmax_weighted_rows(s, v, "f32", 1)
        assert abs(out[0, 0] - float(printed)) <= float(tol)
        assert abs(out[0, 0] - 1.0 / (1.0 + math.exp(-float(np.float32(z))))) <= 1e-15


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_one_hot_values_give_the_softmax(dtype):
    rng = np.random.default_rng(40)
    rows, cols = 6, 37
    s = W.to_format(4 * rng.standard_normal((rows, cols)), dtype)
    eye = W.to_format(np.eye(cols)[None].repeat(2, axis=0), dtype)
    valid = np.array([37, 0, 5, 1, 20, 37], dtype=np.int32)
    mask = W.MaskSpec("valid_len", valid_len=valid)
    out, st = oracle.softmax_weighted_rows(s, eye, dtype, 3, mask)
    p, cls, st2 = oracle.softmax_rows(s, dtype, mask)
    assert np.array_equal(st, st2)
    assert np.array_equal(out, p)  # one nonzero term per component: bit-equal


def test_constant_values_and_linearity():
    rng = np.random.default_rng(41)
    rows, cols, d = 8, 50, 5
    s, _ = _sv(rng, rows, cols, d, 2, "f32")
    # small integers, so a * v1 + b * v2 below is exact in float32
    v1 = rng.integers(-8, 9, (2, cols, d)).astype(np.float32)
    c = rng.standard_normal(d).astype(np.float32)
    vc = np.broadcast_to(c, (2, cols, d)).copy()
    out, st = oracle.softmax_weighted_rows(s, vc, "f32", 4)
    assert np.allclose(out, c[None].astype(np.float64), rtol=1e-14, atol=1e-15)
    # the weights are a convex combination: out = a * out(v1) + b * out(v2)
    v2 = rng.integers(-8, 9, (2, cols, d)).astype(np.float32)
    a, b = 0.75, -2.0
    o1, _ = oracle.softmax_weighted_rows(s, v1, "f32", 4)
    o2, _ = oracle.softmax_weighted_rows(s, v2, "f32", 4)
    o12, _ = oracle.softmax_weighted_rows(s, (a * v1 + b * v2).astype(np.float32), "f32", 4)
    assert np.allclose(o12, a * o1 + b * o2, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_matches_torch_softmax_matmul_float64(dtype):
    rng = np.random.default_rng(42)
    rows, cols, d, rpg = 12, 70, 9, 4
    s, v = _sv(rng, rows, cols, d, rows // rpg, dtype)
    mask = W.MaskSpec("causal", causal_period=rpg, causal_offset=60)
    out, st = oracle.softmax_weighted_rows(s, v, dtype, rpg, mask)
    sf = torch.from_numpy(W.to_float(s, dtype).astype(np.float64))
    vf = torch.from_numpy(W.to_float(v, dtype).astype(np.float64))
    r = torch.arange(rows)
    keep = torch.arange(cols)[None, :] < (r % rpg + 1 + 60)[:, None]
    p = torch.softmax(sf.masked_fill(~keep, -math.inf), dim=1)
    ref = torch.stack([p[i] @ vf[i // rpg] for i in range(rows)]).numpy()
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_merge_worked_example_with_numerators():
    g = golden_dict("merge_worked_example.txt")
    m_a, l_a, m_b, l_b = g["m_a"][0][0], g["l_a"][0][0], g["m_b"][0][0], g["l_b"][0][0]
    o_a = np.array([1.0, -2.0, 0.5])
    o_b = np.array([0.25, 3.0, -1.0])
    m, l, o = oracle.weighted_merge(m_a, l_a, o_a, m_b, l_b, o_b)
    assert m == g["m_merged"][0][0]
    assert abs(l - g["l_merged"][0][0]) <= g["l_merged"][1][0]
    # the first block's numerator takes the same factor as its sum, e^(10 - 12)
    assert np.allclose(o, math.exp(-2.0) * o_a + o_b, rtol=1e-15, atol=0)
    # the mistake the pages warn about: rescaling l but not o
    assert not np.allclose(o, o_a + o_b)
    # order does not matter; the empty state is an identity; a poisoned state poisons
    m2, l2, o2 = oracle.weighted_merge(m_b, l_b, o_b, m_a, l_a, o_a)
    assert (m2, l2) == (m, l) and np.array_equal(o2, o)
    m3, l3, o3 = oracle.weighted_merge(-math.inf, 0.0, np.zeros(3), m_a, l_a, o_a)
    assert (m3, l3) == (m_a, l_a) and np.array_equal(o3, o_a)
    m4, l4, o4 = oracle.weighted_merge(math.nan, math.nan, np.full(3, math.nan), m_a, l_a, o_a)
    assert math.isnan(m4) and math.isnan(l4) and np.isnan(o4).all()


def _segment_state(s_row, v_rows, lo, hi):
    # plain Python floats and float64 vectors (a numpy float32 scalar would
    # keep products in single precision)
    seg = [(float(s_row[j]), v_rows[j].astype(np.float64)) for j in range(lo, hi) if s_row[j] != -math.inf]
    d = v_rows.shape[1]
    if not seg:
        return -math.inf, 0.0, np.zeros(d)
    m = max(x for x, _ in seg)
    l = math.fsum(math.exp(x - m) for x, _ in seg)
    o = np.array([math.fsum(math.exp(x - m) * vv[k] for x, vv in seg) for k in range(d)])
    return m, l, o


def _fold(states, merge):
    m, l, o = -math.inf, 0.0, np.zeros_like(states[0][2])
    for st in states:
        m, l, o = merge(m, l, o, *st)
    return m, l, o


def _wrong_merge(m_a, l_a, o_a, m_b, l_b, o_b):
    # the pages' common error: the sum is rescaled when the maximum moves,
    # the numerator is not
    m, l, _ = oracle.weighted_merge(m_a, l_a, o_a, m_b, l_b, o_b)
    return m, l, o_a + o_b


def test_brute_force_every_split_and_merge_order():
    rng = np.random.default_rng(43)
    vals = [-math.inf, -30.0, -1.0, 0.0, 0.5, 3.0, 8.0]
    caught = 0
    checked = 0
    for n in (1, 2, 3, 4):
        for row in itertools.product(vals, repeat=n):
            if all(x == -math.inf for x in row):
                continue
            s = np.array([row], dtype=np.float32)
            v = rng.integers(-3, 4, size=(1, n, 2)).astype(np.float32)
            want, st = oracle.softmax_weighted_rows(s, v, "f32", 1)
            for cuts in itertools.product([0, 1], repeat=n - 1):
                bounds = [0] + [i + 1 for i, c in enumerate(cuts) if c] + [n]
                states = [_segment_state(s[0], v[0], a, b) for a, b in zip(bounds, bounds[1:])]
                for perm in itertools.permutations(states):
                    m, l, o = _fold(list(perm), oracle.weighted_merge)
                    assert np.allclose(o / l, want[0], rtol=1e-13, atol=1e-13), (row, cuts)
                    checked += 1
                    mw, lw, ow = _fold(list(perm), _wrong_merge)
                    if not np.allclose(ow / lw, want[0], rtol=1e-9, atol=1e-9):
                        caught += 1
    assert checked > 10000
    assert caught > 1000  # the comparison detects the numerator that was not rescaled


@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
def test_chunk_states_merge_to_the_direct_result(chunk):
    rng = np.random.default_rng(44 + chunk)
    rows, cols, d, rpg = 10, 61, 4, 5
    s, v = _sv(rng, rows, cols, d, rows // rpg, "bf16")
    valid = np.array([61, 0, 1, 30, 61, 7, 61, 59, 2, 61], dtype=np.int32)
    mask = W.MaskSpec("valid_len", valid_len=valid)
    W.set_bits(s, 4, 3, "bf16", W.QNAN["bf16"])      # poisoned row
    W.set_bits(s, 6, 50, "bf16", W.NEG_INF["bf16"])  # a -inf lane
    want, st = oracle.softmax_weighted_rows(s, v, "bf16", rpg, mask)
    m, l, o = oracle.weighted_chunk_states(s, v, "bf16", rpg, chunk, mask)
    for r in range(rows):
        mm, ll, oo = -math.inf, 0.0, np.zeros(d)
        for c in range(m.shape[1]):
            mm, ll, oo = oracle.weighted_merge(mm, ll, oo, m[r, c], l[r, c], o[r, c])
        if st[r] == oracle.ROW_POISON:
            assert np.isnan(want[r]).all() and math.isnan(mm) and np.isnan(oo).all()
        elif st[r] == oracle.ROW_EMPTY:
            assert (want[r] == 0).all() and mm == -math.inf and ll == 0 and (oo == 0).all()
        else:
            assert np.allclose(oo / ll, want[r], rtol=1e-13, atol=1e-14), r


def test_policy_rows():
    s = np.array([[1.0, 2.0, np.inf], [1.0, np.nan, 0.0], [-np.inf, -np.inf, -np.inf],
                  [3.0, -np.inf, 1.0], [3.0, 5.0, 1.0]], dtype=np.float32)
    v = np.arange(5 * 3 * 2, dtype=np.float32).reshape(5, 3, 2)
    valid = np.array([3, 3, 3, 3, 1], dtype=np.int32)
    out, st = oracle.softmax_weighted_rows(s, v, "f32", 1, W.MaskSpec("valid_len", valid_len=valid))
    assert list(st) == [oracle.ROW_POISON, oracle.ROW_POISON, oracle.ROW_EMPTY, oracle.ROW_OK, oracle.ROW_OK]
    assert np.isnan(out[:2]).all() and (out[2] == 0).all()
    # a -inf lane behaves as a masked lane; a single valid lane returns its value row
    p = np.exp(np.array([3.0, 1.0]) - 3.0) / np.exp(np.array([3.0, 1.0]) - 3.0).sum()
    assert np.allclose(out[3], p[0] * v[3, 0] + p[1] * v[3, 2], rtol=1e-15)
    assert np.array_equal(out[4], v[4, 0].astype(np.float64))


@pytest.mark.parametrize("offset", [16384.0, -16384.0, 2.0 ** 20])
def test_shift_invariance_at_large_references(offset):
    # A common shift of a row's scores cancels in o / l ("Online stable
    # softmax", deriving the update: any common shift cancels). Scores on a
    # grid of 2^-3 within [-8, 8] stay exact in float32 after adding the
    # offset, so the shifted rows must give the same sums to double rounding,
    # with references far past the range where a float exponent would
    # overflow.
    rng = np.random.default_rng(43)
    rows, cols, d, rpg = 6, 90, 7, 3
    s = (np.round(rng.uniform(-8, 8, (rows, cols)) * 8) / 8).astype(np.float32)
    shifted = (s.astype(np.float64) + offset).astype(np.float32)
    assert np.array_equal(shifted.astype(np.float64) - offset, s.astype(np.float64))  # the shift is exact
    v = rng.standard_normal((rows // rpg, cols, d)).astype(np.float32)
    mask = W.MaskSpec("causal", causal_period=rpg, causal_offset=80)
    o1, st1 = oracle.softmax_weighted_rows(s, v, "f32", rpg, mask)
    o2, st2 = oracle.softmax_weighted_rows(shifted, v, "f32", rpg, mask)
    assert np.array_equal(st1, st2)
    assert np.allclose(o2, o1, rtol=1e-14, atol=1e-15)

"""ctypes wrapper around the plain double-precision CPU oracle (oracle.c).

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The product path (the
HIP library and its binding) must never import it.

Every function here only marshals numpy arrays into the C routines; the
arithmetic is all in oracle.c, which cites the page passage each routine
follows.
"""
from __future__ import annotations

import ctypes as C
import os
import time
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
DTYPE_CODE = {"f32": F32, "f16": F16, "bf16": BF16}
LANE_NUMERIC, LANE_ZERO, LANE_NAN = 0, 1, 2
ROW_OK, ROW_EMPTY, ROW_POISON = 0, 1, 2
_MASK_CODE = {"none": 0, "valid_len": 1, "causal": 2, "keep": 3}


class _Mask(C.Structure):
    _fields_ = [
        ("kind", C.c_int),
        ("valid_len", C.c_void_p),
        ("causal_period", C.c_int64),
        ("causal_offset", C.c_int64),
        ("keep", C.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b

            _b.build()
        L = C.CDLL(_LIB_PATH)
        vp, i64, i32, dp = C.c_void_p, C.c_int64, C.c_int, C.POINTER(C.c_double)
        mp = C.POINTER(_Mask)
        L.oracle_decode.argtypes = [vp, i32, i64]
        L.oracle_decode.restype = C.c_double
        L.oracle_valid_prefix.argtypes = [mp, i64, i64]
        L.oracle_valid_prefix.restype = i64
        L.oracle_softmax_rows.argtypes = [vp, i32, i64, i64, mp, i64, i64, vp, vp, vp]
        L.oracle_chunk_stats.argtypes = [vp, i32, i64, i64, mp, i64, i64, i64, vp, vp]
        L.oracle_merge.argtypes = [C.c_double] * 4 + [dp, dp]
        L.oracle_merge.restype = None
        L.oracle_merge_all.argtypes = [vp, vp, i64, dp, dp]
        L.oracle_merge_all.restype = None
        L.oracle_merge_normalize.argtypes = [vp, i32, i64, i64, mp, vp, vp, i64, i64, i64, vp, vp, vp]
        for n in ("oracle_online_elementwise", "oracle_online_no_rescale"):
            getattr(L, n).argtypes = [vp, i64, vp, vp]
            getattr(L, n).restype = None
        L.oracle_online_tiled.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_online_tiled.restype = None
        L.oracle_log_softmax_rows.argtypes = [vp, i32, i64, i64, mp, i64, i64, vp, vp]
        L.oracle_softmax_backward_rows.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp]
        L.oracle_cross_entropy_rows.argtypes = [vp, i32, i64, i64, mp, vp, i64, i64, vp, vp]
        L.oracle_softmax_weighted_rows.argtypes = [vp, vp, i32, i64, i64, i64, i64, mp, i64, i64, vp, vp]
        L.oracle_weighted_chunk_states.argtypes = [vp, vp, i32, i64, i64, i64, i64, mp, i64, i64, i64,
                                                   vp, vp, vp]
        L.oracle_weighted_merge.argtypes = [C.c_double, C.c_double, vp, C.c_double, C.c_double, vp, i64,
                                            dp, dp, vp]
        L.oracle_weighted_merge.restype = None
        L.oracle_round_f32_bits.argtypes = [C.c_double]
        L.oracle_round_f32_bits.restype = C.c_uint32
        L.oracle_round_f16_bits.argtypes = [C.c_double]
        L.oracle_round_f16_bits.restype = C.c_uint16
        L.oracle_round_bf16_bits.argtypes = [C.c_double]
        L.oracle_round_bf16_bits.restype = C.c_uint16
        L.oracle_encode.argtypes = [vp, i64, i32, vp]
        L.oracle_encode.restype = None
        L.oracle_softmax_rows_encode_mt.argtypes = [vp, vp, i32, i64, i64, mp, i32]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _mask_struct(mask, rows: int, cols: int):
    """Build the C mask struct; returns (struct, keepalive arrays)."""
    m = _Mask()
    keep = []
    if mask is None or mask.kind == "none":
        m.kind = 0
        return m, keep
    m.kind = _MASK_CODE[mask.kind]
    if mask.kind == "valid_len":
        v = np.ascontiguousarray(mask.valid_len, dtype=np.int32)
        assert v.shape == (rows,)
        m.valid_len = v.ctypes.data
        keep.append(v)
    elif mask.kind == "causal":
        m.causal_period = int(mask.causal_period)
        m.causal_offset = int(mask.causal_offset)
    else:
        k = np.ascontiguousarray(mask.keep, dtype=np.uint8)
        assert k.shape == (rows, cols)
        m.keep = k.ctypes.data
        keep.append(k)
    return m, keep


def _raw(x: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float32 if dtype == "f32" else np.uint16
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"{dtype} input must be stored as {want.__name__}, got {x.dtype}")
    return x


def softmax_rows(x: np.ndarray, dtype: str, mask=None, r0: int = 0, r1: Optional[int] = None
                 ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Three-pass reference for rows [r0, r1). Returns (p float64, lane_class uint8, row_status int32)."""
    x = _raw(x, dtype)
    rows, cols = x.shape
    r1 = rows if r1 is None else r1
    n = r1 - r0
    p = np.empty((n, cols), dtype=np.float64)
    cls = np.empty((n, cols), dtype=np.uint8)
    st = np.empty(n, dtype=np.int32)
    ms, keep = _mask_struct(mask, rows, cols)
    rc = lib().oracle_softmax_rows(_ptr(x), DTYPE_CODE[dtype], rows, cols, C.byref(ms), r0, r1,
                                   _ptr(p), _ptr(cls), _ptr(st))
    if rc != 0:
        raise ValueError("oracle_softmax_rows: bad arguments")
    return p, cls, st


def chunk_stats(x: np.ndarray, dtype: str, chunk_cols: int, mask=None, r0: int = 0,
                r1: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    x = _raw(x, dtype)
    rows, cols = x.shape
    r1 = rows if r1 is None else r1
    nch = (cols + chunk_cols - 1) // chunk_cols
    m = np.empty((r1 - r0, nch), dtype=np.float64)
    l = np.empty((r1 - r0, nch), dtype=np.float64)
    ms, keep = _mask_struct(mask, rows, cols)
    rc = lib().oracle_chunk_stats(_ptr(x), DTYPE_CODE[dtype], rows, cols, C.byref(ms), chunk_cols,
                                  r0, r1, _ptr(m), _ptr(l))
    if rc != 0:
        raise ValueError("oracle_chunk_stats: bad arguments")
    return m, l


def merge(m_a: float, l_a: float, m_b: float, l_b: float) -> Tuple[float, float]:
    mo, lo = C.c_double(), C.c_double()
    lib().oracle_merge(m_a, l_a, m_b, l_b, C.byref(mo), C.byref(lo))
    return mo.value, lo.value


def merge_all(m: np.ndarray, l: np.ndarray) -> Tuple[float, float]:
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    mo, lo = C.c_double(), C.c_double()
    lib().oracle_merge_all(_ptr(m), _ptr(l), m.size, C.byref(mo), C.byref(lo))
    return mo.value, lo.value


def merge_normalize(x: np.ndarray, dtype: str, m: np.ndarray, l: np.ndarray, mask=None,
                    r0: int = 0, r1: Optional[int] = None):
    x = _raw(x, dtype)
    rows, cols = x.shape
    r1 = rows if r1 is None else r1
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    nch = m.shape[1]
    assert m.shape == (r1 - r0, nch) and l.shape == m.shape
    p = np.empty((r1 - r0, cols), dtype=np.float64)
    cls = np.empty((r1 - r0, cols), dtype=np.uint8)
    st = np.empty(r1 - r0, dtype=np.int32)
    ms, keep = _mask_struct(mask, rows, cols)
    rc = lib().oracle_merge_normalize(_ptr(x), DTYPE_CODE[dtype], rows, cols, C.byref(ms), _ptr(m),
                                      _ptr(l), nch, r0, r1, _ptr(p), _ptr(cls), _ptr(st))
    if rc != 0:
        raise ValueError("oracle_merge_normalize: bad arguments")
    return p, cls, st


def _trace(fn, x, *extra):
    x = np.ascontiguousarray(x, dtype=np.float64)
    n_out = x.size if not extra else -(-x.size // extra[0])
    m = np.empty(n_out, dtype=np.float64)
    d = np.empty(n_out, dtype=np.float64)
    fn(_ptr(x), x.size, *extra, _ptr(m), _ptr(d))
    return m, d


def online_elementwise(x):
    return _trace(lib().oracle_online_elementwise, x)


def online_tiled(x, tile: int):
    return _trace(lib().oracle_online_tiled, x, tile)


def online_no_rescale(x):
    """Deliberately wrong negative control: never rescales the running sum."""
    return _trace(lib().oracle_online_no_rescale, x)


def log_softmax_rows(x: np.ndarray, dtype: str, mask=None, r0: int = 0, r1: Optional[int] = None):
    x = _raw(x, dtype)
    rows, cols = x.shape
    r1 = rows if r1 is None else r1
    lse = np.empty(r1 - r0, dtype=np.float64)
    logp = np.empty((r1 - r0, cols), dtype=np.float64)
    ms, keep = _mask_struct(mask, rows, cols)
    rc = lib().oracle_log_softmax_rows(_ptr(x), DTYPE_CODE[dtype], rows, cols, C.byref(ms), r0, r1,
                                       _ptr(lse), _ptr(logp))
    if rc != 0:
        raise ValueError("oracle_log_softmax_rows: bad arguments")
    return lse, logp


def softmax_backward_rows(p: np.ndarray, g: np.ndarray, dtype: str, r0: int = 0,
                          r1: Optional[int] = None) -> np.ndarray:
    p = _raw(p, dtype)
    g = _raw(g, dtype)
    rows, cols = p.shape
    r1 = rows if r1 is None else r1
    dx = np.empty((r1 - r0, cols), dtype=np.float64)
    rc = lib().oracle_softmax_backward_rows(_ptr(p), _ptr(g), DTYPE_CODE[dtype], rows, cols, r0, r1,
                                            _ptr(dx))
    if rc != 0:
        raise ValueError("oracle_softmax_backward_rows: bad arguments")
    return dx


def cross_entropy_rows(x: np.ndarray, dtype: str, target: np.ndarray, mask=None, r0: int = 0,
                       r1: Optional[int] = None, want_dx: bool = True):
    """Per-row loss LSE - x_t (float64) and, if asked, dx = p - onehot(t)."""
    x = _raw(x, dtype)
    rows, cols = x.shape
    r1 = rows if r1 is None else r1
    t = np.ascontiguousarray(target, dtype=np.int32)
    assert t.shape == (rows,)
    loss = np.empty(r1 - r0, dtype=np.float64)
    dx = np.empty((r1 - r0, cols), dtype=np.float64) if want_dx else None
    ms, keep = _mask_struct(mask, rows, cols)
    rc = lib().oracle_cross_entropy_rows(_ptr(x), DTYPE_CODE[dtype], rows, cols, C.byref(ms), _ptr(t), r0, r1,
                                         _ptr(loss), _ptr(dx))
    if rc != 0:
        raise ValueError("oracle_cross_entropy_rows: bad arguments")
    return loss, dx


def softmax_weighted_rows(s: np.ndarray, v: np.ndarray, dtype: str, rows_per_group: int, mask=None,
                          r0: int = 0, r1: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """out[r] = softmax(s[r]) @ v[r // rows_per_group] in double; returns (out [r1-r0, d], row status)."""
    s = _raw(s, dtype)
    v = _raw(v, dtype)
    rows, cols = s.shape
    d = v.shape[-1]
    if v.shape != (rows // rows_per_group, cols, d):
        raise ValueError(f"v must be [rows / rows_per_group, cols, d], got {v.shape}")
    r1 = rows if r1 is None else r1
    out = np.empty((r1 - r0, d), dtype=np.float64)
    st = np.empty(r1 - r0, dtype=np.int32)
    ms, keep = _mask_struct(mask, rows, cols)
    rc = lib().oracle_softmax_weighted_rows(_ptr(s), _ptr(v), DTYPE_CODE[dtype], rows, cols, d, rows_per_group,
                                            C.byref(ms), r0, r1, _ptr(out), _ptr(st))
    if rc != 0:
        raise ValueError("oracle_softmax_weighted_rows: bad arguments")
    return out, st


def weighted_chunk_states(s: np.ndarray, v: np.ndarray, dtype: str, rows_per_group: int, chunk_cols: int,
                          mask=None, r0: int = 0, r1: Optional[int] = None):
    """Per-chunk (m, l, o) states: m, l [r1-r0, n_chunks], o [r1-r0, n_chunks, d]."""
    s = _raw(s, dtype)
    v = _raw(v, dtype)
    rows, cols = s.shape
    d = v.shape[-1]
    r1 = rows if r1 is None else r1
    nch = (cols + chunk_cols - 1) // chunk_cols
    m = np.empty((r1 - r0, nch), dtype=np.float64)
    l = np.empty((r1 - r0, nch), dtype=np.float64)
    o = np.empty((r1 - r0, nch, d), dtype=np.float64)
    ms, keep = _mask_struct(mask, rows, cols)
    rc = lib().oracle_weighted_chunk_states(_ptr(s), _ptr(v), DTYPE_CODE[dtype], rows, cols, d, rows_per_group,
                                            C.byref(ms), chunk_cols, r0, r1, _ptr(m), _ptr(l), _ptr(o))
    if rc != 0:
        raise ValueError("oracle_weighted_chunk_states: bad arguments")
    return m, l, o


def weighted_merge(m_a: float, l_a: float, o_a: np.ndarray, m_b: float, l_b: float, o_b: np.ndarray):
    o_a = np.ascontiguousarray(o_a, dtype=np.float64)
    o_b = np.ascontiguousarray(o_b, dtype=np.float64)
    out = np.empty_like(o_a)
    mo, lo = C.c_double(), C.c_double()
    lib().oracle_weighted_merge(m_a, l_a, _ptr(o_a), m_b, l_b, _ptr(o_b), o_a.size, C.byref(mo), C.byref(lo),
                                _ptr(out))
    return mo.value, lo.value, out


def round_f16_bits(v: float) -> int:
    return int(lib().oracle_round_f16_bits(float(v)))


def round_bf16_bits(v: float) -> int:
    return int(lib().oracle_round_bf16_bits(float(v)))


def round_f32_bits(v: float) -> int:
    return int(lib().oracle_round_f32_bits(float(v)))


def encode(p: np.ndarray, dtype: str) -> np.ndarray:
    """Round doubles to the element format's raw storage (float32 or uint16 bits)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    out = np.empty(p.shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    lib().oracle_encode(_ptr(p), p.size, DTYPE_CODE[dtype], _ptr(out))
    return out


def softmax_rows_encode_mt(x: np.ndarray, dtype: str, mask=None, threads: int = 1,
                           out: Optional[np.ndarray] = None):
    """The CPU baseline: three-pass rows over `threads` host threads, written in
    the element format (into `out` when given: raw storage of x's shape).
    Returns (y, seconds)."""
    x = _raw(x, dtype)
    rows, cols = x.shape
    if out is not None:
        if out.shape != x.shape or out.dtype != x.dtype or not out.flags.c_contiguous:
            raise ValueError("out must be contiguous raw storage of x's shape")
        y = out
    else:
        y = np.empty_like(x)
    ms, keep = _mask_struct(mask, rows, cols)
    t0 = time.perf_counter()
    rc = lib().oracle_softmax_rows_encode_mt(_ptr(x), _ptr(y), DTYPE_CODE[dtype], rows, cols,
                                             C.byref(ms), int(threads))
    dt = time.perf_counter() - t0
    if rc != 0:
        raise RuntimeError("oracle_softmax_rows_encode_mt failed")
    return y, dt


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact decode of raw storage into float64, element by element, through oracle_decode."""
    x = _raw(x, dtype)
    flat = x.reshape(-1)
    L = lib()
    return np.array([L.oracle_decode(_ptr(flat), DTYPE_CODE[dtype], i) for i in range(flat.size)],
                    dtype=np.float64).reshape(x.shape)

"""Python binding of the gfx950 row-softmax library (libsmx.so).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI declared in include/smx.h, and every step
of the computation runs in the library's HIP kernels. PyTorch supplies device
memory and streams. There is no CPU fallback: if the library is not built,
importing this package raises.

Functions keep the C names:
  softmax_rows(x, ...)              -> y
  softmax_rows_noalloc(x, out, ...) -> out (allocates no device memory)
  softmax_row_stats(x, chunk_cols)  -> stats [rows, n_chunks, 2] (m, l)
  softmax_merge_normalize(x, stats, chunk_cols) -> y
  log_softmax_rows(x, ...)          -> (y, lse)
  softmax_backward_rows(p, g)       -> dx
  softmax_cross_entropy_rows(x, t)  -> (loss, dx)
  softmax_default_chunk_cols(rows, cols, dtype)
  softmax_select_path(rows, cols, dtype)
  stream_copy(x, y)                 (a plain copy: the bandwidth reference, no softmax step)
  smx_last_error()
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch  # loads the HIP runtime this library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmx.so")

SMX_OK, SMX_EINVAL, SMX_EHIP = 0, 1, 2
DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
DTYPE_NAME = {"f32": 0, "f16": 1, "bf16": 2}
MASK = {"none": 0, "valid_len": 1, "causal": 2, "keep": 3}
PATH = {"auto": 0, "wave": 1, "lds": 2, "split": 3}
PATH_NAME = {v: k for k, v in PATH.items()}


class SmxMask(C.Structure):
    _fields_ = [
        ("kind", C.c_int),
        ("valid_len", C.c_void_p),
        ("causal_period", C.c_int64),
        ("causal_offset", C.c_int64),
        ("keep", C.c_void_p),
    ]


class SmxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"smx error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> C.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with numerically_stable_online_amd/build.py "
                "(or __graft_entry__.build()); there is no fallback implementation")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        mp = C.POINTER(SmxMask)
        L.softmax_rows.argtypes = [vp, vp, i64, i64, i32, mp, vp]
        L.softmax_rows.restype = i32
        L.softmax_rows_path.argtypes = [vp, vp, i64, i64, i32, mp, i32, i64, vp]
        L.softmax_rows_path.restype = i32
        L.softmax_rows_noalloc.argtypes = [vp, vp, i64, i64, i32, mp, i32, i64, vp]
        L.softmax_rows_noalloc.restype = i32
        L.softmax_select_path.argtypes = [i64, i64, i32]
        L.softmax_select_path.restype = i32
        L.softmax_row_stats.argtypes = [vp, i64, i64, i32, mp, i64, vp, vp]
        L.softmax_row_stats.restype = i32
        L.softmax_merge_normalize.argtypes = [vp, vp, i64, i64, i32, mp, i64, vp, i64, vp]
        L.softmax_merge_normalize.restype = i32
        L.log_softmax_rows.argtypes = [vp, vp, vp, i64, i64, i32, mp, vp]
        L.log_softmax_rows.restype = i32
        L.log_softmax_rows_path.argtypes = [vp, vp, vp, i64, i64, i32, mp, i32, i64, vp]
        L.log_softmax_rows_path.restype = i32
        L.softmax_cross_entropy_rows.argtypes = [vp, vp, vp, vp, i64, i64, i32, mp, vp]
        L.softmax_cross_entropy_rows.restype = i32
        L.softmax_cross_entropy_rows_path.argtypes = [vp, vp, vp, vp, i64, i64, i32, mp, i32, i64, vp]
        L.softmax_cross_entropy_rows_path.restype = i32
        L.softmax_backward_rows.argtypes = [vp, vp, vp, i64, i64, i32, vp]
        L.softmax_backward_rows.restype = i32
        L.softmax_backward_rows_path.argtypes = [vp, vp, vp, i64, i64, i32, i32, i64, vp]
        L.softmax_backward_rows_path.restype = i32
        L.softmax_weighted_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, mp, vp]
        L.softmax_weighted_rows.restype = i32
        L.softmax_weighted_states.argtypes = [vp, vp, i64, i64, i64, i64, i32, mp, i64, vp, vp, vp]
        L.softmax_weighted_states.restype = i32
        L.softmax_weighted_merge.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp]
        L.softmax_weighted_merge.restype = i32
        L.softmax_default_chunk_cols.argtypes = [i64, i64, i32]
        L.softmax_default_chunk_cols.restype = i64
        L.smx_stream_copy.argtypes = [vp, vp, i64, vp]
        L.smx_stream_copy.restype = i32
        L.smx_last_error.argtypes = []
        L.smx_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def smx_last_error() -> str:
    return lib().smx_last_error().decode()


def _check(rc: int) -> None:
    if rc != SMX_OK:
        raise SmxError(rc, smx_last_error())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, device) -> int:
    """The hipStream_t to launch on: the given stream, else torch's current
    stream on x's device."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16") from None


def _rows_cols(x: torch.Tensor):
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (row-major)")
    if x.device.type != "cuda":
        raise ValueError("x must be a device tensor")
    return x.shape[0], x.shape[1]


def _on(t: torch.Tensor, device, what: str) -> None:
    if t.device != device:
        raise ValueError(f"{what} must be on {device} (the library reads it on the device), got {t.device}")


def make_mask(rows: int, cols: int, valid_len: Optional[torch.Tensor] = None,
              causal_period: Optional[int] = None, causal_offset: int = 0,
              keep: Optional[torch.Tensor] = None, device=None):
    """Build the C mask descriptor; returns (struct or None, tensors to keep alive)."""
    given = sum(v is not None for v in (valid_len, causal_period, keep))
    if given > 1:
        raise ValueError("give at most one of valid_len, causal_period, keep")
    if given == 0:
        return None, ()
    m = SmxMask()
    if valid_len is not None:
        if valid_len.dtype != torch.int32 or valid_len.shape != (rows,) or not valid_len.is_contiguous():
            raise ValueError("valid_len must be a contiguous int32 device tensor of shape [rows]")
        if device is not None:
            _on(valid_len, device, "valid_len")
        m.kind = MASK["valid_len"]
        m.valid_len = valid_len.data_ptr()
        return m, (valid_len,)
    if causal_period is not None:
        m.kind = MASK["causal"]
        m.causal_period = int(causal_period)
        m.causal_offset = int(causal_offset)
        return m, ()
    if keep.dtype not in (torch.uint8, torch.bool) or keep.shape != (rows, cols) or not keep.is_contiguous():
        raise ValueError("keep must be a contiguous uint8/bool device tensor of shape [rows, cols]")
    if device is not None:
        _on(keep, device, "keep")
    m.kind = MASK["keep"]
    m.keep = keep.data_ptr()
    return m, (keep,)


def _mask_arg(m):
    return None if m is None else C.byref(m)


def stream_copy(x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """smx_stream_copy: y[:] = x through the library's streaming copy (the
    bandwidth reference; x and y contiguous device tensors of equal byte size,
    16-byte aligned, disjoint)."""
    nbytes = x.numel() * x.element_size()
    if not (x.is_contiguous() and y.is_contiguous()) or y.numel() * y.element_size() != nbytes:
        raise ValueError("x and y must be contiguous and of the same byte size")
    if x.device.type != "cuda":
        raise ValueError("x must be a device tensor")
    _on(y, x.device, "y")
    _check(lib().smx_stream_copy(x.data_ptr(), y.data_ptr(), nbytes, _stream_handle(stream, x.device)))
    return y


def softmax_rows(x: torch.Tensor, out: Optional[torch.Tensor] = None, *, valid_len=None,
                 causal_period=None, causal_offset: int = 0, keep=None, path: str = "auto",
                 chunk_cols: int = 0, stream=None) -> torch.Tensor:
    """Row-wise stable softmax of x [rows, cols] (float32, float16 or bfloat16)."""
    rows, cols = _rows_cols(x)
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("out must be a contiguous tensor of x's shape and dtype")
    _on(y, x.device, "out")
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, x.device)
    rc = lib().softmax_rows_path(x.data_ptr(), y.data_ptr(), rows, cols, _dtype_code(x), _mask_arg(m),
                                 PATH[path], int(chunk_cols), _stream_handle(stream, x.device))
    _check(rc)
    return y


def softmax_rows_noalloc(x: torch.Tensor, out: torch.Tensor, *, valid_len=None, causal_period=None,
                         causal_offset: int = 0, keep=None, path: str = "auto", chunk_cols: int = 0,
                         stream=None) -> torch.Tensor:
    """softmax_rows into a caller-given out, through the entry point that
    allocates no device memory (the split path's summaries live in the
    library's fixed per-device scratch; calls that overlap on one device race)."""
    rows, cols = _rows_cols(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of x's shape and dtype")
    _on(out, x.device, "out")
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, x.device)
    rc = lib().softmax_rows_noalloc(x.data_ptr(), out.data_ptr(), rows, cols, _dtype_code(x), _mask_arg(m),
                                    PATH[path], int(chunk_cols), _stream_handle(stream, x.device))
    _check(rc)
    return out


def log_softmax_rows(x: torch.Tensor, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     *, want_y: bool = True, want_lse: bool = True, valid_len=None, causal_period=None,
                     causal_offset: int = 0, keep=None, path: str = "auto", chunk_cols: int = 0, stream=None):
    """Log-probabilities y = x - LSE and the per-row log-sum-exp (float32 [rows]).
    Returns (y or None, lse or None)."""
    rows, cols = _rows_cols(x)
    if not (want_y or want_lse):
        raise ValueError("ask for y, lse or both")
    y = None
    if want_y:
        y = torch.empty_like(x) if out is None else out
        if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
            raise ValueError("out must be a contiguous tensor of x's shape and dtype")
        _on(y, x.device, "out")
    ls = None
    if want_lse:
        ls = torch.empty(rows, dtype=torch.float32, device=x.device) if lse is None else lse
        if ls.shape != (rows,) or ls.dtype != torch.float32 or not ls.is_contiguous():
            raise ValueError("lse must be a contiguous float32 tensor [rows]")
        _on(ls, x.device, "lse")
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, x.device)
    rc = lib().log_softmax_rows_path(x.data_ptr(), None if y is None else y.data_ptr(),
                                     None if ls is None else ls.data_ptr(), rows, cols, _dtype_code(x),
                                     _mask_arg(m), PATH[path], int(chunk_cols), _stream_handle(stream, x.device))
    _check(rc)
    return y, ls


def softmax_cross_entropy_rows(x: torch.Tensor, target: torch.Tensor, loss: Optional[torch.Tensor] = None,
                               dx: Optional[torch.Tensor] = None, *, want_dx: bool = True, valid_len=None,
                               causal_period=None, causal_offset: int = 0, keep=None, path: str = "auto",
                               chunk_cols: int = 0, stream=None):
    """Per-row cross-entropy LSE - x_t (float32 [rows]) and, if asked, the
    gradient softmax(x) - onehot(t) in x's dtype. Returns (loss, dx or None)."""
    rows, cols = _rows_cols(x)
    if target.dtype != torch.int32 or target.shape != (rows,) or not target.is_contiguous():
        raise ValueError("target must be a contiguous int32 tensor [rows]")
    _on(target, x.device, "target")
    ls = torch.empty(rows, dtype=torch.float32, device=x.device) if loss is None else loss
    if ls.shape != (rows,) or ls.dtype != torch.float32 or not ls.is_contiguous():
        raise ValueError("loss must be a contiguous float32 tensor [rows]")
    _on(ls, x.device, "loss")
    g = None
    if want_dx:
        g = torch.empty_like(x) if dx is None else dx
        if g.shape != x.shape or g.dtype != x.dtype or not g.is_contiguous():
            raise ValueError("dx must be a contiguous tensor of x's shape and dtype")
        _on(g, x.device, "dx")
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, x.device)
    rc = lib().softmax_cross_entropy_rows_path(x.data_ptr(), target.data_ptr(), ls.data_ptr(),
                                               None if g is None else g.data_ptr(), rows, cols, _dtype_code(x),
                                               _mask_arg(m), PATH[path], int(chunk_cols),
                                               _stream_handle(stream, x.device))
    _check(rc)
    return ls, g


def softmax_weighted_rows(s: torch.Tensor, v: torch.Tensor, out: Optional[torch.Tensor] = None, *,
                          valid_len=None, causal_period=None, causal_offset: int = 0, keep=None,
                          stream=None) -> torch.Tensor:
    """out[r] = softmax(s[r]) @ v[r // rows_per_group]: s [rows, cols], v [groups, cols, d]
    (rows_per_group = rows / groups), out [rows, d], all float16 or all bfloat16."""
    rows, cols = _rows_cols(s)
    if v.dim() != 3 or v.shape[1] != cols or v.dtype != s.dtype or not v.is_contiguous():
        raise ValueError("v must be a contiguous [groups, cols, d] tensor of s's dtype")
    _on(v, s.device, "v")
    groups, _, d = v.shape
    if groups == 0 or rows % groups != 0:
        raise ValueError("rows must be a multiple of the number of value matrices")
    o = torch.empty((rows, d), dtype=s.dtype, device=s.device) if out is None else out
    if o.shape != (rows, d) or o.dtype != s.dtype or not o.is_contiguous():
        raise ValueError("out must be a contiguous [rows, d] tensor of s's dtype")
    _on(o, s.device, "out")
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, s.device)
    rc = lib().softmax_weighted_rows(s.data_ptr(), v.data_ptr(), o.data_ptr(), rows, cols, d, rows // groups,
                                     _dtype_code(s), _mask_arg(m), _stream_handle(stream, s.device))
    _check(rc)
    return o


def softmax_weighted_states(s: torch.Tensor, v: torch.Tensor, chunk_cols: int, ml: Optional[torch.Tensor] = None,
                            o: Optional[torch.Tensor] = None, *, valid_len=None, causal_period=None,
                            causal_offset: int = 0, keep=None, stream=None):
    """Per-(row, key chunk) states of softmax(s) @ v: ml float32 [rows, n_chunks, 2] (the chunk
    maximum m and l = sum exp(s - m)) and o float32 [rows, n_chunks, d] (sum exp(s - m) v).
    Returns (ml, o)."""
    rows, cols = _rows_cols(s)
    if v.dim() != 3 or v.shape[1] != cols or v.dtype != s.dtype or not v.is_contiguous():
        raise ValueError("v must be a contiguous [groups, cols, d] tensor of s's dtype")
    _on(v, s.device, "v")
    groups, _, d = v.shape
    if groups == 0 or rows % groups != 0:
        raise ValueError("rows must be a multiple of the number of value matrices")
    nch = -(-cols // chunk_cols) if chunk_cols > 0 else 0
    ml = torch.empty((rows, nch, 2), dtype=torch.float32, device=s.device) if ml is None else ml
    o = torch.empty((rows, nch, d), dtype=torch.float32, device=s.device) if o is None else o
    for t, shape, name in ((ml, (rows, nch, 2), "ml"), (o, (rows, nch, d), "o")):
        if t.shape != shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor {list(shape)}")
        _on(t, s.device, name)
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, s.device)
    rc = lib().softmax_weighted_states(s.data_ptr(), v.data_ptr(), rows, cols, d, rows // groups, _dtype_code(s),
                                       _mask_arg(m), int(chunk_cols), ml.data_ptr(), o.data_ptr(),
                                       _stream_handle(stream, s.device))
    _check(rc)
    return ml, o


def softmax_weighted_merge(ml: torch.Tensor, o: torch.Tensor, dtype: torch.dtype, out: Optional[torch.Tensor] = None,
                           *, stream=None) -> torch.Tensor:
    """Fold each row's chunk states (as softmax_weighted_states writes them) and write
    O / L in dtype (torch.float16 or torch.bfloat16): out [rows, d]."""
    if ml.dim() != 3 or ml.shape[2] != 2 or ml.dtype != torch.float32 or not ml.is_contiguous():
        raise ValueError("ml must be a contiguous float32 tensor [rows, n_chunks, 2]")
    rows, nch, _ = ml.shape
    if o.dim() != 3 or o.shape[:2] != (rows, nch) or o.dtype != torch.float32 or not o.is_contiguous():
        raise ValueError("o must be a contiguous float32 tensor [rows, n_chunks, d]")
    _on(o, ml.device, "o")
    d = o.shape[2]
    y = torch.empty((rows, d), dtype=dtype, device=ml.device) if out is None else out
    if y.shape != (rows, d) or y.dtype != dtype or not y.is_contiguous():
        raise ValueError("out must be a contiguous [rows, d] tensor of the given dtype")
    _on(y, ml.device, "out")
    rc = lib().softmax_weighted_merge(ml.data_ptr(), o.data_ptr(), rows, nch, d, DTYPE[dtype], y.data_ptr(),
                                      _stream_handle(stream, ml.device))
    _check(rc)
    return y


def softmax_backward_rows(p: torch.Tensor, g: torch.Tensor, out: Optional[torch.Tensor] = None, *,
                          path: str = "auto", chunk_cols: int = 0, stream=None) -> torch.Tensor:
    """dx = p * (g - sum(g * p)) row by row (the softmax vector-Jacobian product)."""
    rows, cols = _rows_cols(p)
    if g.shape != p.shape or g.dtype != p.dtype or not g.is_contiguous():
        raise ValueError("g must be a contiguous tensor of p's shape and dtype")
    _on(g, p.device, "g")
    dx = torch.empty_like(p) if out is None else out
    if dx.shape != p.shape or dx.dtype != p.dtype or not dx.is_contiguous():
        raise ValueError("out must be a contiguous tensor of p's shape and dtype")
    _on(dx, p.device, "out")
    rc = lib().softmax_backward_rows_path(p.data_ptr(), g.data_ptr(), dx.data_ptr(), rows, cols, _dtype_code(p),
                                          PATH[path], int(chunk_cols), _stream_handle(stream, p.device))
    _check(rc)
    return dx


def softmax_row_stats(x: torch.Tensor, chunk_cols: int, out: Optional[torch.Tensor] = None, *,
                      valid_len=None, causal_period=None, causal_offset: int = 0, keep=None,
                      stream=None) -> torch.Tensor:
    """Per-chunk (m, l) summaries, float32 [rows, n_chunks, 2]."""
    rows, cols = _rows_cols(x)
    nch = -(-cols // chunk_cols) if chunk_cols > 0 else 0
    st = torch.empty((rows, nch, 2), dtype=torch.float32, device=x.device) if out is None else out
    if st.shape != (rows, nch, 2) or st.dtype != torch.float32 or not st.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor [rows, n_chunks, 2]")
    _on(st, x.device, "out")
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, x.device)
    rc = lib().softmax_row_stats(x.data_ptr(), rows, cols, _dtype_code(x), _mask_arg(m), int(chunk_cols),
                                 st.data_ptr(), _stream_handle(stream, x.device))
    _check(rc)
    return st


def softmax_merge_normalize(x: torch.Tensor, stats: torch.Tensor, chunk_cols: int,
                            out: Optional[torch.Tensor] = None, *, valid_len=None, causal_period=None,
                            causal_offset: int = 0, keep=None, stream=None) -> torch.Tensor:
    """Merge each row's chunk summaries and write exp(x - M) / L."""
    rows, cols = _rows_cols(x)
    if stats.dim() != 3 or stats.shape[0] != rows or stats.shape[2] != 2 or stats.dtype != torch.float32 \
            or not stats.is_contiguous():
        raise ValueError("stats must be a contiguous float32 tensor [rows, n_chunks, 2]")
    _on(stats, x.device, "stats")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("out must be a contiguous tensor of x's shape and dtype")
    _on(y, x.device, "out")
    m, keepalive = make_mask(rows, cols, valid_len, causal_period, causal_offset, keep, x.device)
    rc = lib().softmax_merge_normalize(x.data_ptr(), y.data_ptr(), rows, cols, _dtype_code(x), _mask_arg(m),
                                       int(chunk_cols), stats.data_ptr(), stats.shape[1],
                                       _stream_handle(stream, x.device))
    _check(rc)
    return y


def softmax_default_chunk_cols(rows: int, cols: int, dtype) -> int:
    code = DTYPE[dtype] if isinstance(dtype, torch.dtype) else DTYPE_NAME[dtype]
    return int(lib().softmax_default_chunk_cols(rows, cols, code))


def softmax_select_path(rows: int, cols: int, dtype) -> str:
    code = DTYPE[dtype] if isinstance(dtype, torch.dtype) else DTYPE_NAME[dtype]
    return PATH_NAME[int(lib().softmax_select_path(rows, cols, code))]

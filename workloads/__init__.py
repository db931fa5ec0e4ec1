"""Seeded synthetic inputs for the row-softmax workloads.

Shared by the tests, the benchmark and the smoke check, on both sides of
every comparison (the CPU oracle and the HIP library). This module holds no
softmax arithmetic: it draws random logits, rounds them to the element
format, places the special values of the declared policy, and describes the
masks as plain data.

The five workload shapes stand in for the "attention-score rows" the source
pages talk about; no public dataset or suite is involved:

* ``small_rows`` fp32, 64 x 1024, logits 3*N(0,1); plus the two fixed rows
  [20, 18, 17, -5] ("Softmax numerics architecture", worked fp16 example) and
  [1000, 999, 997] ("Online stable softmax", opening example).
* ``spiked_rows`` bf16, 8192 x 4096, logits 8*N(0,1) plus +30 at one random
  column per row.
* ``masked_rows`` fp16, 32768 x 512, logits U(-40, 40), per-row valid length
  uniform on {0, ..., 512}.
* ``long_rows`` fp32, 64 x 1048576, logits 4*N(0,1) plus a ramp 50*j/(cols-1).
* ``causal_scores`` bf16, 256 groups x 2048 rows x 2048 cols, scores q.k^T/sqrt(128)
  of N(0,1) q, k with head dimension 128, causal (row i of a group keeps
  columns 0..i), with five injected special rows per group.
* ``vocab_rows`` bf16, 4096 x 32768, logits 4*N(0,1): output-head rows over
  a vocabulary ("Softmax numerics architecture", memory-traffic account:
  the softmax and loss of the output head).

Every generator takes a seed (defaults 1 to 6, in the order above) and optional
smaller shapes, so a test can draw the same distribution at a size the
oracle finishes in seconds.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2}
MASK_CODE = {"none": 0, "valid_len": 1, "causal": 2, "keep": 3}


@dataclasses.dataclass
class MaskSpec:
    """A mask in the library's descriptor form (plain data)."""

    kind: str = "none"  # none | valid_len | causal | keep
    valid_len: Optional[np.ndarray] = None  # int32 [rows]
    causal_period: int = 0
    causal_offset: int = 0
    keep: Optional[np.ndarray] = None  # uint8 [rows, cols]

    def __post_init__(self):
        if self.kind not in MASK_CODE:
            raise ValueError(f"unknown mask kind {self.kind!r}")


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    x: np.ndarray  # float32 (f32) or uint16 bit patterns (f16, bf16), [rows, cols]
    mask: MaskSpec
    seed: int
    special_rows: Dict[str, np.ndarray] = dataclasses.field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.x.shape[0])

    @property
    def cols(self) -> int:
        return int(self.x.shape[1])


# --------------------------------------------------------------------------
# Element-format helpers (input preparation only).
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns, nearest-even; NaN -> 0x7FC0."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_format(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round real values to the raw storage of an element format."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f16":
        return f64_to_f16_bits(a)
    if dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    raise ValueError(dtype)


def to_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode raw storage to float32 (exact for every format)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return f16_bits_to_f32(x)
    return bf16_bits_to_f32(x)


# special bit patterns
POS_INF = {"f32": np.float32(np.inf), "f16": np.uint16(0x7C00), "bf16": np.uint16(0x7F80)}
NEG_INF = {"f32": np.float32(-np.inf), "f16": np.uint16(0xFC00), "bf16": np.uint16(0xFF80)}
QNAN = {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
# a negative signalling NaN: a policy that only looks for the canonical quiet
# NaN would miss it
NEG_SNAN = {"f32": np.uint32(0xFF800001), "f16": np.uint16(0xFC01), "bf16": np.uint16(0xFF81)}


def set_bits(x: np.ndarray, r: int, c: int, dtype: str, bits) -> None:
    if dtype == "f32":
        x.view(np.uint32)[r, c] = np.uint32(bits)
    else:
        x[r, c] = np.uint16(bits)


def _rng(seed, *stream) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


# --------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------

def small_rows(seed: int = 1, rows: int = 64, cols: int = 1024) -> Workload:
    rng = _rng(seed)
    x = (3.0 * rng.standard_normal((rows, cols))).astype(np.float32)
    return Workload(f"f32_{rows}x{cols}", "f32", x, MaskSpec(), seed)


def fixed_rows() -> List[Workload]:
    """The two rows the pages print, as 1-row fp32 workloads."""
    a = np.array([[20.0, 18.0, 17.0, -5.0]], dtype=np.float32)
    b = np.array([[1000.0, 999.0, 997.0]], dtype=np.float32)
    return [Workload("fixed_20_18_17_m5", "f32", a, MaskSpec(), 0),
            Workload("fixed_1000_999_997", "f32", b, MaskSpec(), 0)]


def spiked_rows(seed: int = 2, rows: int = 8192, cols: int = 4096) -> Workload:
    rng = _rng(seed)
    x = 8.0 * rng.standard_normal((rows, cols), dtype=np.float32)
    spike = rng.integers(0, cols, size=rows)
    x[np.arange(rows), spike] += np.float32(30.0)
    return Workload(f"bf16_{rows}x{cols}_spike", "bf16", f32_to_bf16_bits(x), MaskSpec(), seed,
                    {"spike_col": spike})


def masked_rows(seed: int = 3, rows: int = 32768, cols: int = 512) -> Workload:
    rng = _rng(seed)
    x = rng.uniform(-40.0, 40.0, size=(rows, cols))
    valid = rng.integers(0, cols + 1, size=rows).astype(np.int32)  # both ends inclusive
    return Workload(f"f16_{rows}x{cols}_validlen", "f16", f64_to_f16_bits(x),
                    MaskSpec("valid_len", valid_len=valid), seed)


def long_rows(seed: int = 4, rows: int = 64, cols: int = 1 << 20) -> Workload:
    rng = _rng(seed)
    x = 4.0 * rng.standard_normal((rows, cols), dtype=np.float32)
    x += (50.0 * np.arange(cols, dtype=np.float64) / max(cols - 1, 1)).astype(np.float32)[None, :]
    return Workload(f"f32_{rows}x{cols}_ramp", "f32", x, MaskSpec(), seed)


CAUSAL_SPECIALS = ("pos_inf_valid", "nan_valid", "nan_masked", "pos_inf_masked", "all_neg_inf")


def causal_score_group(g: int, seed: int = 5, n: int = 2048, head_dim: int = 128,
                       inject: bool = True):
    """One (n x n) causal score block, rows g*n .. g*n+n-1 of causal_scores.

    Returns (bits uint16 [n, n], {special name: in-group row index}).
    """
    rng = _rng(seed, g)
    q = rng.standard_normal((n, head_dim), dtype=np.float32)
    k = rng.standard_normal((n, head_dim), dtype=np.float32)
    s = (q @ np.ascontiguousarray(k.T)) * np.float32(1.0 / np.sqrt(head_dim))
    bits = f32_to_bf16_bits(s)
    specials: Dict[str, int] = {}
    if inject and n >= 8:
        srng = _rng(seed, g, 7)
        rows = srng.choice(n - 1, size=5, replace=False)  # row n-1 has no masked lane
        nan_bits = QNAN["bf16"] if g % 2 == 0 else NEG_SNAN["bf16"]
        for name, i in zip(CAUSAL_SPECIALS, rows):
            i = int(i)
            specials[name] = i
            if name in ("pos_inf_valid", "nan_valid"):
                j = int(srng.integers(0, i + 1))
                bits[i, j] = POS_INF["bf16"] if name == "pos_inf_valid" else nan_bits
            elif name in ("nan_masked", "pos_inf_masked"):
                j = int(srng.integers(i + 1, n))
                bits[i, j] = nan_bits if name == "nan_masked" else POS_INF["bf16"]
            else:
                bits[i, : i + 1] = NEG_INF["bf16"]
    return bits, specials


def causal_scores(seed: int = 5, groups: int = 256, n: int = 2048, head_dim: int = 128,
                  out: Optional[np.ndarray] = None) -> Workload:
    rows = groups * n
    x = out if out is not None else np.empty((rows, n), dtype=np.uint16)
    special = {name: [] for name in CAUSAL_SPECIALS}
    for g in range(groups):
        bits, sp = causal_score_group(g, seed, n, head_dim)
        x[g * n:(g + 1) * n] = bits
        for name, i in sp.items():
            special[name].append(g * n + i)
    return Workload(f"bf16_{groups}x{n}x{n}_causal", "bf16", x,
                    MaskSpec("causal", causal_period=n), seed,
                    {k: np.asarray(v, dtype=np.int64) for k, v in special.items()})


def causal_values(seed: int = 5, groups: int = 256, n: int = 2048, head_dim: int = 128) -> np.ndarray:
    """Value vectors for causal_scores' groups (the attention workload that
    weights them by the scores' softmax): per group an [n, head_dim] matrix
    of seeded N(0, 1) values rounded to bf16. Returns uint16 bits
    [groups, n, head_dim]."""
    v = np.empty((groups, n, head_dim), dtype=np.uint16)
    for g in range(groups):
        rng = _rng(seed, g, 11)
        v[g] = f32_to_bf16_bits(rng.standard_normal((n, head_dim), dtype=np.float32))
    return v


def vocab_rows(seed: int = 6, rows: int = 4096, cols: int = 32768) -> Workload:
    """Output-head rows: one row of logits per token over a vocabulary of
    32768 classes, bf16, logits 4*N(0,1). Rows of 64 KiB: longer than the
    registers of one workgroup hold, short enough to stay on chip."""
    rng = _rng(seed)
    x = 4.0 * rng.standard_normal((rows, cols), dtype=np.float32)
    return Workload(f"bf16_{rows}x{cols}_vocab", "bf16", to_format(x, "bf16"), MaskSpec(), seed)


# by short name, in the benchmark's order (its headline is the largest)
WORKLOADS = {"spiked": spiked_rows, "small": small_rows, "masked": masked_rows, "long": long_rows,
             "causal": causal_scores, "vocab": vocab_rows}


def random_rows(rows: int, cols: int, dtype: str, seed: int, scale: float = 4.0,
                dist: str = "normal") -> np.ndarray:
    """Generic seeded logits for odd-shape sweeps."""
    rng = _rng(seed, rows, cols)
    if dist == "normal":
        a = scale * rng.standard_normal((rows, cols))
    elif dist == "uniform":
        a = rng.uniform(-scale, scale, size=(rows, cols))
    else:
        raise ValueError(dist)
    return to_format(a, dtype)


def class_targets(rows: int, cols: int, seed: int) -> np.ndarray:
    """Seeded class indices in [0, cols), one per row (int32), for the
    cross-entropy entry point."""
    rng = _rng(seed, rows, cols, 7)
    return rng.integers(0, cols, rows).astype(np.int32)

"""The entry point that allocates nothing, softmax_rows_noalloc, through the C
ABI. Its split path keeps the chunk summaries in the library's fixed
per-device scratch instead of a stream-ordered allocation; every other step
is the same kernels, so its output must equal softmax_rows_path's bit for bit,
and both are held to the oracle. The calls come in pairs on the shared
scratch, the second with a smaller input than the first, so a summary left
behind by the first call would show up in the second.
"""
import numpy as np
import pytest
import torch

import numerically_stable_online_amd as smx
import oracle
import workloads as W
from smx_compare import check, to_device, to_host

pytestmark = pytest.mark.gpu


def banner(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def _mask(kind, rows, cols, rng):
    if kind == "valid_len":
        v = rng.integers(0, cols + 1, rows).astype(np.int32)
        v[0] = 0  # an empty row
        return W.MaskSpec("valid_len", valid_len=v), {"valid_len": torch.from_numpy(v).cuda()}
    if kind == "causal":
        return W.MaskSpec("causal", causal_period=rows, causal_offset=cols // 3), \
            {"causal_period": rows, "causal_offset": cols // 3}
    return W.MaskSpec(), {}


# pairs of calls (dtype, rows, cols, path, chunk_cols, mask); the second call
# of each pair is smaller than the first
PAIRS = [
    [("f32", 64, 262144, "split", 0, "none"), ("f32", 5, 70001, "split", 4096, "none")],
    # more than 1024 chunks per row: the per-row merged summaries use scratch too
    [("bf16", 3, 300000, "split", 256, "causal"), ("bf16", 2, 140000, "split", 128, "none")],
    [("f16", 300, 20000, "split", 2048, "valid_len"), ("f16", 100, 9000, "split", 1000, "valid_len")],
    # paths that need no scratch
    [("bf16", 1024, 4096, "auto", 0, "none"), ("f32", 1000, 512, "auto", 0, "causal")],
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_equals_path_call(pair):
    rng = np.random.default_rng(900 + pair)
    for dtype, rows, cols, path, chunk, mk in PAIRS[pair]:
        banner(f"softmax_rows_noalloc {dtype} {rows}x{cols} path={path} chunk={chunk} mask={mk}")
        xr = W.random_rows(rows, cols, dtype, seed=900 + pair, scale=6.0)
        if rows > 2:
            inf_bits = W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype]
            W.set_bits(xr, 1, cols // 2, dtype, inf_bits)  # a poisoned row (in a valid lane, or masked)
        mask, kw = _mask(mk, rows, cols, rng)
        x = to_device(xr, dtype)
        y_ref = torch.empty_like(x)
        y_new = torch.full_like(x, 7.0)
        smx.softmax_rows(x, y_ref, path=path, chunk_cols=chunk, **kw)
        smx.softmax_rows_noalloc(x, y_new, path=path, chunk_cols=chunk, **kw)
        torch.cuda.synchronize()
        a, b = to_host(y_ref, dtype), to_host(y_new, dtype)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (dtype, rows, cols, path, chunk)
        p, cls, st = oracle.softmax_rows(xr, dtype, mask)
        check(b, dtype, p, cls, st, f"noalloc {dtype} {rows}x{cols} {path}")


def test_noalloc_rejects_beyond_its_scratch():
    """A split-path call whose summaries exceed the scratch is refused before
    anything runs, and the output is left untouched."""
    x = torch.zeros((4096, 8192), dtype=torch.float32, device="cuda")
    y = torch.full_like(x, 3.0)
    with pytest.raises(smx.SmxError) as e:
        smx.softmax_rows_noalloc(x, y, path="split", chunk_cols=16)  # 4096 x 512 x 8 B = 16 MiB
    assert e.value.code == smx.SMX_EINVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    # the same shape with chunks large enough to fit runs
    smx.softmax_rows_noalloc(x, y, path="split", chunk_cols=4096)
    torch.cuda.synchronize()
    assert torch.allclose(y, torch.full_like(y, 1.0 / 8192), rtol=1e-6, atol=0)

"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every comparison is element by element, to the bars in smx_compare: f32 within
1e-6 relative and rows summing to 1 within 1e-5, f16/bf16 within 1 ulp of the
correctly rounded oracle value, policy lanes bit-exact. The five workloads run
at their full sizes, with the launch configuration the benchmark times (the
automatic path), and again on every other path that can hold them.
"""
import numpy as np
import pytest
import torch

import numerically_stable_online_amd as smx
import oracle
import workloads as W
from smx_compare import TORCH_DTYPE, check, to_device, to_host

pytestmark = pytest.mark.gpu


def banner(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def mask_kwargs(mask: W.MaskSpec):
    if mask is None or mask.kind == "none":
        return {}
    if mask.kind == "valid_len":
        return {"valid_len": torch.from_numpy(np.ascontiguousarray(mask.valid_len, dtype=np.int32)).cuda()}
    if mask.kind == "causal":
        return {"causal_period": mask.causal_period, "causal_offset": mask.causal_offset}
    return {"keep": torch.from_numpy(np.ascontiguousarray(mask.keep, dtype=np.uint8)).cuda()}


def run_rows(x_raw, dtype, mask=None, path="auto", chunk_cols=0, misalign=False):
    rows, cols = x_raw.shape
    if misalign:  # shift x and y one element off any 16-byte boundary
        buf = torch.empty(rows * cols + 1, dtype=TORCH_DTYPE[dtype], device="cuda")
        x = buf[1:].view(rows, cols)
        x.copy_(to_device(x_raw, dtype))
        ybuf = torch.empty(rows * cols + 1, dtype=TORCH_DTYPE[dtype], device="cuda")
        y = ybuf[1:].view(rows, cols)
    else:
        x = to_device(x_raw, dtype)
        y = torch.empty_like(x)
    smx.softmax_rows(x, y, path=path, chunk_cols=chunk_cols, **mask_kwargs(mask))
    torch.cuda.synchronize()
    return to_host(y, dtype)


def check_full(x_raw, dtype, mask, y_raw, what):
    p, cls, st = oracle.softmax_rows(x_raw, dtype, mask)
    return check(y_raw, dtype, p, cls, st, what)


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def test_select_path_for_workloads():
    assert smx.softmax_select_path(64, 1024, "f32") == "wave"
    assert smx.softmax_select_path(8192, 4096, "bf16") == "lds"
    assert smx.softmax_select_path(32768, 512, "f16") == "wave"
    assert smx.softmax_select_path(64, 1 << 20, "f32") == "split"
    assert smx.softmax_select_path(524288, 2048, "bf16") == "wave"


@pytest.mark.parametrize("path", ["auto", "wave", "lds", "split"])
def test_small_rows(path):
    w = W.small_rows()
    banner(f"small {path}")
    y = run_rows(w.x, "f32", w.mask, path=path, chunk_cols=256 if path == "split" else 0)
    r = check_full(w.x, "f32", w.mask, y, f"small/{path}")
    banner(f"small {path}: {r}")


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_fixed_rows(dtype):
    for w in W.fixed_rows():
        x = W.to_format(W.to_float(w.x, "f32").astype(np.float64), dtype)
        for path in ("auto", "split"):
            banner(f"{w.name} {dtype} {path}")
            y = run_rows(x, dtype, None, path=path, chunk_cols=2 if path == "split" else 0)
            check_full(x, dtype, None, y, f"{w.name}/{dtype}/{path}")
            assert np.isfinite(W.to_float(y, dtype)).all()


def test_worked_example_printed_values():
    """[20, 18, 17, -5] on the GPU reproduces the printed probabilities."""
    x = np.array([[20.0, 18.0, 17.0, -5.0]], dtype=np.float32)
    y = run_rows(x, "f32")
    assert np.allclose(y[0, :3], [0.84380, 0.11420, 0.04201], atol=1e-5)
    assert abs(y[0, 3] - 1.17e-11) <= 5e-14


@pytest.mark.parametrize("path", ["auto", "wave", "split"])
def test_spiked_rows_full(path):
    w = W.spiked_rows()
    banner(f"spiked {path}")
    y = run_rows(w.x, "bf16", w.mask, path=path)
    r = check_full(w.x, "bf16", w.mask, y, f"spiked/{path}")
    banner(f"spiked {path}: {r}")


@pytest.mark.parametrize("path", ["auto", "lds", "split"])
def test_masked_rows_full(path):
    w = W.masked_rows()
    banner(f"masked {path}")
    y = run_rows(w.x, "f16", w.mask, path=path)
    r = check_full(w.x, "f16", w.mask, y, f"masked/{path}")
    banner(f"masked {path}: {r}")


@pytest.mark.parametrize("path", ["auto", "split"])
def test_vocab_rows_full(path):
    """The vocabulary rows (4096 x 32768 bf16, 64 KiB each) at full size:
    resident in LDS on the automatic path, and through the split path."""
    w = W.vocab_rows()
    assert smx.softmax_select_path(w.rows, w.cols, w.dtype) == "lds"
    banner(f"vocab {path}")
    y = run_rows(w.x, "bf16", w.mask, path=path)
    r = check_full(w.x, "bf16", w.mask, y, f"vocab/{path}")
    banner(f"vocab {path}: {r}")


@pytest.mark.parametrize("chunk", [0, 4096, 100000])
def test_long_rows_full(chunk):
    w = W.long_rows()
    banner(f"long split chunk={chunk}")
    y = run_rows(w.x, "f32", w.mask, path="auto" if chunk == 0 else "split", chunk_cols=chunk)
    r = check_full(w.x, "f32", w.mask, y, f"long/chunk{chunk}")
    banner(f"long chunk={chunk}: {r}")


@pytest.mark.timeout(600)
def test_causal_scores_full():
    banner("causal generate")
    w = W.causal_scores()
    x = to_device(w.x, "bf16")
    banner("causal run")
    y = smx.softmax_rows(x, causal_period=w.mask.causal_period)
    torch.cuda.synchronize()
    del x
    y_raw = to_host(y, "bf16")
    del y
    banner("causal compare")
    n = 2048
    worst = 0
    for g in range(w.rows // n):
        r0, r1 = g * n, (g + 1) * n
        p, cls, st = oracle.softmax_rows(w.x, "bf16", w.mask, r0, r1)
        r = check(y_raw[r0:r1], "bf16", p, cls, st, f"causal/group{g}")
        worst = max(worst, r["max_ulp"])
    # the injected rows follow the declared policy
    nanrows = np.concatenate([w.special_rows["pos_inf_valid"], w.special_rows["nan_valid"]])
    assert (y_raw[nanrows] == 0x7FC0).all()
    assert (y_raw[w.special_rows["all_neg_inf"]] == 0).all()
    banner(f"causal: max ulp {worst}")


def test_very_long_rows_split():
    """Two fp32 rows of 2^26 lanes (256 MiB each): the automatic path is the
    split one with 32 KiB chunks, so each row's merge folds 8192 chunk
    summaries (32 per thread of the merging workgroup); the second row's
    valid length ends inside a chunk."""
    cols = 1 << 26
    x = W.random_rows(2, cols, "f32", seed=77, scale=4.0)
    mask = W.MaskSpec("valid_len", valid_len=np.array([cols, cols - 12345], dtype=np.int32))
    assert smx.softmax_select_path(2, cols, "f32") == "split"
    assert smx.softmax_default_chunk_cols(2, cols, "f32") == 8192
    banner("two rows of 2^26 lanes, split path")
    y = run_rows(x, "f32", mask)
    r = check_full(x, "f32", mask, y, "very long rows")
    banner(f"very long rows: {r}")


def test_row_merge_matches_direct_merge():
    """Beyond 1024 chunks per row the split path merges each row's summaries
    once before normalizing, and so does the public softmax_row_stats +
    softmax_merge_normalize pair (its summary reads then grow linearly with
    the chunk count): at 4096 chunks per row the pair is bitwise
    softmax_rows on the split path, and both meet the oracle; at 1024 chunks
    (every workgroup merging all of its row's summaries) and 1025 (merged
    once per row first) the pair meets the oracle too. Log-softmax,
    cross-entropy and the backward take the same two-level merge and meet
    the oracle. Rows: full, a valid length ending inside a chunk, empty, and
    NaN in a valid lane."""
    rows, cols, chunk = 4, 1 << 22, 1024  # 4096 chunks per row
    x = W.random_rows(rows, cols, "f32", seed=91, scale=5.0)
    x[3, 777_777] = np.float32("nan")
    vl = np.array([cols, cols - 1000, 0, cols], dtype=np.int32)
    mask = W.MaskSpec("valid_len", valid_len=vl)
    xd = to_device(x, "f32")
    kw = mask_kwargs(mask)
    banner("row merge: softmax")
    y_two = smx.softmax_rows(xd, path="split", chunk_cols=chunk, **kw)
    st = smx.softmax_row_stats(xd, chunk, **kw)
    y_direct = smx.softmax_merge_normalize(xd, st, chunk, **kw)
    torch.cuda.synchronize()
    assert _same_bits(y_two, y_direct)
    check_full(x, "f32", mask, to_host(y_two, "f32"), "row merge softmax")
    for ch in (cols // 1024, -(-cols // 1025)):  # 1024 and 1025 chunks per row
        banner(f"public stats + merge, {-(-cols // ch)} chunks per row")
        st = smx.softmax_row_stats(xd, ch, **kw)
        y_pub = smx.softmax_merge_normalize(xd, st, ch, **kw)
        torch.cuda.synchronize()
        check_full(x, "f32", mask, to_host(y_pub, "f32"), f"public merge {ch}")
    banner("row merge: log-softmax")
    y, lse = run_log(x, "f32", mask, path="split", chunk_cols=chunk)
    check_log_full(x, "f32", mask, y, lse, "row merge log-softmax")
    banner("row merge: cross-entropy")
    t = xent_targets(rows, cols, seed=93)
    loss, dx = run_xent(x, "f32", t, mask, path="split", chunk_cols=chunk)
    check_xent_full(x, "f32", t, mask, loss, dx, "row merge cross-entropy")
    banner("row merge: backward")
    p_raw, g_raw = bwd_inputs(x[:2], "f32", W.MaskSpec("valid_len", valid_len=vl[:2]), seed=92)
    dxb = run_bwd(p_raw, g_raw, "f32", path="split", chunk_cols=chunk)
    check_bwd_full(p_raw, g_raw, "f32", dxb, "row merge backward")


def test_beyond_2_31_elements():
    """Tensors of more than 2^31 elements, so element offsets pass 2^31 on
    every path (64-bit addressing): 2^20 + 512 rows of 2048 bf16 lanes
    through the wave, LDS and split paths, and the weighted sums over 520
    groups of 2048 x 2048 causal scores. Rows at both ends and on each side
    of element 2^31 are checked against the oracle."""
    rows, cols = (1 << 20) + 512, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(123)
    x = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    for r in range(0, rows, 1 << 18):
        x[r:r + (1 << 18)] = (6.0 * torch.randn(min(1 << 18, rows - r), cols, device="cuda", generator=g)).to(torch.bfloat16)
    edge = (1 << 31) // cols
    sample = [0, 1, rows // 2, edge - 1, edge, edge + 1, rows - 2, rows - 1]
    xs = to_host(x[sample].contiguous(), "bf16")
    p, cls, st = oracle.softmax_rows(xs, "bf16", W.MaskSpec("none"))
    for path, chunk in (("wave", 0), ("lds", 0), ("split", 512)):
        banner(f"2^31+: softmax {path}")
        y = smx.softmax_rows(x, path=path, chunk_cols=chunk)
        torch.cuda.synchronize()
        check(to_host(y[sample].contiguous(), "bf16"), "bf16", p, cls, st, f"2^31+ {path}")
        del y
    del x
    groups, n, d = 520, 2048, 128
    banner("2^31+: weighted sums")
    sc = torch.empty(groups * n, n, dtype=torch.bfloat16, device="cuda")
    for gi in range(0, groups, 64):
        k = min(64, groups - gi)
        sc[gi * n:(gi + k) * n] = (3.0 * torch.randn(k * n, n, device="cuda", generator=g)).to(torch.bfloat16)
    v = torch.randn(groups, n, d, device="cuda", generator=g).to(torch.bfloat16)
    out = smx.softmax_weighted_rows(sc, v, causal_period=n)
    torch.cuda.synchronize()
    mask = W.MaskSpec("causal", causal_period=n)
    for gi in (0, edge // n, edge // n + 1, groups - 1):
        s_g = to_host(sc[gi * n:(gi + 1) * n].contiguous(), "bf16")
        v_g = to_host(v[gi:gi + 1].contiguous().view(n, d), "bf16").reshape(1, n, d)
        rows_g = [0, 1, 777, n - 1]
        for r in rows_g:
            ref, st_w, scale = weighted_reference(s_g, v_g, "bf16", n, mask, r, r + 1)
            got = to_host(out[gi * n + r:gi * n + r + 1].contiguous(), "bf16")
            check_weighted(got, "bf16", ref, st_w, scale, f"2^31+ weighted group {gi} row {r}")


def test_row_slices_past_2_20_workgroups():
    """Launches split into slices of at most 2^20 workgroups: a causal mask's
    row index and the NaN policy must carry across the slice boundary.
    (1) 2^24 + 37 one-lane fp32 rows on the wave path (16 rows per
    workgroup: 2^20 + 3 workgroups, two slices); causal period 5, offset -1
    leaves rows r = 0 (mod 5) empty and every other row one valid lane, so
    every output is +0.0 or exactly 1.0 (the one-valid-lane special case),
    NaN rows aside. (2) 2^20 + 300 causal bf16 rows of 256 lanes on the LDS
    path (two slices), sampled rows on both sides of row 2^20 held to the
    oracle under their global row index."""
    banner("slices: wave path, 2^24 + 37 one-lane rows")
    rows = (1 << 24) + 37
    b = 1 << 24  # first row of the second slice
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = (4.0 * torch.randn(rows, 1, device="cuda", generator=g)).contiguous()
    nan_rows = [b - 2, b - 1, b, b + 1, b + 4, b + 5, rows - 1]  # b = 1 (mod 5): b - 1 and b + 4 are empty, their NaN masked
    x[nan_rows, 0] = float("nan")
    x[b + 2, 0] = float("inf")
    y = smx.softmax_rows(x, causal_period=5, causal_offset=-1, path="wave")
    torch.cuda.synchronize()
    got = y.view(torch.int32).cpu().numpy().reshape(-1).view(np.uint32)
    r = np.arange(rows)
    want = np.where(r % 5 == 0, np.uint32(0), np.uint32(0x3F800000))
    for q in nan_rows + [b + 2]:
        if q % 5 != 0:
            want[q] = 0x7FC00000
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:8]}: got {got[bad[:8]]}, want {want[bad[:8]]}"
    del x, y

    banner("slices: LDS path, 2^20 + 500 causal rows")
    rows, cols, period = (1 << 20) + 500, 256, 1000
    b = 1 << 20  # r mod 1000 = 576 at r = b: rows b - 2 ... b + 423 keep all 256 lanes
    x = (6.0 * torch.randn(rows, cols, device="cuda", generator=g)).to(torch.bfloat16)
    x[b - 1, 3] = float("nan")    # valid lane: NaN row
    x[b, 200] = float("nan")      # valid lane: NaN row
    x[b + 1, 5] = float("inf")    # valid lane: NaN row
    x[b + 424, 100] = float("nan")  # r mod 1000 = 0, one valid lane: the NaN is masked, p = (1, 0, ...)
    y = smx.softmax_rows(x, causal_period=period, path="lds")
    torch.cuda.synchronize()
    sample = [0, 1, 999, 1000, b - 3, b - 2, b - 1, b, b + 1, b + 2, b + 424, b + 425, rows - 2, rows - 1]
    vl = np.clip(np.array(sample) % period + 1, 0, cols).astype(np.int32)
    xs = to_host(x[sample].contiguous(), "bf16")
    p, cls, st = oracle.softmax_rows(xs, "bf16", W.MaskSpec("valid_len", valid_len=vl))
    check(to_host(y[sample].contiguous(), "bf16"), "bf16", p, cls, st, "LDS slices, causal")
    assert list(st[6:9]) == [oracle.ROW_POISON] * 3 and st[10] == oracle.ROW_OK

def test_stream_copy_is_exact():
    """The bandwidth reference copy moves every byte: sizes from one 16-byte
    pack through ragged multiples to the headline footprint, on the default
    and on a separate stream; from 1 GiB it copies 16 KiB per workgroup in
    the XCDs' contiguous order, with the grid padded to a multiple of 8 (the
    second large size leaves a ragged last chunk and padding workgroups)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    for nbytes in (16, 48, 4096 + 16, 1 << 20, (1 << 26) + 4080, 8192 * 4096 * 2, 1 << 30,
                   (1 << 30) + 3 * 16384 + 48):
        banner(f"stream copy {nbytes} B")
        x = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
        y = torch.full_like(x, 0x5A5A5A5A)
        guard = torch.full((1024,), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
        yy = torch.cat([y, guard])  # a guard zone after y: the copy writes nothing past its bytes
        smx.stream_copy(x, yy[:x.numel()])
        torch.cuda.synchronize()
        assert torch.equal(yy[:x.numel()], x)
        assert torch.equal(yy[x.numel():], guard)
    s = torch.cuda.Stream()
    x = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    with torch.cuda.stream(s):
        smx.stream_copy(x, y)
    s.synchronize()
    assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# Shapes, alignments, masks and paths
# ---------------------------------------------------------------------------

ODD_COLS = [1, 3, 7, 8, 63, 64, 65, 255, 511, 513, 1000, 2047, 2048, 2049, 4095, 4096, 4104, 8191, 8192, 16384, 16385, 33000]


def _masks(rows, cols, rng):
    valid = rng.integers(-2, cols + 3, rows).astype(np.int32)
    keep = (rng.random((rows, cols)) < 0.7).astype(np.uint8)
    return [W.MaskSpec(), W.MaskSpec("valid_len", valid_len=valid),
            W.MaskSpec("causal", causal_period=max(1, rows // 3), causal_offset=1),
            W.MaskSpec("keep", keep=keep)]


def _paths(dtype, cols, misalign):
    paths = ["auto", "split"]
    vec = not misalign and (cols * (4 if dtype == "f32" else 2)) % 16 == 0
    wave_max = 64 * 8 * (4 if dtype == "f32" else 8) if vec else 64 * 32
    if cols <= wave_max:
        paths.append("wave")
    if vec and cols * (4 if dtype == "f32" else 2) <= 152 * 1024:  # held in registers up to 32 KiB, then in LDS
        paths.append("lds")
    return paths


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_large_maxima_switch_the_exponential(dtype):
    """16-bit rows whose maximum reaches 2^15 in magnitude: the wave and LDS
    kernels fold the row's shift into one constant below that and subtract it
    explicitly at and above it; both sides of the switch, and rows around
    +-40000, on every path, held to the oracle."""
    rng = np.random.default_rng(77)
    rows, cols = 12, 1024
    a = np.empty((rows, cols))
    a[0::4] = 40000.0 + 100.0 * rng.standard_normal((3, cols))
    a[1::4] = -40000.0 + 100.0 * rng.standard_normal((3, cols))
    a[2::4] = 32768.0 - 16.0 * rng.integers(0, 4, (3, cols))  # maximum 2^15: explicit subtraction
    a[3::4] = 32752.0 - 16.0 * rng.integers(0, 4, (3, cols))  # maximum below 2^15 (f16): one constant
    x = W.to_format(a, dtype)
    p, cls, st = oracle.softmax_rows(x, dtype, W.MaskSpec())
    for path in ("wave", "lds", "split"):
        banner(f"{dtype} large maxima path={path}")
        y = run_rows(x, dtype, W.MaskSpec(), path=path, chunk_cols=256 if path == "split" else 0)
        check(y, dtype, p, cls, st, f"{dtype} large maxima path={path}")


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_ragged_long_rows_default_chunks(dtype):
    """Rows past the LDS budget that are not a whole number of the default
    chunk, through the automatic path (the split path at its default chunk
    width, so the last chunk of each row is partial): 16-byte multiples and
    odd lengths (no 128-bit accesses), each under every mask kind, with a
    +inf row and a NaN lane."""
    rng = np.random.default_rng(95)
    rows = 9 if dtype == "f32" else 17  # enough chunks for the full default width
    for cols in (1000032, 1000007):
        x = W.random_rows(rows, cols, dtype, seed=cols, scale=5.0)
        inf = W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype]
        W.set_bits(x, 1, cols // 2, dtype, inf)
        W.set_bits(x, 3, cols - 1, dtype, W.NEG_SNAN[dtype])
        assert smx.softmax_select_path(rows, cols, dtype) == "split"
        assert smx.softmax_default_chunk_cols(rows, cols, dtype) == 32768 // W.ITEMSIZE[dtype]
        for mask in _masks(rows, cols, rng):
            what = f"{dtype} ragged long rows cols={cols} mask={mask.kind} chunk={smx.softmax_default_chunk_cols(rows, cols, dtype)}"
            banner(what)
            y = run_rows(x, dtype, mask)
            check_full(x, dtype, mask, y, what)


def _beyond_2_31_rows(dtype):
    """Eight rows whose maxima are 2^31 to 3e38 in magnitude, each lane 0 to
    3 steps of the format below its row's maximum."""
    rng = np.random.default_rng(91)
    rows, cols = 8, 1024
    big = [2.0 ** 31, 2.0 ** 32, -2.0 ** 32, 1e30, -1e30, 3e38, 2.0 ** 40, -2.0 ** 31]
    step = 2.0 ** -21 if dtype == "f32" else 2.0 ** -6  # at least one step of the format
    a = np.empty((rows, cols))
    for r, b in enumerate(big):
        k = rng.integers(0, 4, cols)
        a[r] = b * (1.0 - step * k) if b > 0 else b * (1.0 + step * k)
    return W.to_format(a, dtype)


@pytest.mark.parametrize("op", ["softmax", "log", "xent"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_maxima_beyond_2_31(dtype, op):
    """Rows whose maximum is 2^31 or more in magnitude, where m - 160 rounds
    back to m in fp32: lanes one or more format steps below the maximum lie
    thousands below it and must give exactly 0 (not 1), and the lanes equal
    to the maximum share the row; the log-softmax's LSE is m + log(count) and
    the cross-entropy's loss m - x_t + log(count). Every path, the split path
    with several chunks per row (its stats pass serves all three)."""
    x = _beyond_2_31_rows(dtype)
    rows, cols = x.shape
    mask = W.MaskSpec()
    if op == "softmax":
        p, cls, st = oracle.softmax_rows(x, dtype, mask)
    t = W.class_targets(rows, cols, seed=92)
    for path in ("wave", "lds", "split"):
        chunk = 256 if path == "split" else 0
        what = f"{dtype} {op} maxima beyond 2^31 path={path}"
        banner(what)
        if op == "softmax":
            y = run_rows(x, dtype, mask, path=path, chunk_cols=chunk)
            check(y, dtype, p, cls, st, what)
        elif op == "log":
            y, lse = run_log(x, dtype, mask, path=path, chunk_cols=chunk)
            check_log_full(x, dtype, mask, y, lse, what)
        else:
            loss, dx = run_xent(x, dtype, t, mask, path=path, chunk_cols=chunk)
            check_xent_full(x, dtype, t, mask, loss, dx, what)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_odd_shapes_masks_paths(dtype):
    rng = np.random.default_rng(100)
    for cols in ODD_COLS:
        rows = 13
        x = W.random_rows(rows, cols, dtype, seed=cols, scale=12.0)
        for mask in _masks(rows, cols, rng):
            banner(f"{dtype} cols={cols} mask={mask.kind}")
            p, cls, st = oracle.softmax_rows(x, dtype, mask)
            for misalign in (False, True):
                for path in _paths(dtype, cols, misalign):
                    options = [c for c in (1, 5, 64, 200, 4096) if -(-cols // c) <= 512]
                    chunk = 0 if path != "split" else int(rng.choice(options))
                    what = f"{dtype} cols={cols} mask={mask.kind} misalign={misalign} path={path} chunk={chunk}"
                    y = run_rows(x, dtype, mask, path=path, chunk_cols=chunk, misalign=misalign)
                    check(y, dtype, p, cls, st, what)


# ---------------------------------------------------------------------------
# Rows above the register budget (32 KiB) up to 152 KiB: resident in LDS
# ---------------------------------------------------------------------------

RES_COLS = {"f32": [8196, 16384, 25132, 38912], "f16": [16392, 32768, 50264, 77824],
            "bf16": [16392, 32768, 50264, 65536, 77824]}
RES_MAX = {"f32": 38912, "f16": 77824, "bf16": 77824}


def _res_case(rng, dtype, rows, cols, mask_kind):
    """Seeded rows with policy rows (+inf in a valid lane, NaN in a lane
    that is masked or, without a mask, valid; all -inf) under a mask."""
    x = W.random_rows(rows, cols, dtype, seed=int(rng.integers(1 << 30)), scale=6.0)
    inf = W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype]
    W.set_bits(x, 2, 5, dtype, inf)
    W.set_bits(x, 3, cols - 1, dtype, W.NEG_SNAN[dtype])
    x[4] = W.to_format(np.full(cols, -np.inf), dtype)
    if mask_kind == "valid_len":
        vl = rng.integers(0, cols + 1, rows).astype(np.int32)
        vl[:6] = [cols, cols - 3, cols, cols - 1, cols, 0]
        return x, W.MaskSpec("valid_len", valid_len=vl)
    if mask_kind == "causal":
        return x, W.MaskSpec("causal", causal_period=rows, causal_offset=cols // 2 - rows // 2)
    if mask_kind == "keep":
        keep = (rng.random((rows, cols)) < 0.6).astype(np.uint8)
        keep[2, 5] = 1
        return x, W.MaskSpec("keep", keep=keep)
    return x, W.MaskSpec()


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_lds_resident_rows(dtype):
    """Rows past the register budget stay in LDS for all three passes: every
    dtype from just past 32 KiB to the 152 KiB maximum (ragged last pieces),
    every mask kind, the policy rows, and the log-softmax and cross-entropy
    epilogues, each against the oracle."""
    rng = np.random.default_rng(610 + W.DTYPES.index(dtype))
    kinds = ["none", "valid_len", "causal", "keep"]
    for i, cols in enumerate(RES_COLS[dtype]):
        kind = kinds[i % 4]
        x, mask = _res_case(rng, dtype, 37, cols, kind)
        what = f"lds-resident {dtype} 37x{cols} {kind}"
        banner(what)
        y = run_rows(x, dtype, mask, path="lds")
        check_full(x, dtype, mask, y, what)
        yl, lse = run_log(x, dtype, mask, path="lds")
        check_log_full(x, dtype, mask, yl, lse, what + " log-softmax")
        t = xent_targets(37, cols, seed=cols)
        t[7] = -1  # ignored
        t[8] = 3
        x8 = x.copy()
        x8[8] = W.to_format(np.where(np.arange(cols) == 3, 40.0, 1.0), dtype)  # a confident target
        loss, dx = run_xent(x8, dtype, t, mask, path="lds")
        check_xent_full(x8, dtype, t, mask, loss, dx, what + " cross-entropy")
    # one past the maximum is refused on the forced path and goes split on auto
    assert smx.softmax_select_path(4096, RES_MAX[dtype], dtype) == "lds"
    assert smx.softmax_select_path(4096, RES_MAX[dtype] + 16 // W.ITEMSIZE[dtype], dtype) == "split"
    xx = torch.zeros((2, RES_MAX[dtype] + 16 // W.ITEMSIZE[dtype]), dtype=TORCH_DTYPE[dtype], device="cuda")
    with pytest.raises(smx.SmxError):
        smx.softmax_rows(xx, path="lds")


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_lds_resident_many_rows_per_workgroup(dtype):
    """Workgroups stay resident and take several rows each, loading the next
    row while they normalize the current one: valid lengths that differ from
    row to row (empty rows, one lane, full rows) change how many pieces each
    wave loads and waits for between consecutive rows. The automatic path
    takes these rows, at the largest width and at a width two rows of which
    share a CU."""
    rng = np.random.default_rng(620 + W.DTYPES.index(dtype))
    for cols, rows in ((RES_MAX[dtype], 1100), (RES_MAX[dtype] // 2, 1500)):
        x = W.random_rows(rows, cols, dtype, seed=int(rng.integers(1 << 30)), scale=5.0)
        vl = rng.integers(0, cols + 1, rows).astype(np.int32)
        vl[rng.random(rows) < 0.1] = 0
        vl[rng.random(rows) < 0.1] = 1
        vl[rng.random(rows) < 0.2] = cols
        mask = W.MaskSpec("valid_len", valid_len=vl)
        assert smx.softmax_select_path(rows, cols, dtype) == "lds"
        what = f"lds-resident {dtype} {rows}x{cols} valid lengths"
        banner(what)
        y = run_rows(x, dtype, mask)
        check_full(x, dtype, mask, y, what)
        y2 = run_rows(x, dtype, mask)
        assert np.array_equal(y.view(np.uint8), y2.view(np.uint8)), "not deterministic"


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_policy_rows_bit_exact(dtype):
    cols = 40
    rows = 10
    base = W.to_format(np.linspace(-5, 5, cols)[None, :].repeat(rows, 0), dtype)
    x = base.copy()
    pinf = W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype]
    ninf = W.NEG_INF[dtype].view(np.uint32) if dtype == "f32" else W.NEG_INF[dtype]
    W.set_bits(x, 0, 3, dtype, pinf)                 # +inf valid -> NaN row
    W.set_bits(x, 1, 39, dtype, W.QNAN[dtype])        # NaN valid (last lane)
    W.set_bits(x, 2, 0, dtype, W.NEG_SNAN[dtype])     # -sNaN valid
    W.set_bits(x, 3, 30, dtype, W.QNAN[dtype])        # NaN masked -> ignored
    W.set_bits(x, 4, 35, dtype, pinf)                 # +inf masked -> ignored
    for j in range(cols):
        W.set_bits(x, 5, j, dtype, ninf)              # all -inf -> zero row
    for j in range(0, cols, 2):
        W.set_bits(x, 6, j, dtype, ninf)              # half -inf
    valid = np.array([40, 40, 40, 20, 20, 40, 40, 0, 1, 40], dtype=np.int32)  # row 7 empty
    mask = W.MaskSpec("valid_len", valid_len=valid)
    p, cls, st = oracle.softmax_rows(x, dtype, mask)
    assert list(st[:3]) == [oracle.ROW_POISON] * 3 and st[5] == st[7] == oracle.ROW_EMPTY
    for path in ("auto", "wave", "lds", "split"):
        if path == "lds" and (cols * (4 if dtype == "f32" else 2)) % 16:
            continue
        banner(f"policy {dtype} {path}")
        y = run_rows(x, dtype, mask, path=path, chunk_cols=7 if path == "split" else 0)
        check(y, dtype, p, cls, st, f"policy/{dtype}/{path}")
        assert float(W.to_float(y, dtype)[8, 0]) == 1.0  # one valid lane -> exactly 1


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_exact_special_cases(dtype):
    for k in (0, 5, 10, 12):
        n = 1 << k
        x = W.to_format(np.full((3, n), 2.5), dtype)
        for path in ("auto", "split"):
            y = W.to_float(run_rows(x, dtype, path=path), dtype)
            assert (y == np.float32(2.0 ** -k)).all(), (dtype, k, path)
    x = W.to_format(np.array([[-np.inf, 7.0, -np.inf, 7.0]]), dtype)
    y = W.to_float(run_rows(x, dtype), dtype)
    assert list(y[0]) == [0.0, 0.5, 0.0, 0.5]


def test_f32_exponential_sweep():
    """Rows [c, c + d, c + d/2, c - 7] with random offsets c (so x - m has a
    low-order part) and d swept over [-110, 0]: every output probes the fp32
    exponential, including results that are fp32 subnormals."""
    rng = np.random.default_rng(5)
    d = np.concatenate([-rng.uniform(0, 110, 30000), -np.linspace(0, 110, 2001)])
    c = rng.uniform(-50, 50, d.size)
    x = np.stack([c, c + d, c + d / 2, c - 7], 1).astype(np.float32)
    p, cls, st = oracle.softmax_rows(x, "f32")
    for path, chunk in (("wave", 0), ("lds", 0), ("split", 1), ("split", 2), ("split", 4)):
        banner(f"exp sweep {path} {chunk}")
        y = run_rows(x, "f32", path=path, chunk_cols=chunk)
        r = check(y, "f32", p, cls, st, f"exp sweep/{path}/{chunk}")
        banner(f"exp sweep {path} {chunk}: {r}")
    tiny = p[p > 0].min()
    assert tiny < 2.0 ** -126  # subnormal outputs are exercised


# ---------------------------------------------------------------------------
# The summary calls on their own
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", W.DTYPES)
def test_row_stats_against_oracle(dtype):
    rng = np.random.default_rng(7)
    rows, cols = 19, 5000
    x = W.random_rows(rows, cols, dtype, seed=3, scale=20.0)
    valid = rng.integers(0, cols + 1, rows).astype(np.int32)
    valid[0] = 0
    mask = W.MaskSpec("valid_len", valid_len=valid)
    W.set_bits(x, 1, 10, dtype, W.QNAN[dtype])
    tol = 2e-6 if dtype == "f32" else 2e-5
    for chunk in (1, 100, 1024, 4096, 5000, 9999):
        banner(f"stats {dtype} chunk={chunk}")
        st = smx.softmax_row_stats(to_device(x, dtype), chunk, **mask_kwargs(mask)).cpu().numpy()
        m, l = oracle.chunk_stats(x, dtype, chunk, mask)
        nan = np.isnan(m)
        assert np.array_equal(np.isnan(st[..., 0]), nan) and np.array_equal(np.isnan(st[..., 1]), nan)
        fin = ~nan
        assert np.array_equal(st[..., 0][fin], m[fin].astype(np.float32))  # the max is exact
        empty = fin & (m == -np.inf)
        assert (st[..., 1][empty] == 0).all()
        live = fin & ~empty
        rel = np.abs(st[..., 1][live] - l[live]) / l[live]
        assert rel.max() <= tol, rel.max()


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_merge_normalize_with_oracle_summaries(dtype):
    """Summaries computed by the oracle (then rounded to fp32) go into the
    library's merge/normalize; the oracle merges the same rounded summaries."""
    rng = np.random.default_rng(8)
    rows, cols, chunk = 11, 3000, 256
    x = W.random_rows(rows, cols, dtype, seed=4, scale=30.0)
    keep = (rng.random((rows, cols)) < 0.5).astype(np.uint8)
    keep[2] = 0
    mask = W.MaskSpec("keep", keep=keep)
    m, l = oracle.chunk_stats(x, dtype, chunk, mask)
    m32, l32 = m.astype(np.float32), l.astype(np.float32)
    st = torch.from_numpy(np.stack([m32, l32], axis=-1)).cuda()
    banner(f"merge_normalize {dtype}")
    y = smx.softmax_merge_normalize(to_device(x, dtype), st, chunk, **mask_kwargs(mask))
    torch.cuda.synchronize()
    p, cls, s = oracle.merge_normalize(x, dtype, m32.astype(np.float64), l32.astype(np.float64), mask)
    check(to_host(y, dtype), dtype, p, cls, s, f"merge_normalize/{dtype}")


def test_merge_normalize_external_summaries_policy():
    """Caller-made summaries: a NaN summary poisons its row, all-empty
    summaries give a zero row, (-inf, 0) is an identity."""
    x = W.to_format(np.zeros((3, 8)), "f32")
    st = np.array([[[0.0, 4.0], [-np.inf, 0.0]],
                   [[np.nan, np.nan], [0.0, 4.0]],
                   [[-np.inf, 0.0], [-np.inf, 0.0]]], dtype=np.float32)
    y = smx.softmax_merge_normalize(to_device(x, "f32"), torch.from_numpy(st).cuda(), 4)
    y = to_host(y, "f32")
    assert (y[0] == 0.25).all()
    assert (y[1].view(np.uint32) == 0x7FC00000).all()
    assert (y[2].view(np.uint32) == 0).all()


# ---------------------------------------------------------------------------
# Determinism, aliasing, streams and stray writes
# ---------------------------------------------------------------------------

def test_determinism_and_aliasing():
    w = W.spiked_rows(rows=512)
    x = to_device(w.x, "bf16")
    for path in ("auto", "wave", "split"):
        y1 = smx.softmax_rows(x, path=path)
        y2 = smx.softmax_rows(x, path=path)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), path
        z = x.clone()
        smx.softmax_rows(z, z, path=path)  # in place
        torch.cuda.synchronize()
        assert torch.equal(z.view(torch.int16), y1.view(torch.int16)), path


def test_no_stray_writes():
    rows, cols = 37, 2000
    x_raw = W.random_rows(rows, cols, "f32", seed=9)
    for path in ("auto", "wave", "lds", "split"):
        guard = 4096
        buf = torch.full((rows * cols + 2 * guard,), 123.0, device="cuda")
        y = buf[guard:guard + rows * cols].view(rows, cols)
        smx.softmax_rows(to_device(x_raw, "f32"), y, path=path)
        torch.cuda.synchronize()
        assert (buf[:guard] == 123.0).all() and (buf[-guard:] == 123.0).all(), path


def test_nondefault_stream():
    w = W.masked_rows(rows=1024)
    x = to_device(w.x, "f16")
    vl = torch.from_numpy(w.mask.valid_len).cuda()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = smx.softmax_rows(x, valid_len=vl)
    s.synchronize()
    check_full(w.x, "f16", w.mask, to_host(y, "f16"), "stream")


def _same_bits(a, b):
    a = a if isinstance(a, tuple) else (a,)
    b = b if isinstance(b, tuple) else (b,)
    return len(a) == len(b) and all(
        torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8)) for u, v in zip(a, b))


def _graph_cases():
    """(name, inputs(seed) -> tensors, call(*tensors)) for every entry point and
    path; the split paths allocate their stream-ordered workspace inside."""
    def rows(r, c, dt, scale):
        return lambda seed: [to_device(W.random_rows(r, c, dt, seed=seed, scale=scale), dt)]

    vl = torch.from_numpy(np.random.default_rng(3).integers(0, 513, 4096).astype(np.int32)).cuda()
    tgt = torch.from_numpy(W.class_targets(1024, 4096, 5)).cuda()

    vl40 = torch.from_numpy(np.random.default_rng(4).integers(0, 2049, 40).astype(np.int32)).cuda()

    def split_inputs(seed):
        rng = np.random.default_rng(seed)
        s = to_device(W.to_format(3.0 * rng.standard_normal((40, 2048)), "bf16"), "bf16")
        v = to_device(W.to_format(rng.standard_normal((40 * 2048, 128)), "bf16"), "bf16").view(40, 2048, 128)
        return [s, v]

    def weighted_inputs(seed):
        rng = np.random.default_rng(seed)
        s = to_device(W.to_format(3.0 * rng.standard_normal((256, 200)), "bf16"), "bf16")
        v = to_device(W.to_format(rng.standard_normal((2 * 200, 64)), "bf16"), "bf16").view(2, 200, 64)
        return [s, v]

    return [
        ("softmax, LDS path", rows(1024, 4096, "bf16", 8.0), lambda x: smx.softmax_rows(x)),
        ("softmax, wave path, valid lengths", rows(4096, 512, "f16", 30.0),
         lambda x: smx.softmax_rows(x, valid_len=vl)),
        ("softmax, split path", rows(8, 300000, "f32", 4.0),
         lambda x: smx.softmax_rows(x, path="split", chunk_cols=4096)),
        ("log-softmax, LDS path", rows(1024, 4096, "bf16", 8.0), lambda x: smx.log_softmax_rows(x)),
        ("cross-entropy, LDS path", rows(1024, 4096, "bf16", 8.0),
         lambda x: smx.softmax_cross_entropy_rows(x, tgt)),
        ("backward, split path", lambda seed: rows(8, 300000, "f32", 1.0)(seed) + rows(8, 300000, "f32", 1.0)(seed + 50),
         lambda p, g: smx.softmax_backward_rows(p, g, path="split", chunk_cols=4096)),
        ("weighted sums, causal", weighted_inputs,
         lambda s, v: smx.softmax_weighted_rows(s, v, causal_period=128)),
        ("weighted sums, key split (one row per group)", split_inputs,
         lambda s, v: smx.softmax_weighted_rows(s, v, valid_len=vl40)),
    ]


def test_graph_capture_replays():
    """Each call captured into a HIP graph and replayed with alternating inputs,
    with eager work and synchronizations between the replays: every replay
    equals the eager call on the same input bit for bit (the eager results are
    the ones the other tests hold to the oracle)."""
    for name, inputs, call in _graph_cases():
        banner(f"graph: {name}")
        a, b = inputs(1), inputs(2)
        static = [t.clone() for t in a]
        call(*static)  # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = call(*static)
        for rep, src in enumerate((a, b, a, b)):
            for dst, t in zip(static, src):
                dst.copy_(t)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ref = call(*[t.clone() for t in src])
            torch.cuda.synchronize()
            assert _same_bits(out, ref), f"{name}: replay {rep} differs from the eager call"
        del g


def test_two_streams_at_once():
    """Split-path calls in flight on two streams at once (each call's workspace
    is allocated in its own stream's order): every result equals the same call
    made alone, bit for bit."""
    xa = to_device(W.random_rows(8, 300000, "f32", seed=11, scale=4.0), "f32")
    xb = to_device(W.random_rows(8, 300000, "f32", seed=12, scale=4.0), "f32")
    ref_a = smx.softmax_rows(xa, path="split", chunk_cols=4096)
    ref_b = smx.log_softmax_rows(xb, path="split", chunk_cols=4096)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ya = smx.softmax_rows(xa, path="split", chunk_cols=4096)
        with torch.cuda.stream(s2):
            yb = smx.log_softmax_rows(xb, path="split", chunk_cols=4096)
        outs.append((ya, yb))
    s1.synchronize()
    s2.synchronize()
    for ya, yb in outs:
        assert _same_bits(ya, ref_a) and _same_bits(yb, ref_b)


def test_c_program_through_the_abi(tmp_path):
    """A plain C program (tests/csrc/abi_from_c.c) calls every entry point of
    include/smx.h on device buffers and a stream of its own, with no Python
    in between; its results meet the oracle at the same bars as the
    binding's, and an invalid call is rejected with a message."""
    import os
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(smx.LIB_PATH)
    exe = tmp_path / "abi_from_c"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{root}/include", f"{root}/tests/csrc/abi_from_c.c", "-L/opt/rocm/lib", "-lamdhip64",
                    f"-L{libdir}", "-lsmx", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                   check=True)
    rows, cols, wrows, wcols, d, rpg, chunk = 300, 1000, 256, 200, 64, 128, 96
    rng = np.random.default_rng(40)
    x = W.random_rows(rows, cols, "f32", seed=41, scale=6.0)
    vl = rng.integers(-2, cols + 3, rows).astype(np.int32)
    vl[:3] = [0, 1, cols]
    xb = W.random_rows(rows, cols, "bf16", seed=42, scale=8.0)
    tgt = rng.integers(-1, cols + 1, rows).astype(np.int32)
    g = W.random_rows(rows, cols, "f32", seed=43, scale=1.0)
    sc = W.to_format(3.0 * rng.standard_normal((wrows, wcols)), "bf16")
    v = W.to_format(rng.standard_normal((wrows // rpg, wcols, d)), "bf16")
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([rows, cols, wrows, wcols, d, rpg, chunk], dtype=np.int64).tobytes())
        for a in (x, vl, xb, tgt, g, sc, v):
            f.write(np.ascontiguousarray(a).tobytes())
    banner("C program through the ABI")
    r = subprocess.run([str(exe), str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "rejected:" in r.stdout and r.stdout.strip().endswith("ok"), r.stdout
    raw = open(outp, "rb").read()
    parts, off = [], 0
    for dt, count in ((np.float32, rows * cols), (np.float32, rows * cols), (np.uint16, rows * cols),
                      (np.float32, rows), (np.float32, rows), (np.uint16, rows * cols), (np.float32, rows * cols),
                      (np.uint16, wrows * d), (np.uint16, wrows * d)):
        nbytes = count * np.dtype(dt).itemsize
        parts.append(np.frombuffer(raw[off:off + nbytes], dtype=dt))
        off += nbytes
    assert off == len(raw)
    y, y2, logp, lse, loss, dxb, dx, o, o2 = parts
    mask = W.MaskSpec("valid_len", valid_len=vl)
    check_full(x, "f32", mask, y.reshape(rows, cols), "C: softmax_rows")
    check_full(x, "f32", mask, y2.reshape(rows, cols), "C: softmax_row_stats + softmax_merge_normalize")
    check_log_full(xb, "bf16", mask, logp.reshape(rows, cols), lse, "C: log_softmax_rows")
    check_xent_full(xb, "bf16", tgt, W.MaskSpec("none"), loss, dxb.reshape(rows, cols), "C: cross-entropy")
    check_bwd_full(y.reshape(rows, cols), g, "f32", dx.reshape(rows, cols), "C: softmax_backward_rows")
    ref, st, scale = weighted_reference(sc, v, "bf16", rpg, W.MaskSpec("causal", causal_period=rpg))
    check_weighted(o.reshape(wrows, d), "bf16", ref, st, scale, "C: softmax_weighted_rows")
    check_weighted(o2.reshape(wrows, d), "bf16", ref, st, scale, "C: softmax_weighted_states + softmax_weighted_merge")


def test_invalid_arguments_raise():
    x = torch.zeros(4, 8, device="cuda")
    with pytest.raises(smx.SmxError):
        smx.softmax_rows(x.view(-1)[1:29].view(4, 7), path="lds")  # misaligned rows
    with pytest.raises(smx.SmxError):
        smx.softmax_rows(torch.zeros(2, 5000, device="cuda"), path="wave")  # too long for registers
    with pytest.raises(smx.SmxError):
        smx.softmax_merge_normalize(x, torch.zeros(4, 3, 2, device="cuda"), 4)  # wrong n_chunks


# ---------------------------------------------------------------------------
# Log-softmax and log-sum-exp
# ---------------------------------------------------------------------------

from smx_compare import check_log  # noqa: E402


def run_log(x_raw, dtype, mask=None, path="auto", chunk_cols=0, want_y=True, misalign=False):
    rows, cols = x_raw.shape
    if misalign:
        buf = torch.empty(rows * cols + 1, dtype=TORCH_DTYPE[dtype], device="cuda")
        x = buf[1:].view(rows, cols)
        x.copy_(to_device(x_raw, dtype))
        ybuf = torch.empty(rows * cols + 1, dtype=TORCH_DTYPE[dtype], device="cuda")
        y = ybuf[1:].view(rows, cols)
    else:
        x = to_device(x_raw, dtype)
        y = torch.empty_like(x)
    y, lse = smx.log_softmax_rows(x, y if want_y else None, want_y=want_y, path=path, chunk_cols=chunk_cols,
                                  **mask_kwargs(mask))
    torch.cuda.synchronize()
    return (to_host(y, dtype) if want_y else None), lse.cpu().numpy()


def check_log_full(x_raw, dtype, mask, y, lse, what, r0=0, r1=None):
    r1 = x_raw.shape[0] if r1 is None else r1
    lse_ref, logp = oracle.log_softmax_rows(x_raw, dtype, mask, r0, r1)
    _, cls, st = oracle.softmax_rows(x_raw, dtype, mask, r0, r1)
    xf = W.to_float(x_raw[r0:r1], dtype)
    return check_log(None if y is None else y[r0:r1], dtype, logp, lse_ref, lse[r0:r1], cls, st, xf, what)


@pytest.mark.parametrize("cfg,path", [("small", "auto"), ("small", "wave"), ("small", "lds"), ("small", "split"), ("spiked", "auto"),
                                      ("spiked", "split"), ("masked", "auto"), ("masked", "split"), ("long", "auto"), ("vocab", "auto")])
def test_log_softmax_workloads(cfg, path):
    w = W.WORKLOADS[cfg]()
    banner(f"log {cfg} {path}")
    y, lse = run_log(w.x, w.dtype, w.mask, path=path)
    r = check_log_full(w.x, w.dtype, w.mask, y, lse, f"log {cfg}/{path}")
    banner(f"log {cfg} {path}: {r}")
    _, lse_only = run_log(w.x, w.dtype, w.mask, path=path, want_y=False)
    assert np.array_equal(lse_only.view(np.uint32), lse.view(np.uint32))  # LSE-only: the same bits


@pytest.mark.timeout(600)
def test_log_softmax_causal_scores():
    banner("log causal generate")
    w = W.causal_scores()
    banner("log causal run")
    y, lse = run_log(w.x, "bf16", w.mask)
    n = 2048
    groups = list(range(0, 256, 8))
    for g in groups:
        check_log_full(w.x, "bf16", w.mask, y, lse, f"log causal/group{g}", g * n, (g + 1) * n)
    nanrows = np.concatenate([w.special_rows["pos_inf_valid"], w.special_rows["nan_valid"]])
    assert (y[nanrows] == 0x7FC0).all() and np.isnan(lse[nanrows]).all()
    empty = w.special_rows["all_neg_inf"]
    assert (y[empty] == 0xFF80).all() and (lse[empty] == -np.inf).all()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_log_softmax_lse_precision_16bit(dtype):
    """A row of one maximum and 1000 equal lanes a little below it, shifted so
    that the log-sum-exp is near 0 (where its bar, 1e-6 absolute, is
    tightest): every lane's exponential then carries the same rounding, so
    nothing averages out, and an exponential good only to 16-bit precision
    (2.6e-6) misses the fp32 log-sum-exp by 1.3e-6. The difference chosen is
    one whose exponent argument, biased by 64, rounds furthest. Every path,
    the rows repeated with more columns."""
    x0, x1 = (-6.125, -6.9375) if dtype == "bf16" else (-6.671875, -6.91015625)
    for cols in (1001, 4096, 40000):
        rows = 4
        a = np.full((rows, cols), -np.inf)
        a[:, :1001] = x1
        a[:, 0] = x0
        a[1] = np.roll(a[1], 500)  # the maximum elsewhere in the row
        x = W.to_format(a, dtype)
        for path in _paths(dtype, cols, False):
            what = f"lse precision {dtype} cols={cols} {path}"
            banner(what)
            y, lse = run_log(x, dtype, None, path=path, chunk_cols=300 if path == "split" else 0)
            check_log_full(x, dtype, None, y, lse, what)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_log_softmax_odd_shapes_and_policy(dtype):
    rng = np.random.default_rng(200)
    for cols in (1, 7, 64, 513, 2048, 2049, 4096, 5000, 8192, 16384):
        rows = 11
        x = W.random_rows(rows, cols, dtype, seed=cols + 1, scale=30.0)
        W.set_bits(x, 2, 0, dtype, W.QNAN[dtype])
        for mask in _masks(rows, cols, rng):
            banner(f"log {dtype} cols={cols} mask={mask.kind}")
            for misalign in (False, True):
                for path in _paths(dtype, cols, misalign):
                    chunk = 0 if path != "split" else 64
                    y, lse = run_log(x, dtype, mask, path=path, chunk_cols=chunk, misalign=misalign)
                    check_log_full(x, dtype, mask, y, lse, f"log {dtype} cols={cols} {mask.kind} {path} {misalign}")


def test_log_softmax_matches_softmax_and_torch():
    """log_softmax agrees with torch.log_softmax in float64 on fp32 rows, and
    exp(log_softmax) with softmax_rows."""
    x = W.random_rows(64, 1000, "f32", seed=9, scale=20.0)
    y, lse = run_log(x, "f32")
    ref = torch.log_softmax(torch.from_numpy(x.astype(np.float64)), 1).numpy()
    assert np.allclose(y, ref, rtol=0, atol=1e-6 * max(1.0, np.abs(ref).max()))
    p = run_rows(x, "f32")
    assert np.allclose(np.exp(y.astype(np.float64)), p, rtol=2e-5, atol=1e-30)


# ---------------------------------------------------------------------------
# Softmax backward
# ---------------------------------------------------------------------------

from smx_compare import check_bwd  # noqa: E402


def bwd_inputs(x_raw, dtype, mask, seed):
    """p = the oracle's softmax of x in the element format; g seeded N(0, 1)."""
    p, cls, st = oracle.softmax_rows(x_raw, dtype, mask)
    p_raw = oracle.encode(p, dtype)
    g_raw = W.random_rows(x_raw.shape[0], x_raw.shape[1], dtype, seed=seed, scale=1.0)
    return p_raw, g_raw


def run_bwd(p_raw, g_raw, dtype, path="auto", chunk_cols=0, misalign=False, inplace=False):
    rows, cols = p_raw.shape
    if misalign:
        bufs = [torch.empty(rows * cols + 1, dtype=TORCH_DTYPE[dtype], device="cuda") for _ in range(3)]
        p, g, dx = (b[1:].view(rows, cols) for b in bufs)
        p.copy_(to_device(p_raw, dtype))
        g.copy_(to_device(g_raw, dtype))
    else:
        p, g = to_device(p_raw, dtype), to_device(g_raw, dtype)
        dx = g if inplace else torch.empty_like(p)
    smx.softmax_backward_rows(p, g, dx, path=path, chunk_cols=chunk_cols)
    torch.cuda.synchronize()
    return to_host(dx, dtype)


def check_bwd_full(p_raw, g_raw, dtype, dx, what):
    ref = oracle.softmax_backward_rows(p_raw, g_raw, dtype)
    return check_bwd(dx, dtype, ref, W.to_float(p_raw, dtype).astype(np.float64),
                     W.to_float(g_raw, dtype).astype(np.float64), what)


@pytest.mark.parametrize("cfg,path", [("small", "auto"), ("small", "wave"), ("small", "lds"), ("small", "split"), ("spiked", "auto"),
                                      ("spiked", "split"), ("masked", "auto"), ("long", "auto"), ("vocab", "auto")])
def test_backward_workloads(cfg, path):
    w = W.WORKLOADS[cfg]()
    p_raw, g_raw = bwd_inputs(w.x, w.dtype, w.mask, seed=100 + w.seed)
    banner(f"backward {cfg} {path}")
    dx = run_bwd(p_raw, g_raw, w.dtype, path=path)
    r = check_bwd_full(p_raw, g_raw, w.dtype, dx, f"backward {cfg}/{path}")
    banner(f"backward {cfg} {path}: {r}")


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_backward_odd_shapes(dtype):
    for cols in (1, 3, 64, 511, 512, 2048, 2049, 4096, 8192, 9000, 16384, 33000):
        rows = 9
        x = W.random_rows(rows, cols, dtype, seed=cols + 7, scale=10.0)
        p_raw, g_raw = bwd_inputs(x, dtype, None, seed=cols)
        if cols > 3:
            W.set_bits(g_raw, 4, 2, dtype, W.QNAN[dtype])  # a NaN gradient poisons its row
        for misalign in (False, True):
            for path in ("auto", "wave", "lds", "split"):
                vec = not misalign and (cols * (4 if dtype == "f32" else 2)) % 16 == 0
                e = (4 if dtype == "f32" else 8) if vec else 1
                if path == "wave" and cols > 64 * 8 * e:
                    continue
                if path == "lds" and cols > 256 * 8 * e:
                    continue
                what = f"backward {dtype} cols={cols} {path} misalign={misalign}"
                dx = run_bwd(p_raw, g_raw, dtype, path=path, chunk_cols=700 if path == "split" else 0,
                             misalign=misalign)
                check_bwd_full(p_raw, g_raw, dtype, dx, what)


def test_backward_in_place_and_deterministic():
    w = W.spiked_rows(rows=256)
    p_raw, g_raw = bwd_inputs(w.x, "bf16", w.mask, seed=3)
    a = run_bwd(p_raw, g_raw, "bf16")
    b = run_bwd(p_raw, g_raw, "bf16", inplace=True)
    assert np.array_equal(a, b)
    check_bwd_full(p_raw, g_raw, "bf16", a, "backward in place")


# ---------------------------------------------------------------------------
# Cross-entropy with logits
# ---------------------------------------------------------------------------

from smx_compare import check_xent  # noqa: E402


def xent_targets(rows, cols, seed):
    return W.class_targets(rows, cols, seed)


def run_xent(x_raw, dtype, target, mask=None, path="auto", chunk_cols=0, want_dx=True, inplace=False,
             misalign=False):
    rows, cols = x_raw.shape
    if misalign:
        buf = torch.empty(rows * cols + 1, dtype=TORCH_DTYPE[dtype], device="cuda")
        x = buf[1:].view(rows, cols)
        x.copy_(to_device(x_raw, dtype))
    else:
        x = to_device(x_raw, dtype)
    t = torch.from_numpy(np.ascontiguousarray(target, dtype=np.int32)).cuda()
    dx = x if inplace else None
    loss, g = smx.softmax_cross_entropy_rows(x, t, dx=dx, want_dx=want_dx, path=path, chunk_cols=chunk_cols,
                                             **mask_kwargs(mask))
    torch.cuda.synchronize()
    return loss.cpu().numpy(), (to_host(g, dtype) if want_dx else None)


def check_xent_full(x_raw, dtype, target, mask, loss, dx, what):
    lr, dref = oracle.cross_entropy_rows(x_raw, dtype, target, mask)
    return check_xent(loss, dx, dtype, lr, dref, W.to_float(x_raw, dtype), target, what)


@pytest.mark.parametrize("cfg,path", [("small", "auto"), ("small", "wave"), ("small", "lds"), ("small", "split"), ("spiked", "auto"),
                                      ("spiked", "split"), ("masked", "auto"), ("masked", "split"), ("long", "auto"), ("vocab", "auto")])
def test_cross_entropy_workloads(cfg, path):
    w = W.WORKLOADS[cfg]()
    t = xent_targets(w.rows, w.cols, seed=300 + w.seed)
    t[::17] = -1  # ignored rows
    banner(f"xent {cfg} {path}")
    loss, dx = run_xent(w.x, w.dtype, t, w.mask, path=path)
    r = check_xent_full(w.x, w.dtype, t, w.mask, loss, dx, f"xent {cfg}/{path}")
    banner(f"xent {cfg} {path}: {r}")
    loss2, _ = run_xent(w.x, w.dtype, t, w.mask, path=path, want_dx=False)
    assert np.array_equal(loss2.view(np.uint32), loss.view(np.uint32))  # loss alone: the same bits


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_cross_entropy_confident_and_policy(dtype):
    rng = np.random.default_rng(301)
    for cols in (2, 7, 64, 1000, 2048, 4096, 8192, 16384, 20000):
        rows = 12
        a = rng.standard_normal((rows, cols)) * 3
        t = rng.integers(0, cols, rows).astype(np.int32)
        a[np.arange(rows), t] = a.max(1) + 30.0  # p_t = 1 - O(e^-30): a tiny loss
        x = W.to_format(a, dtype)
        W.set_bits(x, 3, (int(t[3]) + 1) % cols, dtype, W.QNAN[dtype])  # poisoned row
        t[4] = -5
        t[5] = cols  # ignored rows
        valid = np.full(rows, cols, dtype=np.int32)
        valid[6] = 0  # empty row
        valid[7] = int(t[7])  # the target is masked
        mask = W.MaskSpec("valid_len", valid_len=valid)
        for misalign in (False, True):
            for path in _paths(dtype, cols, misalign):
                what = f"xent confident {dtype} cols={cols} {path} misalign={misalign}"
                banner(what)
                loss, dx = run_xent(x, dtype, t, mask, path=path, chunk_cols=300 if path == "split" else 0,
                                    misalign=misalign)
                check_xent_full(x, dtype, t, mask, loss, dx, what)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_cross_entropy_ignored_rows_holding_inf_or_nan(dtype):
    """An ignored row (target outside [0, cols)) has loss 0 and gradient +0.0
    even when a valid lane holds +inf or NaN: the ignore wins over the
    poison. Rows of every length class (wave, LDS, LDS-resident, split),
    aligned and not, next to a poisoned row that is not ignored."""
    rng = np.random.default_rng(303)
    inf = W.POS_INF[dtype].view(np.uint32) if dtype == "f32" else W.POS_INF[dtype]
    for cols in (7, 1000, 4096, 20000, 40000):
        rows = 6
        x = W.random_rows(rows, cols, dtype, seed=cols + 1, scale=4.0)
        t = rng.integers(0, cols, rows).astype(np.int32)
        W.set_bits(x, 0, cols // 2, dtype, inf)
        t[0] = -1  # ignored, +inf in a valid lane
        W.set_bits(x, 1, cols - 1, dtype, W.QNAN[dtype])
        t[1] = cols  # ignored, NaN in a valid lane
        W.set_bits(x, 2, 0, dtype, inf)  # poisoned, not ignored
        for misalign in (False, True):
            for path in _paths(dtype, cols, misalign):
                what = f"xent ignored+poisoned {dtype} cols={cols} {path} misalign={misalign}"
                banner(what)
                loss, dx = run_xent(x, dtype, t, None, path=path, chunk_cols=300 if path == "split" else 0,
                                    misalign=misalign)
                check_xent_full(x, dtype, t, None, loss, dx, what)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_cross_entropy_loss_precision_16bit(dtype):
    """16-bit logits whose target is the row's maximum: the loss is then
    log1p of the other lanes' share, held to 1e-6 relative (the fp32 loss's
    own bar, with no absolute floor), so the exponentials that sum those
    lanes must carry fp32 precision even though the inputs and the gradient
    are 16-bit. Short rows at large and small logit scales (where a few
    lanes a few units below the maximum make the whole loss) and longer ones,
    on every path that holds them."""
    rng = np.random.default_rng(304)
    cases = [(2, 4.0), (5, 0.5), (17, 4.0), (17, 30.0), (64, 8.0), (1000, 4.0), (20000, 4.0)]
    for cols, scale in cases:
        rows = 2048 if cols <= 64 else 64
        x = W.random_rows(rows, cols, dtype, seed=int(rng.integers(1 << 30)), scale=scale)
        t = np.argmax(W.to_float(x, dtype), axis=1).astype(np.int32)
        for path in _paths(dtype, cols, False):
            what = f"xent 16-bit loss {dtype} cols={cols} scale={scale} {path}"
            banner(what)
            loss, dx = run_xent(x, dtype, t, None, path=path, chunk_cols=300 if path == "split" else 0)
            check_xent_full(x, dtype, t, None, loss, dx, what)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cross_entropy_confident_rows_far_below(dtype):
    """Rows whose target holds the maximum (0) and whose other logits all lie
    95 to 115 below it (every other row: all exactly 100 below): the loss,
    log1p of the others' share, is made of terms whose unscaled merge factors
    e^(m - x_t) are subnormal fp32 numbers. A merge that applies such a
    factor before the 2^64 scale keeps only the subnormal spacing's absolute
    precision (a subnormal factor times a long row's sum, or one subnormal
    rounding per lane, all in one direction on equal lanes). The loss must
    still meet its 1e-6 bar (with the 2^-126 floor of the fp32 output), at
    widths that reach the wave, LDS, LDS-resident and split kernels."""
    rng = np.random.default_rng(317)
    for cols in (1000, 4096, 16384, 40000, 262144):
        rows = max(2, min(64, (1 << 22) // cols))
        vals = rng.uniform(-115.0, -95.0, size=(rows, cols))
        vals[::2] = -100.0
        t = rng.integers(0, cols, rows).astype(np.int32)
        vals[np.arange(rows), t] = 0.0
        x = oracle.encode(vals, dtype)
        for path in _paths(dtype, cols, False):
            what = f"xent confident far-below {dtype} cols={cols} {path}"
            banner(what)
            loss, dx = run_xent(x, dtype, t, None, path=path)
            check_xent_full(x, dtype, t, None, loss, dx, what)


def test_cross_entropy_lane_reference_below_the_cutoff():
    """LDS-resident rows keep each lane's sum against a reference that moves
    only when the lane maximum passes it by more than 8, and bring the sum to
    the lane's maximum once per row before the merge, whose factor drops
    lanes more than 120 below the row maximum. Here every lane's first packs
    lie at -120.0625 (below that cutoff) and its later ones at -112.0625
    (within 8 of the first, so the reference never moves), with the target
    at the row maximum 0: the loss, about 1.5e-44, is made of the later
    packs and exceeds its absolute floor (1e-6 of 2^-126), so a merge that
    took the factor from the reference would return 0 and fail. f16 rows of
    77,824 logits (152 KiB, the LDS-resident kernel's largest)."""
    rows, cols = 8, 77824
    vals = np.full((rows, cols), -112.0625)
    vals[:, :8192] = -120.0625  # the first 16 KiB: every lane's first packs
    t = np.array([0, 1, 4095, 8191, 100, 3, 7, 2], dtype=np.int32)
    vals[np.arange(rows), t] = 0.0
    x = oracle.encode(vals, "f16")
    for path in ("auto", "lds"):
        what = f"xent lane reference below the cutoff f16 {path}"
        banner(what)
        loss, dx = run_xent(x, "f16", t, None, path=path)
        check_xent_full(x, "f16", t, None, loss, dx, what)
        assert (loss > 0).all(), f"{what}: {loss}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cross_entropy_split_chunks_narrower_than_a_round(dtype):
    """Split path with chunks far narrower than one register round of the
    normalize pass: each target's gradient is written by the workgroup of
    its own chunk (a round reaching into the next chunk must not write it),
    targets in late chunks included; guard zones around dx stay untouched."""
    rows, cols, chunk = 6, 5000, 100
    x_raw = W.random_rows(rows, cols, dtype, seed=31, scale=5.0)
    t = np.array([0, 150, 199, 4999, 2531, 100], dtype=np.int32)
    guard = 4096
    buf = torch.full((rows * cols + 2 * guard,), 77.0, dtype=TORCH_DTYPE[dtype], device="cuda")
    dx = buf[guard:guard + rows * cols].view(rows, cols)
    x = to_device(x_raw, dtype)
    loss, _ = smx.softmax_cross_entropy_rows(x, torch.from_numpy(t).cuda(), dx=dx, path="split", chunk_cols=chunk)
    torch.cuda.synchronize()
    assert bool((buf[:guard] == 77.0).all()) and bool((buf[-guard:] == 77.0).all())
    check_xent_full(x_raw, dtype, t, None, loss.cpu().numpy(), to_host(dx, dtype), f"xent narrow chunks {dtype}")


def test_cross_entropy_in_place():
    w = W.long_rows(rows=4, cols=1 << 16)
    t = xent_targets(4, 1 << 16, seed=9)
    for path in ("split", "auto"):
        loss, dx = run_xent(w.x, "f32", t, path=path)
        loss2, dx2 = run_xent(w.x, "f32", t, path=path, inplace=True)
        assert np.array_equal(loss, loss2) and np.array_equal(dx, dx2)
    w = W.spiked_rows(rows=64)
    t = xent_targets(64, 4096, seed=10)
    loss, dx = run_xent(w.x, "bf16", t)
    loss2, dx2 = run_xent(w.x, "bf16", t, inplace=True)
    assert np.array_equal(loss, loss2) and np.array_equal(dx, dx2)
    check_xent_full(w.x, "bf16", t, w.mask, loss, dx, "xent in place")


# ---------------------------------------------------------------------------
# Softmax-weighted value sums: out[r] = softmax(s[r]) @ V[r // rows_per_group]
# ---------------------------------------------------------------------------

from smx_compare import check_weighted  # noqa: E402


def run_weighted(s_raw, v_raw, dtype, mask=None):
    rows, cols = s_raw.shape
    s = to_device(s_raw, dtype)
    v = to_device(v_raw.reshape(-1, v_raw.shape[-1]), dtype).view(v_raw.shape)
    out = smx.softmax_weighted_rows(s, v, **mask_kwargs(mask))
    torch.cuda.synchronize()
    return to_host(out, dtype)


def abs_bits(v_raw, dtype):
    return (v_raw & np.uint16(0x7FFF)).astype(np.uint16)


def weighted_reference(s_raw, v_raw, dtype, rpg, mask, r0=0, r1=None):
    ref, st = oracle.softmax_weighted_rows(s_raw, v_raw, dtype, rpg, mask, r0, r1)
    scale, _ = oracle.softmax_weighted_rows(s_raw, abs_bits(v_raw, dtype), dtype, rpg, mask, r0, r1)
    return ref, st, scale


def _weighted_case(rng, dtype, rows_per_group, groups, cols, d, mask_kind):
    rows = rows_per_group * groups
    s = W.to_format(3.0 * rng.standard_normal((rows, cols)), dtype)
    v = W.to_format(rng.standard_normal((groups, cols, d)), dtype)
    if mask_kind == "none":
        mask = W.MaskSpec("none")
    elif mask_kind == "causal":
        mask = W.MaskSpec("causal", causal_period=rows_per_group, causal_offset=3)
    elif mask_kind == "valid_len":
        vl = rng.integers(0, cols + 1, rows).astype(np.int32)
        vl[:3] = [0, 1, cols]
        mask = W.MaskSpec("valid_len", valid_len=vl)
    else:
        mask = W.MaskSpec("keep", keep=(rng.random((rows, cols)) < 0.7).astype(np.uint8))
    # policy rows: NaN / +inf in a valid lane, NaN in a masked lane, all -inf
    W.set_bits(s, 5, 0, dtype, W.QNAN[dtype])
    W.set_bits(s, 6, 1, dtype, W.POS_INF[dtype])
    s[7, :] = W.NEG_INF[dtype]
    return s, v, mask


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_weighted_rows_small(dtype, d):
    rng = np.random.default_rng(500 + d)
    for mask_kind in ("none", "causal", "valid_len", "keep"):
        # 130 rows per group: a second, two-row tile; 200 columns: three full
        # blocks of 64 and a ragged one
        s, v, mask = _weighted_case(rng, dtype, 130, 2, 200, d, mask_kind)
        what = f"weighted {dtype} d={d} {mask_kind}"
        banner(what)
        out = run_weighted(s, v, dtype, mask)
        ref, st, scale = weighted_reference(s, v, dtype, 130, mask)
        res = check_weighted(out, dtype, ref, st, scale, what)
        banner(f"{what}: {res}")


# Key-split weighted sums: per-(row, chunk) states (m, l, o) and their merge.
STATE_TOL = 4e-6  # relative, on l and (against sum |w v|) on o; derived in DESIGN


def _split_case(rng, dtype, rpg, groups, cols, d, mask_kind):
    rows = rpg * groups
    s = W.to_format(3.0 * rng.standard_normal((rows, cols)), dtype)
    v = W.to_format(rng.standard_normal((groups, cols, d)), dtype)
    if mask_kind == "none":
        mask = W.MaskSpec("none")
    elif mask_kind == "causal":
        mask = W.MaskSpec("causal", causal_period=rpg, causal_offset=cols // 2)
    elif mask_kind == "valid_len":
        vl = rng.integers(0, cols + 1, rows).astype(np.int32)
        vl[0] = 0
        mask = W.MaskSpec("valid_len", valid_len=vl)
    else:
        mask = W.MaskSpec("keep", keep=(rng.random((rows, cols)) < 0.7).astype(np.uint8))
    if rows >= 4:  # policy rows: NaN and +inf in a valid lane, all -inf
        W.set_bits(s, 1, 5, dtype, W.QNAN[dtype])
        W.set_bits(s, 2, cols - 1, dtype, W.POS_INF[dtype])
        s[3, :] = W.NEG_INF[dtype]
    return s, v, mask


def _check_states(ml, o, s, v, dtype, rpg, chunk, mask, what):
    m_ref, l_ref, o_ref = oracle.weighted_chunk_states(s, v, dtype, rpg, chunk, mask)
    _, _, o_abs = oracle.weighted_chunk_states(s, abs_bits(v, dtype), dtype, rpg, chunk, mask)
    m_g = ml[..., 0].astype(np.float64)
    l_g = ml[..., 1].astype(np.float64)
    o_g = o.astype(np.float64)
    pois = np.isnan(m_ref)
    empty = m_ref == -np.inf
    live = ~pois & ~empty
    assert np.isnan(m_g[pois]).all() and np.isnan(l_g[pois]).all() and np.isnan(o_g[pois]).all(), what
    assert (m_g[empty] == -np.inf).all() and (l_g[empty] == 0).all() and (o_g[empty] == 0).all(), what
    assert np.array_equal(m_g[live], m_ref[live]), f"{what}: m is the exact chunk maximum"
    rel = np.abs(l_g[live] - l_ref[live]) / l_ref[live]
    assert rel.max(initial=0) <= STATE_TOL, f"{what}: l off by {rel.max():.3e}"
    err = np.abs(o_g[live] - o_ref[live])
    bound = STATE_TOL * o_abs[live] + 1e-30
    assert (err <= bound).all(), f"{what}: o off by {(err / bound).max():.3f} of the bound"
    return int(live.sum())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_weighted_states_and_merge(dtype, d):
    """States against the oracle's chunk states, then the merge of the GPU
    states and of the oracle's (rounded to fp32) against the oracle's direct
    weighted sums, over ragged chunks, every mask kind and policy rows."""
    rng = np.random.default_rng(700 + d)
    for rpg, groups, cols, chunk in ((1, 9, 2056, 512), (3, 3, 200, 64), (8, 2, 4096, 2048), (4, 2, 1000, 300)):
        for mask_kind in ("none", "causal", "valid_len", "keep"):
            s, v, mask = _split_case(rng, dtype, rpg, groups, cols, d, mask_kind)
            what = f"states {dtype} d={d} rpg={rpg} cols={cols} chunk={chunk} {mask_kind}"
            banner(what)
            sd = to_device(s, dtype)
            vd = to_device(v.reshape(-1, d), dtype).view(groups, cols, d)
            ml, o = smx.softmax_weighted_states(sd, vd, chunk, **mask_kwargs(mask))
            torch.cuda.synchronize()
            _check_states(ml.cpu().numpy(), o.cpu().numpy(), s, v, dtype, rpg, chunk, mask, what)
            ref, st, scale = weighted_reference(s, v, dtype, rpg, mask)
            out = smx.softmax_weighted_merge(ml, o, TORCH_DTYPE[dtype])
            torch.cuda.synchronize()
            check_weighted(to_host(out, dtype), dtype, ref, st, scale, what + " merged")
            # the merge alone, fed with the oracle's states
            m_ref, l_ref, o_ref = oracle.weighted_chunk_states(s, v, dtype, rpg, chunk, mask)
            ml_o = torch.from_numpy(np.stack([m_ref, l_ref], -1).astype(np.float32)).cuda()
            o_o = torch.from_numpy(o_ref.astype(np.float32)).cuda()
            out2 = smx.softmax_weighted_merge(ml_o, o_o, TORCH_DTYPE[dtype])
            torch.cuda.synchronize()
            check_weighted(to_host(out2, dtype), dtype, ref, st, scale, what + " merge of oracle states")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_weighted_rows_few_rows_per_group(dtype):
    """Groups of at most 4 rows (8 when there are few groups) take the key
    split inside softmax_weighted_rows (states in a workspace, then the
    merge): the fused call meets the oracle for 1, 3 and 8 rows per group;
    constant values come back exactly."""
    rng = np.random.default_rng(720)
    for rpg, groups, cols, d in ((1, 40, 2048, 128), (3, 7, 200, 64), (8, 5, 4104, 32)):
        for mask_kind in ("none", "causal", "valid_len", "keep"):
            s, v, mask = _split_case(rng, dtype, rpg, groups, cols, d, mask_kind)
            what = f"weighted split {dtype} rpg={rpg} cols={cols} d={d} {mask_kind}"
            banner(what)
            out = run_weighted(s, v, dtype, mask)
            ref, st, scale = weighted_reference(s, v, dtype, rpg, mask)
            check_weighted(out, dtype, ref, st, scale, what)
    s = W.to_format(4.0 * rng.standard_normal((6, 512)), dtype)
    c = W.to_format(rng.standard_normal(64), dtype)
    vc = np.broadcast_to(c, (2, 512, 64)).copy()
    out = run_weighted(s, vc, dtype)
    assert np.array_equal(out, np.broadcast_to(c, (6, 64))), f"weighted split constant {dtype}"


def test_weighted_rows_key_split_past_its_merge_width():
    """One row per group over 8,388,616 keys: at the key split's usual
    512-key chunk a row would leave 16,385 states, one more than the merge
    folds, so the chunk grows (to 1024 keys) and the sums still match the
    oracle."""
    rng = np.random.default_rng(515)
    dtype, groups, cols, d = "bf16", 2, 8_388_616, 32
    s = W.to_format(3.0 * rng.standard_normal((groups, cols), dtype=np.float32), dtype)
    v = W.to_format(rng.standard_normal((groups, cols, d), dtype=np.float32), dtype)
    mask = W.MaskSpec("none")
    banner(f"weighted key split {groups} x {cols} d={d}")
    out = run_weighted(s, v, dtype, mask)
    ref, st, scale = weighted_reference(s, v, dtype, 1, mask)
    check_weighted(out, dtype, ref, st, scale, "weighted key split past its merge width")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_weighted_rows_special_values(dtype):
    rng = np.random.default_rng(510)
    rows, cols = 128, 64
    s = W.to_format(4.0 * rng.standard_normal((rows, cols)), dtype)
    # one-hot values (V = I): the output is the softmax itself
    eye = W.to_format(np.eye(cols)[None], dtype)
    out = run_weighted(s, eye, dtype)
    p, cls, st = oracle.softmax_rows(s, dtype)
    ref, st2, scale = weighted_reference(s, eye, dtype, rows, None)
    assert np.array_equal(st, st2)
    check_weighted(out, dtype, ref, st2, scale, f"weighted one-hot {dtype}")
    # constant values: every row returns the constant exactly
    c = W.to_format(rng.standard_normal(32), dtype)
    vc = np.broadcast_to(c, (1, cols, 32)).copy()
    out = run_weighted(s, vc, dtype)
    assert np.array_equal(out, np.broadcast_to(c, (rows, 32))), f"weighted constant {dtype}"
    # a single valid lane returns that lane's value row
    vl = np.full(rows, 1, dtype=np.int32)
    v = W.to_format(rng.standard_normal((1, cols, 64)), dtype)
    out = run_weighted(s, v, dtype, W.MaskSpec("valid_len", valid_len=vl))
    assert np.array_equal(out, np.broadcast_to(v[0, 0], (rows, 64))), f"weighted single lane {dtype}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_weighted_rows_reference_paths(dtype):
    """The slow paths of the running reference, against the oracle: rows whose
    maximum climbs by 20 at every 64-column block (beyond either slack, so
    the state is rescaled at every block), rows offset by +40000 and by
    -40000 (references beyond 2^15 in magnitude are subtracted explicitly),
    rows whose first third is -inf (the reference starts late); with one
    row per group, a single ragged block of 8 columns, and several tiles."""
    rng = np.random.default_rng(530)
    for rpg, groups, cols, d in ((130, 2, 200, 128), (1, 40, 72, 64), (64, 2, 8, 32)):
        rows = rpg * groups
        x = rng.standard_normal((rows, cols))
        j = np.arange(cols)
        x[0::4] += 20.0 * (j // 64)
        x[1::4] = 40000.0 + 100.0 * x[1::4]  # distinct values at the coarse spacing there
        x[2::4] = -40000.0 + 100.0 * x[2::4]
        s = W.to_format(x, dtype)
        s[3::4, : cols // 3] = W.NEG_INF[dtype]
        v = W.to_format(rng.standard_normal((groups, cols, d)), dtype)
        what = f"weighted reference paths {dtype} rpg={rpg} cols={cols} d={d}"
        banner(what)
        out = run_weighted(s, v, dtype, W.MaskSpec("none"))
        ref, st, scale = weighted_reference(s, v, dtype, rpg, None)
        res = check_weighted(out, dtype, ref, st, scale, what)
        banner(f"{what}: {res}")


def _step16(v: float, dtype: str, up: bool) -> float:
    """The neighbour of v (a value of the 16-bit format) above it (up) or below it."""
    if dtype == "f16":
        return float(np.nextafter(np.float16(v), np.float16(np.inf if up else -np.inf)))
    bits = int(np.array([v], dtype=np.float32).view(np.uint32)[0]) >> 16
    bits += 1 if (v >= 0) == up else -1
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_weighted_rows_reference_moves_at_large_maxima(dtype):
    """Rows whose maximum lies between 2^8 and 2^13 in magnitude (below the
    explicit-subtraction threshold) and moves past the slack once, in the
    last block, after as many columns at the old maximum as make the terms
    before and after the move weigh the same; the values are +1 before the
    move and -1 at it, so the output is near 0 and any disagreement between
    the rescaling of the earlier terms and the constants their weights were
    formed with shows in full (a relative mismatch e gives an error of about
    e / 2 against a sum of |weight x value| of 1). Rows of 256 columns in
    fp16; bf16's coarser spacing makes every move there at least 10, so its
    rows are long (165,000 columns)."""
    rpg, groups, d = 16, 2, 64
    cols = 256 if dtype == "f16" else 165_000
    slack = 2.0 if dtype == "f16" else 8.0
    rows = rpg * groups
    bases = ([600.0, 1000.0, 1500.0, 2500.0, 3000.0, 5000.0, 6000.0, 7000.0] if dtype == "f16"
             else [300.0, 400.0, 500.0, 600.0, 700.0, 800.0, 900.0, 1000.0])
    top_col = cols - 6
    x = np.empty((rows, cols))
    for r in range(rows):
        b0 = bases[r % len(bases)] * (1.0 if (r // len(bases)) % 2 == 0 else -1.0)
        base = float(oracle.decode(W.to_format(np.array([b0]), dtype), dtype)[0])
        top = base
        while top <= base + slack:
            top = _step16(top, dtype, up=True)
        n_old = int(round(np.exp(top - base)))
        assert 1 <= n_old < top_col - 64  # the move lands in a later block than every earlier term
        x[r] = float(oracle.decode(W.to_format(np.array([base - 100.0]), dtype), dtype)[0])  # weight ~e^-100
        x[r, :n_old] = base
        x[r, top_col] = top
    s = W.to_format(x, dtype)
    vrow = np.full(cols, 0.25)
    vrow[: top_col - 64] = 1.0
    vrow[top_col] = -1.0
    v = W.to_format(np.broadcast_to(vrow[None, :, None], (groups, cols, d)).copy(), dtype)
    what = f"weighted reference moves at large maxima {dtype} cols={cols}"
    banner(what)
    out = run_weighted(s, v, dtype, W.MaskSpec("none"))
    ref, st, scale = weighted_reference(s, v, dtype, rpg, None)
    res = check_weighted(out, dtype, ref, st, scale, what)
    banner(f"{what}: {res}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_weighted_rows_few_columns(dtype):
    """The matrix-core path on rows of one 16-byte chunk up to one chunk past
    a block (columns are a multiple of 8): 8, 16, 56, 64 and 72 columns (the
    value rows past the end re-read the last one with weight 0), 16 and 129
    rows per group, with the policy rows, and causal and valid-length
    masks."""
    rng = np.random.default_rng(560)
    for cols in (8, 16, 56, 64, 72):
        for rpg, mask_kind in ((16, "none"), (129, "causal"), (16, "valid_len")):
            s, v, mask = _weighted_case(rng, dtype, rpg, 3, cols, 32, mask_kind)
            what = f"weighted few columns {dtype} cols={cols} rpg={rpg} {mask_kind}"
            out = run_weighted(s, v, dtype, mask)
            ref, st, scale = weighted_reference(s, v, dtype, rpg, mask)
            check_weighted(out, dtype, ref, st, scale, what)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_weighted_rows_output_8_byte_aligned(dtype):
    """An output 8 bytes off a 16-byte boundary (the least alignment the
    call takes) is written by the kernel's 8-byte stores instead of its
    16-byte ones: bitwise the same values as an aligned output, for every
    value width, with the policy rows."""
    rng = np.random.default_rng(570)
    for d in (32, 64, 128):
        s, v, mask = _weighted_case(rng, dtype, 130, 2, 200, d, "causal")
        sd = to_device(s, dtype)
        vd = to_device(v.reshape(-1, d), dtype).view(v.shape)
        aligned = smx.softmax_weighted_rows(sd, vd, **mask_kwargs(mask))
        buf = torch.full((s.shape[0] * d + 4,), 3.0, dtype=TORCH_DTYPE[dtype], device="cuda")
        off = buf[4:].view(s.shape[0], d)
        assert off.data_ptr() % 16 == 8
        smx.softmax_weighted_rows(sd, vd, off, **mask_kwargs(mask))
        torch.cuda.synchronize()
        assert torch.equal(off.view(torch.int16), aligned.view(torch.int16)), f"d={d}"
        assert (buf[:4] == 3.0).all(), "no write before the output"
        ref, st, scale = weighted_reference(s, v, dtype, 130, mask)
        check_weighted(to_host(off, dtype), dtype, ref, st, scale, f"weighted 8-byte-aligned out {dtype} d={d}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_weighted_rows_switch_to_explicit_form(dtype):
    """A wave turns to the explicit subtraction in the middle of its tile:
    one row in every 32 (one per wave) jumps past 2^15 (to 40000) at column
    256, while the other rows hold one value throughout (20272 in fp16,
    21248 in bf16: values whose exponent constant, rounded once, is off from
    the exact one by nearly 2^-10, the most in that range). Their state is
    carried over to the explicit form at the switch; with values +1 before
    column 256 and -1 from it on, the two halves of the row cancel, so an
    error in that conversion (a relative 6.6e-4 if it were left out) shows
    in full against the oracle. Rows whose reference starts at -40000 and
    climbs to 0 (the explicit form throughout) ride along."""
    rpg, groups, cols, d, cut = 128, 2, 512, 64, 256
    rows = rpg * groups
    x = np.full((rows, cols), 20272.0 if dtype == "f16" else 21248.0)
    x[7::32, cut:] = 40000.0
    x[19::64, : cut - 128] = -40000.0
    x[19::64, cut - 128 :] = 0.0
    s = W.to_format(x, dtype)
    vrow = np.where(np.arange(cols) < cut, 1.0, -1.0)
    v = W.to_format(np.broadcast_to(vrow[None, :, None], (groups, cols, d)).copy(), dtype)
    what = f"weighted switch to the explicit form {dtype}"
    banner(what)
    out = run_weighted(s, v, dtype, W.MaskSpec("none"))
    ref, st, scale = weighted_reference(s, v, dtype, rpg, None)
    res = check_weighted(out, dtype, ref, st, scale, what)
    banner(f"{what}: {res}")


def test_weighted_rows_causal_full():
    """The attention workload at full size: 256 groups of 2048 x 2048
    bf16 causal scores (with their injected policy rows) and per group 2048
    value vectors of width 128. Every policy row is checked in every group;
    every row of four whole groups is checked against the oracle (the first
    and last groups and two in between: the kernel hands the 16 row tiles of
    a group to one XCD, so workgroup b takes tile (b mod 8) * 512 + b / 8
    and these groups land on different XCDs and workgroup ranges), and a
    sample of the others (the first, the last and 6 random rows of every
    8th group)."""
    banner("weighted causal generate")
    w = W.causal_scores()
    v = W.causal_values()
    banner("weighted causal run")
    out = run_weighted(w.x, v, "bf16", w.mask)
    n = 2048
    banner("weighted causal policy rows")
    for name, rows in w.special_rows.items():
        sub = out[rows]
        if name in ("pos_inf_valid", "nan_valid"):
            assert (sub == 0x7FC0).all(), name
        elif name == "all_neg_inf":
            assert (sub == 0).all(), name
    worst = 0
    for g in (0, 37, 130, 255):
        banner(f"weighted causal: every row of group {g}")
        ref, st, scale = weighted_reference(w.x, v, "bf16", n, w.mask, g * n, (g + 1) * n)
        res = check_weighted(out[g * n:(g + 1) * n], "bf16", ref, st, scale, f"weighted causal group {g}")
        worst = max(worst, res.get("max_ulp", 0))
    banner("weighted causal sampled rows")
    rng = np.random.default_rng(520)
    for g in range(0, 256, 8):
        picks = sorted({g * n, g * n + n - 1, *(g * n + rng.choice(n, 6, replace=False))})
        for r in picks:
            ref, st, scale = weighted_reference(w.x, v, "bf16", n, w.mask, r, r + 1)
            res = check_weighted(out[r:r + 1], "bf16", ref, st, scale, f"weighted causal row {r}")
            worst = max(worst, res.get("max_ulp", 0))
    banner(f"weighted causal: max ulp {worst}")

"""CPU-only checks of the C ABI boundary: the library loads, exports every
symbol include/smx.h declares, rejects bad arguments before touching a device,
and its scalar arithmetic (built for the host) meets its accuracy claims.
No kernel is launched here.
"""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smx.h")


@pytest.fixture(scope="module")
def smx():
    import numerically_stable_online_amd as m

    if not os.path.exists(m.LIB_PATH):
        from numerically_stable_online_amd import build

        build.build()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:SMX_API\s+)?(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("softmax_rows", "softmax_rows_path", "softmax_row_stats", "softmax_merge_normalize",
              "log_softmax_rows", "log_softmax_rows_path", "softmax_backward_rows",
              "softmax_backward_rows_path", "softmax_cross_entropy_rows", "softmax_cross_entropy_rows_path",
              "softmax_weighted_rows", "softmax_weighted_states", "softmax_weighted_merge",
              "softmax_default_chunk_cols", "softmax_select_path", "smx_last_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol(smx):
    out = subprocess.run(["nm", "-D", "--defined-only", smx.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    extra = sorted(exported - set(declared_functions()))
    assert not extra, f"exported but not declared: {extra}"
    lib = smx.lib()
    for n in declared_functions():
        assert getattr(lib, n) is not None


def test_header_is_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "smx.h"\nint main(void){ smx_stat s; s.m = 0; s.l = 1; return (int)s.l - 1; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", f"-I{ROOT}/include", str(src)],
                   check=True)


def _call(smx, *args):
    return smx.lib().softmax_rows(*args)


def test_argument_checks_need_no_device(smx):
    L = smx.lib()
    EINVAL = smx.SMX_EINVAL
    m = smx.SmxMask()
    cases = [
        ((None, None, -1, 4, 0, None, None), "rows"),
        ((None, None, 4, -1, 0, None, None), "cols"),
        ((None, None, 4, 4, 3, None, None), "dtype"),
        ((None, None, 4, 4, 0, None, None), "x is NULL"),
        ((16, None, 4, 4, 0, None, None), "y is NULL"),
        ((4096, 4096 + 8, 4, 4, 0, None, None), "overlap"),
        ((16, 4096, 1 << 40, 1 << 40, 0, None, None), "overflow"),
    ]
    for args, word in cases:
        assert L.softmax_rows(*args) == EINVAL, word
        assert word.split()[0] in smx.smx_last_error(), (word, smx.smx_last_error())
    m.kind = 1  # VALID_LEN without the array
    assert L.softmax_rows(16, 4096, 4, 4, 0, C.byref(m), None) == EINVAL
    m.kind = 2  # CAUSAL with a bad period
    m.causal_period = 0
    assert L.softmax_rows(16, 4096, 4, 4, 0, C.byref(m), None) == EINVAL
    m.kind = 3  # KEEP without bytes
    assert L.softmax_rows(16, 4096, 4, 4, 0, C.byref(m), None) == EINVAL
    m.kind = 9
    assert L.softmax_rows(16, 4096, 4, 4, 0, C.byref(m), None) == EINVAL
    # forced paths that cannot hold the shape are rejected before any launch
    assert L.softmax_rows_path(16, 1 << 20, 4, 100000, 0, None, 1, 0, None) == EINVAL
    assert L.softmax_rows_path(17, 1 << 20, 4, 64, 0, None, 2, 0, None) == EINVAL
    assert L.softmax_rows_path(16, 1 << 20, 4, 64, 0, None, 7, 0, None) == EINVAL
    assert L.softmax_rows_path(16, 1 << 20, 4, 64, 0, None, 3, -5, None) == EINVAL
    # the summary calls
    assert L.softmax_row_stats(16, 4, 64, 0, None, 0, 64, None) == EINVAL
    assert L.softmax_row_stats(16, 4, 64, 0, None, 16, None, None) == EINVAL
    assert L.softmax_merge_normalize(16, 1 << 20, 4, 64, 0, None, 16, 4096, 3, None) == EINVAL
    assert "n_chunks" in smx.smx_last_error()
    # the entry point that allocates nothing: a split path whose summaries
    # exceed its fixed scratch is refused before any device access, as are
    # the checks it shares with softmax_rows_path
    assert L.softmax_rows_noalloc(16, 1 << 40, 4096, 8192, 0, None, 3, 16, None) == EINVAL
    assert "scratch" in smx.smx_last_error()
    assert L.softmax_rows_noalloc(16, 1 << 40, 1 << 30, 1 << 20, 0, None, 3, 1, None) == EINVAL
    assert L.softmax_rows_noalloc(16, 1 << 20, 4, 100000, 0, None, 1, 0, None) == EINVAL
    assert L.softmax_rows_noalloc(16, 1 << 20, 4, 64, 0, None, 9, 0, None) == EINVAL
    assert L.softmax_rows_noalloc(None, 1 << 20, 4, 64, 0, None, 0, 0, None) == EINVAL


def test_stream_copy_argument_checks(smx):
    """The bandwidth reference copy rejects bad sizes, NULL, misaligned and
    overlapping buffers before any launch (the pointers here are never
    dereferenced)."""
    L = smx.lib()
    EINVAL = smx.SMX_EINVAL
    cases = [
        ((4096, 1 << 20, -16, None), "bytes"),
        ((4096, 1 << 20, 24, None), "bytes"),
        ((None, 1 << 20, 64, None), "NULL"),
        ((4096, None, 64, None), "NULL"),
        ((4104, 1 << 20, 64, None), "aligned"),
        ((4096, 1 << 20 | 8, 64, None), "aligned"),
        ((4096, 4096 + 32, 64, None), "overlap"),
        ((4096, 4096, 64, None), "overlap"),
    ]
    for args, word in cases:
        assert L.smx_stream_copy(*args) == EINVAL, word
        assert word in smx.smx_last_error(), (word, smx.smx_last_error())
    assert L.smx_stream_copy(None, None, 0, None) == smx.SMX_OK


def test_weighted_rows_argument_checks(smx):
    L = smx.lib()
    EINVAL = smx.SMX_EINVAL
    # (s, v, out, rows, cols, d, rows_per_group, dtype, mask, stream)
    cases = [
        ((16, 4096, 1 << 20, 8, 64, 64, 8, 0, None, None), "SMX_F16 or SMX_BF16"),
        ((16, 4096, 1 << 20, 8, 64, 48, 8, 2, None, None), "value width"),
        ((16, 4096, 1 << 20, 8, 64, 64, 3, 2, None, None), "multiple of rows_per_group"),
        ((16, 4096, 1 << 20, 8, 60, 64, 8, 2, None, None), "multiple of 8"),
        ((16, 4096, 1 << 40, 8, (1 << 30) + 8, 64, 8, 2, None, None), "exceeds 2^30"),
        ((18, 4096, 1 << 20, 8, 64, 64, 8, 2, None, None), "aligned"),
        ((16, 4096, 16, 8, 64, 64, 8, 2, None, None), "overlaps"),
        ((16, None, 1 << 20, 8, 64, 64, 8, 2, None, None), "NULL"),
    ]
    for args, word in cases:
        assert L.softmax_weighted_rows(*args) == EINVAL, word
        assert word in smx.smx_last_error(), (word, smx.smx_last_error())
    assert L.softmax_weighted_rows(None, None, None, 0, 64, 64, 8, 2, None, None) == 0


def test_weighted_split_argument_checks(smx):
    """The key-split states and their merge validate like the fused call, plus
    the chunk width (1 .. 2048), the state buffers and the merge's chunk count;
    the failing calls enqueue nothing."""
    lib = smx.lib()
    fake = 1 << 20
    ml, o = fake * 64, fake * 128

    def states(**kw):
        a = dict(s=fake, v=fake * 8, rows=16, cols=4096, d=128, rpg=1, dtype=2, chunk=512, ml=ml, o=o)
        a.update(kw)
        return lib.softmax_weighted_states(a["s"], a["v"], a["rows"], a["cols"], a["d"], a["rpg"], a["dtype"], None,
                                           a["chunk"], a["ml"], a["o"], None)

    assert states(dtype=0) == smx.SMX_EINVAL            # f32
    assert states(d=96) == smx.SMX_EINVAL               # width
    assert states(chunk=0) == smx.SMX_EINVAL
    assert states(chunk=4096) == smx.SMX_EINVAL         # above 2048
    assert states(ml=0) == smx.SMX_EINVAL
    assert states(o=0) == smx.SMX_EINVAL
    assert states(ml=o) == smx.SMX_EINVAL               # ml overlaps o
    assert states(o=fake) == smx.SMX_EINVAL             # o overlaps s
    assert states(rpg=3) == smx.SMX_EINVAL              # rows not a multiple
    assert states(rows=0) == smx.SMX_OK                 # nothing to do

    def merge(**kw):
        a = dict(ml=ml, o=o, rows=16, nch=8, d=128, dtype=2, out=fake)
        a.update(kw)
        return lib.softmax_weighted_merge(a["ml"], a["o"], a["rows"], a["nch"], a["d"], a["dtype"], a["out"], None)

    assert merge(dtype=0) == smx.SMX_EINVAL
    assert merge(d=16) == smx.SMX_EINVAL
    assert merge(nch=16385) == smx.SMX_EINVAL
    assert merge(nch=-1) == smx.SMX_EINVAL
    assert merge(out=0) == smx.SMX_EINVAL
    assert merge(out=fake + 1) == smx.SMX_EINVAL        # odd address
    assert merge(out=ml) == smx.SMX_EINVAL              # out overlaps ml
    assert merge(rows=0) == smx.SMX_OK


def test_empty_shapes_are_noops(smx):
    L = smx.lib()
    assert L.softmax_rows(None, None, 0, 5, 0, None, None) == 0
    assert L.softmax_rows(None, None, 7, 0, 2, None, None) == 0
    assert L.softmax_row_stats(None, 0, 10, 1, None, 4, None, None) == 0
    assert smx.smx_last_error() == ""


def test_path_choice_and_default_chunk(smx):
    assert smx.softmax_select_path(64, 1024, "f32") == "wave"
    assert smx.softmax_select_path(8192, 4096, "bf16") == "lds"
    assert smx.softmax_select_path(32768, 512, "f16") == "wave"
    assert smx.softmax_select_path(64, 1 << 20, "f32") == "split"
    assert smx.softmax_select_path(524288, 2048, "bf16") == "wave"
    # aligned rows past 4 KiB are read once on the LDS path up to 152 KiB,
    # however few; unaligned ones (rows not a multiple of 16 bytes) split
    assert smx.softmax_select_path(4096, 32768, "bf16") == "lds"
    assert smx.softmax_select_path(4096, 77824, "bf16") == "lds"
    assert smx.softmax_select_path(4096, 38912, "f32") == "lds"
    assert smx.softmax_select_path(4096, 77832, "bf16") == "split"
    assert smx.softmax_select_path(100, 32768, "bf16") == "lds"
    assert smx.softmax_select_path(3, 8192, "f32") == "lds"
    assert smx.softmax_select_path(3, 100001, "f16") == "split"
    c = smx.softmax_default_chunk_cols(64, 1 << 20, "f32")
    assert c > 0 and c % 4 == 0 and 64 * (-(-(1 << 20) // c)) >= 1024
    # 32 KiB chunks while the grid keeps at least 1024 workgroups, halved below
    assert smx.softmax_default_chunk_cols(64, 1 << 20, "f32") == 8192
    assert smx.softmax_default_chunk_cols(16, 1 << 22, "bf16") == 16384
    assert smx.softmax_default_chunk_cols(4, 1 << 20, "f32") == 4096   # 1024 workgroups
    assert smx.softmax_default_chunk_cols(4, 1 << 20, "bf16") == 4096
    assert smx.softmax_default_chunk_cols(1, 100000, "f16") == 512     # floor: 64 packs of 8
    for rows, cols, dt in ((1, 10, "bf16"), (3, 100000, "f16"), (1000, 5000, "f32")):
        c = smx.softmax_default_chunk_cols(rows, cols, dt)
        assert c >= 64 and c % (4 if dt == "f32" else 8) == 0


def test_kernel_arithmetic_on_host(tmp_path):
    """The kernels' scalar arithmetic built for the CPU: the fp32 exponential
    is within one ulp of libm's double exp over [-120, 0] (every 8th float,
    and exact differences x - m with a low part), merge identities are exact,
    and bf16 rounding is nearest-even. The fp64-difference exponentials, with
    a correctly rounded base-2 exponential standing in for the hardware one,
    are within one ulp (plus 2^-31 relative) over the same walk and over pairs (x, m) of every
    magnitude, give 1 at the maximum and 0 for -inf, NaN and lanes far below
    it, also where m - 160 rounds back to m in fp32 (|m| >= 2^31)."""
    exe = tmp_path / "check_smx_math"
    subprocess.run(["g++", "-std=c++20", "-O2", "-ffp-contract=off",
                    f"-I{ROOT}/numerically_stable_online_amd/csrc",
                    f"{ROOT}/tests/csrc/check_smx_math.cpp", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe), "8"], capture_output=True, text=True, check=True).stdout
    vals = dict(kv.split("=") for kv in out.split() if "=" in kv)
    assert float(vals["max_ulp"]) < 1.0 and float(vals["max_ulp_pair"]) < 1.0, out
    assert vals["bad_identity"] == "0" and vals["bad_bf16"] == "0", out
    # the fp64-difference forms: a correctly rounded base-2 exponential (half
    # an ulp) and the final rounding (half an ulp) bound them by one ulp plus
    # r's truncation (2^-31 relative) here; the walk reaches 0.9998. The
    # hardware exponential's 0.79 ulp makes the bound about 1.3 on the GPU
    assert float(vals["max_ulp_dd"]) < 1.01 and float(vals["max_ulp_dd_sum"]) < 1.01, out
    assert vals["bad_dd"] == "0", out
    # the merge factor in the 2^64 scale: as exact as the exponential it
    # wraps, also where the unscaled factor would be subnormal
    assert float(vals["max_ulp_diff_b64"]) < 1.0 and vals["bad_scale"] == "0", out


def test_m0_feeds_only_its_direct_loads(tmp_path):
    """Kernels that set m0 (the LDS address of a direct global->LDS load) in
    inline assembly do not declare it clobbered; build() therefore compiles
    each such source to gfx950 assembly and requires every mention of m0 to
    be one of those writes, followed by the wait state and the direct load
    that reads it. The same check runs here on every such source."""
    from numerically_stable_online_amd import build as b

    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc is not installed")
    srcs = [s for s in b.sources() if b.m0_writers(s)]
    assert any(s.endswith("k_pv.hip") for s in srcs), srcs
    for s in srcs:
        assert b.check_m0(s, str(tmp_path / (os.path.basename(s) + ".s"))) > 0

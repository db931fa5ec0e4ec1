"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle (oracle/oracle.c, driven by tests/csrc/oracle_sanitize.c through
every routine on edge-case shapes, masks and values, with buffers of exactly
the sizes its contracts give) and the kernels' scalar arithmetic built for
the host (tests/csrc/check_smx_math.cpp). Any out-of-bounds access, leak or
undefined operation aborts the run (no recovery). CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"{exe} under the sanitizers:\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, f"-I{ROOT}/oracle", f"{ROOT}/oracle/oracle.c",
                    f"{ROOT}/tests/csrc/oracle_sanitize.c", "-o", exe, "-lm", "-lpthread"], check=True)
    assert "sanitize run complete" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_host_math_under_sanitizers(tmp_path):
    exe = str(tmp_path / "check_smx_math")
    subprocess.run(["g++", "-std=c++20", "-ffp-contract=off", *SAN, f"-I{ROOT}/numerically_stable_online_amd/csrc",
                    f"{ROOT}/tests/csrc/check_smx_math.cpp", "-o", exe], check=True)
    out = _run(exe, "64")
    vals = dict(kv.split("=") for kv in out.split() if "=" in kv)
    assert vals["bad_identity"] == "0" and vals["bad_bf16"] == "0", out

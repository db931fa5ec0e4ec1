"""Build the gfx950 HIP library libsmx.so in-tree.

Every .hip source under csrc/ compiles to its own object (in parallel), and
the objects link into numerically_stable_online_amd/libsmx.so.

Every source that sets m0 in inline assembly is also compiled to gfx950
assembly and checked: m0 may appear only in those writes (see check_m0).

Flags of note:
  -ffp-contract=off        every fused multiply-add is written out explicitly
  -target-feature -packed-fp32-ops
                           no packed fp32 instructions are generated
  no -ffast-math, no denormal flushing: subnormal outputs are kept.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsmx.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn and verbose:
        print(warn, flush=True)
    return obj


def m0_writers(src: str) -> bool:
    """Whether a source sets m0 in inline assembly (direct global->LDS loads)."""
    return "m0," in open(src).read()


def check_m0(src: str, asm_path: str) -> int:
    """A source that writes m0 in inline assembly does so without declaring it
    clobbered (the compiler reserves m0 and ignores such a declaration). That
    is sound only while nothing the compiler emits in that file uses m0, so in
    its gfx950 assembly every mention of m0 must be one of those writes,
    followed by the one wait state and the direct load that reads it. Raises
    otherwise; returns the number of writes found."""
    flags = [f for f in CFLAGS if f != "-fPIC"]
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", asm_path], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    lines = [ln.split(";")[0].strip() for ln in open(asm_path)]
    writes = 0
    for i, ln in enumerate(lines):
        if re.search(r"\bm0\b", ln):
            ok = (re.fullmatch(r"s_mov_b32 m0, s\d+", ln) is not None and i + 2 < len(lines)
                  and lines[i + 1] == "s_nop 0" and lines[i + 2].startswith("global_load_lds_dwordx4"))
            if not ok:
                raise RuntimeError(f"{os.path.basename(src)}: m0 used outside the inline direct loads: {ln!r}")
            writes += 1
    if writes == 0:
        raise RuntimeError(f"{os.path.basename(src)}: its inline m0 writes are missing from the assembly")
    return writes


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        m0 = {s: ex.submit(check_m0, s, os.path.join(BUILD_DIR, os.path.basename(s) + ".s"))
              for s in srcs if m0_writers(s)}
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
        for s, f in m0.items():
            n = f.result()
            if verbose:
                print(f"{os.path.basename(s)}: {n} inline m0 writes, each feeding its direct load only", flush=True)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Benchmark: row-softmax effective HBM bandwidth on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads causal,spiked,small,masked,long,vocab]

One step is one softmax_rows call over one batch of the headline workload,
the largest of the workloads: bf16 causal attention scores, 256 groups of
2048 x 2048 (524288 rows x 2048 columns, row i of a group keeping columns
0..i, scores q.k^T / sqrt(128) of seeded N(0, 1) q and k, five injected
+inf / NaN / all -inf rows per group), which the library runs on its
wave-per-row kernel. Smaller inputs rotate through enough resident copies of
x and y (>= 1 GiB in all) that every step streams from HBM instead of
hitting the 256 MB Infinity Cache left warm by the previous step; the
headline's 4 GiB pair is far larger than that cache. Each timed loop follows
its W warm-up calls and, if those took less than 0.25 s, more untimed calls
until 0.25 s has passed (the GPU's clocks settle after the idle gap of input
generation); per_workload reports how many warm-up calls ran.

value  = algorithmic bytes per step / mean step time, in GB/s (1e9 B/s);
         algorithmic bytes = valid input lanes read (twice on the split path),
         every output lane written, plus mask and chunk-summary bytes.
roofline.achieved = the same bytes / the GPU time per launch: HIP events
         recorded on the launch stream around the K timed calls, divided by K
         (so it includes the short gaps between back-to-back launches).
cpu_baseline = the CPU oracle (three-pass, double precision) on the same
         input, on the host cores, writing the element format; sampled rows
         of its output are checked against the oracle's rows-then-encode
         result, so the time is that of the whole work.

Prints one JSON line. Other workloads (--workloads) are reported inside it
under "per_workload".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
# Warm-up floor: after its W warm-up steps each timed loop keeps calling until
# this much wall time has passed, so the GPU's clocks have left the state an
# idle gap (input generation on the host) puts them in; 20-200 calls of a
# 23 us kernel measured 3-5 % slower than the sustained rate.
MIN_WARMUP_S = 0.25
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
MALL_BYTES = 256 * 2 ** 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = {
    "lds": ["k_lds.hip", "k_lds_res.hip", "smx_device.hpp", "smx_math.hpp"],
    "wave": ["k_wave.hip", "smx_device.hpp", "smx_math.hpp"],
    "split": ["k_split.hip", "smx_device.hpp", "smx_math.hpp"],
}
KERNEL_NAME = {"lds": "k_lds", "wave": "k_wave", "split": "k_merge_normalize+k_stats"}
LDS_REGISTER_ROW_BYTES = 32768  # longer rows on the LDS path stay in LDS (k_lds_res)


def kernel_of(path: str, w) -> str:
    """The kernel a workload's softmax runs on its path."""
    from workloads import ITEMSIZE

    if path == "lds" and w.cols * ITEMSIZE[w.dtype] > LDS_REGISTER_ROW_BYTES:
        return "k_lds_res"
    return KERNEL_NAME[path]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="causal,spiked,small,masked,long,vocab",
                    help="workloads to time (names in workloads.WORKLOADS); the first is the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--next-ops", default="spiked,long,vocab",
                    help="workloads on which the log-softmax, softmax-backward and cross-entropy "
                         "entry points are also timed ('' for none)")
    ap.add_argument("--no-weighted", dest="weighted", action="store_false",
                    help="skip the softmax-weighted value sums on the causal scores")
    ap.add_argument("--no-decode", dest="decode", action="store_false",
                    help="skip the softmax-weighted value sums on the decode-shaped input")
    ap.add_argument("--no-copy-context", action="store_true",
                    help="skip timing the two plain copies of the headline input (context only)")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the single-launch spread loop (profiling runs)")
    ap.add_argument("--no-cold-reread", action="store_true",
                    help="skip the split path's passes timed apart with the Infinity Cache evicted between them")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of the headline x (counter calibration)")
    return ap.parse_args()


def code_text(src: str) -> str:
    """A C++ source without its comments and blank lines: what the compiler
    sees, so that editing a comment does not change the hash."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif src[i] == '"':  # a string literal, copied whole
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    lines = [ln.rstrip() for ln in "".join(out).splitlines()]
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_source_sha(path: str) -> str:
    """Hash of the code (comments stripped) of the kernel files a path runs;
    traffic counters are reported only while it matches the hash recorded
    when they were taken."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, "numerically_stable_online_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, path: str, n_chunks: int = 0) -> int:
    """Bytes the method must move for one pass over workload w."""
    from workloads import ITEMSIZE

    s = ITEMSIZE[w.dtype]
    rows, cols, m = w.rows, w.cols, w.mask
    if m.kind == "none":
        valid, mask_bytes = rows * cols, 0
    elif m.kind == "valid_len":
        valid, mask_bytes = int(np.clip(m.valid_len.astype(np.int64), 0, cols).sum()), 4 * rows
    elif m.kind == "causal":
        r = np.arange(rows, dtype=np.int64)
        valid, mask_bytes = int(np.clip(r % m.causal_period + 1 + m.causal_offset, 0, cols).sum()), 0
    else:
        valid, mask_bytes = int(np.count_nonzero(m.keep)), rows * cols
    reads = 2 if path == "split" else 1
    summaries = 2 * rows * n_chunks * 8 if path == "split" else 0
    return reads * valid * s + rows * cols * s + mask_bytes + summaries


def weighted_flops(w) -> int:
    """Multiply-adds of softmax(s) @ V counted as 2 flops: one per valid
    weight and value component (d = 128)."""
    r = np.arange(w.rows, dtype=np.int64)
    valid = int(np.clip(r % w.mask.causal_period + 1 + w.mask.causal_offset, 0, w.cols).sum())
    return 2 * valid * 128


def warm_up(call, warmup: int) -> int:
    """W untimed calls, then more until MIN_WARMUP_S has passed; returns
    how many ran."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        call(n)
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        for _ in range(20):
            call(n)
            n += 1
        torch.cuda.synchronize()
    return n


def make_workload(k: str):
    import workloads as W

    if k not in W.WORKLOADS:
        raise SystemExit(f"unknown workload {k!r}; known: {', '.join(W.WORKLOADS)}")
    return W.WORKLOADS[k]()


def time_workload(w, steps: int, warmup: int, calibrate_copy: bool = False, spread: bool = True,
                  op: str = "softmax_rows"):
    import torch

    import numerically_stable_online_amd as smx
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from smx_compare import to_device

    x0 = to_device(w.x, w.dtype)
    kw = {}
    if w.mask.kind == "valid_len":
        kw["valid_len"] = torch.from_numpy(w.mask.valid_len).cuda()
    elif w.mask.kind == "causal":
        kw["causal_period"] = w.mask.causal_period
        kw["causal_offset"] = w.mask.causal_offset
    pair_bytes = 2 * x0.numel() * x0.element_size()
    free = torch.cuda.mem_get_info()[0]
    copies = max(1, min(64, math.ceil(2 ** 30 / pair_bytes), int(0.5 * free // pair_bytes)))
    if pair_bytes > 4 * MALL_BYTES:
        copies = 1
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    ys = [torch.empty_like(x0) for _ in range(copies)]
    path = smx.softmax_select_path(w.rows, w.cols, x0.dtype)
    n_chunks = 0
    if path == "split":
        chunk = smx.softmax_default_chunk_cols(w.rows, w.cols, x0.dtype)
        n_chunks = -(-w.cols // chunk)
    nbytes = algorithmic_bytes(w, path, n_chunks)
    if op == "softmax_rows":
        def call(i):
            smx.softmax_rows(xs[i % copies], ys[i % copies], **kw)
    elif op == "log_softmax_rows":
        lses = [torch.empty(w.rows, dtype=torch.float32, device=x0.device) for _ in range(copies)]
        nbytes += 4 * w.rows  # the per-row log-sum-exp

        def call(i):
            smx.log_softmax_rows(xs[i % copies], ys[i % copies], lses[i % copies], **kw)
    elif op == "softmax_backward_rows":
        # timing only: p and g are two different resident copies of the input
        s_el = x0.element_size()
        bpath = "split" if w.cols * s_el > 4096 and (w.rows < 1024 or w.cols > 256 * 8 * 16 // s_el) else "row"
        nbytes = 3 * w.rows * w.cols * s_el
        if bpath == "split":
            chunk = smx.softmax_default_chunk_cols(w.rows, w.cols, x0.dtype)
            nbytes += 2 * w.rows * w.cols * s_el + 2 * w.rows * (-(-w.cols // chunk)) * 8
        path = "split" if bpath == "split" else path

        def call(i):
            smx.softmax_backward_rows(xs[i % copies], xs[(i + 1) % copies], ys[i % copies])
    elif op == "softmax_weighted_rows":
        import workloads as W

        # the causal scores weight per group 2048 value vectors of width 128
        groups = w.rows // w.mask.causal_period
        vals = to_device(W.causal_values(w.seed, groups, w.cols, 128).reshape(-1, 128), w.dtype)
        vals = vals.view(groups, w.cols, 128)
        outs = [torch.empty((w.rows, 128), dtype=x0.dtype, device=x0.device) for _ in range(copies)]
        nbytes = algorithmic_bytes(w, "wave") - w.rows * w.cols * 2  # the valid scores read, no y
        nbytes += vals.numel() * 2 + w.rows * 128 * 2  # V read once, out written
        path = "mfma"

        def call(i):
            smx.softmax_weighted_rows(xs[i % copies], vals, outs[i % copies], **kw)
    elif op == "softmax_cross_entropy_rows":
        import workloads as W

        tgt = torch.from_numpy(W.class_targets(w.rows, w.cols, w.seed)).cuda()
        losses = [torch.empty(w.rows, dtype=torch.float32, device=x0.device) for _ in range(copies)]
        nbytes += 4 * w.rows + 4 * w.rows  # the targets read and the losses written
        if path == "split":
            nbytes += 2 * 4 * w.rows  # the target logit passed between the two kernels

        def call(i):
            smx.softmax_cross_entropy_rows(xs[i % copies], tgt, losses[i % copies], ys[i % copies], **kw)
    else:
        raise ValueError(op)

    if calibrate_copy:
        c = torch.empty_like(x0)
        c.copy_(x0)
        torch.cuda.synchronize()

    warm = warm_up(call, warmup)

    # the timed region: K back-to-back calls, bracketed by synchronizations;
    # HIP events on the stream the kernels run on give the GPU time per launch
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / steps

    # spread: single launches bracketed by their own events (not the timed region)
    n_single = min(steps, 20) if spread else 0
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_single)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_single)]
    for i in range(n_single):
        starts[i].record(stream)
        call(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)] or [gpu_ms])
    return {
        "path": path,
        "bytes": nbytes,
        "copies": copies,
        "n_chunks": n_chunks,
        "warmup_steps_run": warm,
        "ms_per_step": wall * 1e3 / steps,
        "gpu_ms_per_launch": gpu_ms,
        "launch_ms_mean": float(launch_ms.mean()),
        "launch_ms_median": float(np.median(launch_ms)),
        "launch_ms_p10": float(np.percentile(launch_ms, 10)),
        "launch_ms_p90": float(np.percentile(launch_ms, 90)),
    }


def split_cold_reread(w, steps: int, warmup: int, scratch_bytes: int = 512 * 2 ** 20):
    """The split path's two passes timed apart, each after a read of
    scratch_bytes, so that each pass, the normalize pass's reread of x
    included, streams from HBM rather than from the Infinity Cache (256 MB)
    the previous pass left warm. The eviction is a read (a sum), so no dirty
    lines are left to drain into the timed pass. Each pass is bracketed by
    its own HIP events; the rate counts the same algorithmic bytes as the
    automatic call (2 R + W + summaries)."""
    import torch

    import numerically_stable_online_amd as smx
    from smx_compare import to_device

    x = to_device(w.x, w.dtype)
    y = torch.empty_like(x)
    chunk = smx.softmax_default_chunk_cols(w.rows, w.cols, x.dtype)
    nch = -(-w.cols // chunk)
    stats = torch.empty((w.rows, nch, 2), dtype=torch.float32, device=x.device)
    scratch = torch.zeros(scratch_bytes // 4, dtype=torch.float32, device=x.device)
    sink = []
    stream = torch.cuda.current_stream()

    def one(i, evs=None):
        sink[:] = [scratch.sum()]
        if evs:
            evs[0].record(stream)
        smx.softmax_row_stats(x, chunk, out=stats)
        if evs:
            evs[1].record(stream)
        sink[:] = [scratch.sum()]
        if evs:
            evs[2].record(stream)
        smx.softmax_merge_normalize(x, stats, chunk, out=y)
        if evs:
            evs[3].record(stream)

    warm_up(one, warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        one(i, ev[i])
    torch.cuda.synchronize()
    t_stats = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_norm = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    nbytes = algorithmic_bytes(w, "split", nch)
    gbs = nbytes / ((t_stats + t_norm) * 1e-3) / 1e9
    return {"stats_ms": round(t_stats, 5), "normalize_ms": round(t_norm, 5), "scratch_read_bytes": scratch_bytes,
            "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": "a read of the scratch (evicting the Infinity Cache), the stats pass, another read of the "
                    "scratch, the normalize pass; each pass timed with its own events; bytes as for the automatic "
                    "call"}


def device_copy(w, steps: int, warmup: int):
    """Two plain device-to-device copies of the workload's input, rotated
    through resident copies the same way as the timed kernels, as context
    beside the roofline: torch copy_ (the runtime's copy kernel) and the
    library's streaming copy (nontemporal 16-byte accesses, the fastest copy
    shape measured on this GPU), i.e. the streaming rate this machine reaches for
    the same bytes."""
    import torch

    import numerically_stable_online_amd as smx
    from smx_compare import to_device

    x0 = to_device(w.x, w.dtype)
    nbytes = x0.numel() * x0.element_size()
    copies = max(1, min(64, math.ceil(2 ** 30 / (2 * nbytes))))
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    ys = [torch.empty_like(x0) for _ in range(copies)]
    out = {}
    stream = torch.cuda.current_stream()
    for name, copy in (("device_copy", lambda a, b: b.copy_(a)), ("stream_copy", smx.stream_copy)):
        def call(i):
            copy(xs[i % copies], ys[i % copies])

        warm_up(call, warmup)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            call(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        out[name] = {"workload": w.name, "bytes": 2 * nbytes, "ms_per_copy": round(ms, 5),
                     "GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1), "buffer_copies": copies}
    out["device_copy"]["kind"] = "torch copy_"
    out["stream_copy"]["kind"] = "smx_stream_copy (nontemporal 16-byte grid-stride copy)"
    return out


def decode_weighted(steps: int, warmup: int, groups: int = 256, keys: int = 32768, d: int = 128):
    """softmax_weighted_rows on a decode-shaped input: one score row per
    group (one query per head) over many keys, the attention workload's
    value width and element type. The seeded synthetic input is drawn on the
    device (timing only; the parity tests check this path on smaller shapes).
    Two copies rotate so V (2 GiB each) streams from HBM. Algorithmic bytes:
    the scores and V read once, the output written."""
    import torch

    import numerically_stable_online_amd as smx

    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    ss = [(3.0 * torch.randn(groups, keys, device="cuda", generator=g)).to(torch.bfloat16) for _ in range(2)]
    vs = [torch.randn(groups, keys, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2)]
    out = torch.empty(groups, d, dtype=torch.bfloat16, device="cuda")
    nbytes = groups * keys * 2 + groups * keys * d * 2 + groups * d * 2
    def call(i):
        smx.softmax_weighted_rows(ss[i % 2], vs[i % 2], out)

    warm_up(call, warmup)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        smx.softmax_weighted_rows(ss[i % 2], vs[i % 2], out)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"bf16_decode_{groups}x1x{keys}_values_d{d}", "path": "key split (states + merge)",
            "algorithmic_bytes": nbytes, "gpu_ms_per_launch": round(ms, 5), "GBps_launch": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def _sub_workload(w, n):
    """The first n rows of workload w, with its mask restricted to them."""
    import workloads as W

    m = w.mask
    if m.kind == "valid_len":
        sub = W.MaskSpec("valid_len", valid_len=m.valid_len[:n])
    elif m.kind == "keep":
        sub = W.MaskSpec("keep", keep=m.keep[:n])
    else:
        sub = m
    return W.Workload(f"{w.name}[:{n}]", w.dtype, w.x[:n], sub, w.seed)


def check_cpu_sample(w, y, n_rows: int = 64) -> int:
    """Sampled rows of the CPU baseline's output y (raw storage) must be
    exactly the oracle's rows-then-encode bytes: rows spread over the input
    plus its special rows. Returns how many rows were checked."""
    import oracle

    rows = set(np.linspace(0, w.rows - 1, n_rows).astype(np.int64).tolist())
    for v in w.special_rows.values():
        rows.update(int(r) for r in np.asarray(v)[:4])
    for r in sorted(rows):
        p, _, _ = oracle.softmax_rows(w.x, w.dtype, w.mask, r, r + 1)
        want = oracle.encode(p, w.dtype).view(np.uint8)
        if not np.array_equal(y[r:r + 1].view(np.uint8), want):
            raise SystemExit(f"cpu_baseline: row {r} of the timed oracle output differs from the oracle's rows")
    return len(rows)


def cpu_baseline(w, nbytes: int):
    """The oracle as it stands, on the host: the whole workload on T threads
    (the CPUs this process may run on, at most 16, the host share of one
    GPU), median of at least 3 runs; then one thread on the first rows of
    the same workload (a whole number of causal periods), about 5 s of work,
    as a second reference point."""
    import oracle

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    out = np.empty_like(w.x)
    times = []
    t_end = time.perf_counter() + 10.0
    while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 10):
        _, dt = oracle.softmax_rows_encode_mt(w.x, w.dtype, w.mask, threads, out=out)
        times.append(dt)
    med = float(np.median(times))
    checked = check_cpu_sample(w, out)
    del out
    # one thread on a prefix of the rows
    n1 = int(min(w.rows, max(1, w.rows * 5.0 / (med * threads))))
    if w.mask.kind == "causal" and n1 >= w.mask.causal_period:
        n1 -= n1 % w.mask.causal_period
    sub = _sub_workload(w, n1)
    b1 = algorithmic_bytes(sub, "lds")
    times1 = []
    for _ in range(2):
        _, dt = oracle.softmax_rows_encode_mt(sub.x, sub.dtype, sub.mask, 1)
        times1.append(dt)
    med1 = float(np.median(times1))
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": nbytes / med / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu": cpu,
            "host_cpus": os.cpu_count(),
            "sample": f"the whole {w.name} input ({w.rows}x{w.cols} {w.dtype}) on {threads} threads, {len(times)} "
                      f"runs, median {med:.3f} s, three-pass double-precision oracle writing {w.dtype}; "
                      f"{checked} sampled output rows checked against the oracle's rows-then-encode bytes",
            "seconds": med,
            "single_thread": {"value": b1 / med1 / 1e9, "unit": "GB/s", "cores": 1, "seconds": med1,
                              "runs": len(times1),
                              "sample": f"rows 0..{n1 - 1} of the same input ({n1 / w.rows:.4f} of it, "
                                        f"{b1} algorithmic bytes)"}}


def load_traffic(path: str, kernel_sha: str, launch_bytes_key: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(launch_bytes_key)
    if not rec or rec.get("source_sha") != kernel_sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(rows are independent: a multi-GPU run would split rows across devices)", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import numerically_stable_online_amd as smx

    smx.lib()
    names = [c for c in args.workloads.split(",") if c]
    per = {}
    head = None
    weighted = None
    for k in names:
        w = make_workload(k)
        r = time_workload(w, args.steps, args.warmup, calibrate_copy=args.calibrate_copy and head is None,
                          spread=not args.no_spread)
        gbs = r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
        kgbs = r["bytes"] / (r["gpu_ms_per_launch"] * 1e-3) / 1e9
        entry = {"workload": w.name, "path": r["path"], "kernel": kernel_of(r["path"], w),
                 "algorithmic_bytes": r["bytes"],
                 "step_ms": round(r["ms_per_step"], 5), "gpu_ms_per_launch": round(r["gpu_ms_per_launch"], 5),
                 "single_launch_ms_mean": round(r["launch_ms_mean"], 5),
                 "launch_ms_p10": round(r["launch_ms_p10"], 5), "launch_ms_p90": round(r["launch_ms_p90"], 5),
                 "GBps_step": round(gbs, 1), "GBps_launch": round(kgbs, 1),
                 "frac_of_peak": round(kgbs / HBM_PEAK_GBS, 4), "buffer_copies": r["copies"],
                 "warmup_steps_run": r["warmup_steps_run"]}
        if r["path"] == "split" and not args.no_cold_reread:
            entry["cold_reread"] = split_cold_reread(w, min(args.steps, 50), args.warmup)
            print(f"# {k}: split path with a cold reread {entry['cold_reread']['GBps']:.0f} GB/s "
                  f"(stats {entry['cold_reread']['stats_ms'] * 1e3:.1f} us + normalize "
                  f"{entry['cold_reread']['normalize_ms'] * 1e3:.1f} us)", file=sys.stderr, flush=True)
        per[k] = entry
        print(f"# {k} {w.name}: path={r['path']} {kgbs:.0f} GB/s per launch "
              f"({r['gpu_ms_per_launch'] * 1e3:.1f} us), {gbs:.0f} GB/s per step", file=sys.stderr, flush=True)
        if k == "causal" and args.weighted:
            rw = time_workload(w, args.steps, args.warmup, spread=False, op="softmax_weighted_rows")
            gw = rw["bytes"] / (rw["gpu_ms_per_launch"] * 1e-3) / 1e9
            flops = weighted_flops(w)
            tfw = flops / (rw["gpu_ms_per_launch"] * 1e-3) / 1e12
            weighted = {"workload": w.name + "_values_d128", "path": "mfma", "algorithmic_bytes": rw["bytes"],
                        "algorithmic_flops": flops, "gpu_ms_per_launch": round(rw["gpu_ms_per_launch"], 5),
                        "GBps_launch": round(gw, 1), "frac_of_hbm_peak": round(gw / HBM_PEAK_GBS, 4),
                        "TFLOPs_launch": round(tfw, 1), "frac_of_bf16_mfma_peak": round(tfw / MFMA_BF16_PEAK_TFLOPS, 4)}
            print(f"# softmax_weighted_rows causal: {gw:.0f} GB/s, {tfw:.0f} TFLOP/s per launch "
                  f"({rw['gpu_ms_per_launch'] * 1e3:.1f} us)", file=sys.stderr, flush=True)
        if head is None:
            head = (k, w, r, gbs, kgbs)
        else:
            del w

    next_ops = {}
    for k2 in [c for c in args.next_ops.split(",") if c]:
        w2 = make_workload(k2)
        for op in ("log_softmax_rows", "softmax_backward_rows", "softmax_cross_entropy_rows"):
            r2 = time_workload(w2, args.steps, args.warmup, spread=False, op=op)
            g2 = r2["bytes"] / (r2["gpu_ms_per_launch"] * 1e-3) / 1e9
            next_ops.setdefault(op, {})[k2] = {
                "workload": w2.name, "path": r2["path"], "algorithmic_bytes": r2["bytes"],
                "gpu_ms_per_launch": round(r2["gpu_ms_per_launch"], 5), "GBps_launch": round(g2, 1),
                "frac_of_peak": round(g2 / HBM_PEAK_GBS, 4)}
            print(f"# {op} {k2}: path={r2['path']} {g2:.0f} GB/s per launch "
                  f"({r2['gpu_ms_per_launch'] * 1e3:.1f} us)", file=sys.stderr, flush=True)
        del w2

    k, w, r, gbs, kgbs = head
    sha = kernel_source_sha(r["path"])
    traffic = load_traffic(r["path"], sha, k)
    out = {
        "metric": "row-softmax effective HBM GB/s (read+write bytes/time) and % of MI355X peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "cols": w.cols, "mask": w.mask.kind,
                   "path": r["path"], "seed": w.seed, "algorithmic_bytes_per_step": r["bytes"],
                   "buffer_copies": r["copies"]},
        "roofline": {"bound": "hbm", "kernel": kernel_of(r["path"], w), "achieved": round(kgbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_source_sha": sha},
        "per_workload": per,
        "next_ops": next_ops,
    }
    if weighted is not None:
        out["next_ops"]["softmax_weighted_rows"] = {"causal": weighted}
    if args.decode:
        dec = decode_weighted(args.steps, args.warmup)
        out["next_ops"].setdefault("softmax_weighted_rows", {})["decode"] = dec
        print(f"# softmax_weighted_rows decode: {dec['GBps_launch']:.0f} GB/s per launch "
              f"({dec['gpu_ms_per_launch'] * 1e3:.1f} us)", file=sys.stderr, flush=True)
    if not args.no_copy_context:
        cp = device_copy(w, args.steps, args.warmup)
        dc, sc = cp["device_copy"], cp["stream_copy"]
        out["context"] = {"device_copy": dc, "stream_copy": sc,
                          "kernel_frac_of_copy": round(kgbs / dc["GBps"], 4),
                          "kernel_frac_of_stream_copy": round(kgbs / sc["GBps"], 4)}
        print(f"# copies of the same input: torch copy_ {dc['GBps']:.0f} GB/s ({dc['ms_per_copy'] * 1e3:.1f} us), "
              f"streaming copy {sc['GBps']:.0f} GB/s ({sc['ms_per_copy'] * 1e3:.1f} us); the kernel reaches "
              f"{kgbs / dc['GBps']:.3f} and {kgbs / sc['GBps']:.3f} of them", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, r["bytes"])
        out["cpu_baseline"]["gpu_over_oracle"] = round(gbs / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

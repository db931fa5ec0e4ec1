"""Host-side checks of bench.py (no GPU): it refuses several GPUs with a
message, and its byte and flop accounting reproduces the totals worked out
by hand for the workloads (a read of the valid lanes, a write of whole rows,
a second read and the chunk summaries on the split path, 4 bytes of mask per
row for valid lengths; 2 flops per valid weight and value component), and its
warm-up runs W calls and then fills a time floor."""
import os
import subprocess
import sys
import types

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _w(rows, cols, dtype, mask):
    return types.SimpleNamespace(rows=rows, cols=cols, dtype=dtype, mask=mask)


def test_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_workloads():
    none = W.MaskSpec("none")
    # 8192 x 4096 bf16: each element read once and written once
    assert bench.algorithmic_bytes(_w(8192, 4096, "bf16", none), "lds") == 134_217_728
    # 64 x 1024 fp32
    assert bench.algorithmic_bytes(_w(64, 1024, "f32", none), "wave") == 524_288
    # 64 x 2^20 fp32 on the split path with 64 chunks per row: two reads, one
    # write, 8-byte summaries written once and read once
    assert bench.algorithmic_bytes(_w(64, 1 << 20, "f32", none), "split", 64) == (
        2 * 268_435_456 + 268_435_456 + 2 * 64 * 64 * 8)
    # 256 groups of 2048 causal bf16 rows: (r mod 2048) + 1 lanes read,
    # whole rows written
    causal = W.MaskSpec("causal", causal_period=2048)
    assert bench.algorithmic_bytes(_w(524_288, 2048, "bf16", causal), "wave") == 1_074_266_112 + 2_147_483_648
    # valid lengths are clamped to [0, cols] and cost 4 bytes per row
    vl = W.MaskSpec("valid_len", valid_len=np.array([0, 1, 512, 600, -3], dtype=np.int32))
    assert bench.algorithmic_bytes(_w(5, 512, "f16", vl), "wave") == (0 + 1 + 512 + 512 + 0) * 2 + 5 * 512 * 2 + 20


def test_weighted_flops_of_the_attention_workload():
    causal = W.MaskSpec("causal", causal_period=2048)
    # 2 flops x 128 components x the valid weights, 256 x (1 + 2 + ... + 2048)
    assert bench.weighted_flops(_w(524_288, 2048, "bf16", causal)) == 2 * 128 * 256 * (2048 * 2049 // 2)
    assert bench.weighted_flops(_w(524_288, 2048, "bf16", causal)) == 137_506_062_336


def test_warm_up_runs_w_calls_then_fills_the_time_floor(monkeypatch):
    """warm_up makes its W calls, then keeps calling (20 at a time, each
    batch ended by a device sync) until MIN_WARMUP_S has passed, and returns
    the number of calls; slow calls end it right after the W."""
    import torch

    syncs = []
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: syncs.append(1))
    clock = [0.0]
    monkeypatch.setattr(bench.time, "perf_counter", lambda: clock[0])
    seen = []

    def fast(i):
        seen.append(i)
        clock[0] += 0.001  # 1 ms a call: the floor needs 250 of them

    n = bench.warm_up(fast, 7)
    assert n == len(seen) and seen == list(range(n))
    assert n >= 250 and (n - 7) % 20 == 0 and n - 20 < 250
    assert len(syncs) == 1 + (n - 7) // 20

    seen.clear()
    clock[0] = 0.0

    def slow(i):
        seen.append(i)
        clock[0] += 0.1  # 100 ms a call: W = 3 already passes the floor

    assert bench.warm_up(slow, 3) == 3 and seen == [0, 1, 2]

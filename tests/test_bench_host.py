"""Host logic of bench.py, no GPU: the algorithmic bytes a decode step is
charged with, the refusal of more than one GPU, and the traffic figure's tie
to the profiled kernel sources.

Bytes per token and KV head follow the block formats (aiwitness.kr table
"Qwen 3.6 27B Q5_K_S + 64k context KLD results": 32 codes of b bits plus one
2-byte fp16 scale per block; a scale-and-min block adds a 2-byte minimum) and
the bf16 precision tail (aitrends.kr article 92204, glossary "Precision
Tail": 2 bytes per element, K and V).  The totals below are those block sizes
multiplied out for each workload by hand."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("name,want", [
    # d64 K4 V4: 2 blocks x (16 + 2) B x 2 planes = 72 B per token, 256 tokens
    ("tiny", 256 * 72),
    # d128 K8 V8: 4 x (32 + 2) x 2 = 272 B, 4096 tokens, 8 KV heads
    ("small", 8 * 4096 * 272),
    # d128 K4 V4: 4 x (16 + 2) x 2 = 144 B, 16 sequences x 8 heads x 32768
    ("mid", 16 * 8 * 32768 * 144),
    # d128 K8 V4 with 1024 bf16 tail tokens: 64512 x (4 x 34 + 4 x 18) + 1024 x 512
    ("long", 8 * 8 * (64512 * 208 + 1024 * 2 * 128 * 2)),
    # d256 K5 V4: 8 x (20 + 2) + 8 x (16 + 2) = 320 B
    ("huge", 32 * 4 * 131072 * 320),
])
def test_bytes_per_step(name, want):
    w = workloads.workload(name)
    assert bench.cache_bytes_per_step(w, [w["n"]] * w["B"]) == want


def test_bytes_per_step_formats_and_lengths():
    w = workloads.workload("long", B=2)
    # a sequence shorter than the tail is all tail
    assert bench.cache_bytes_per_step(w, [100, 0]) == 8 * 100 * 512
    # scale-and-min blocks add 2 B per block and plane
    wm = dict(workloads.workload("mid", B=1), km=True, vm=True)
    assert bench.cache_bytes_per_step(wm, [64]) == 8 * 64 * (144 + 2 * 4 * 2)
    # 32 outlier channels: 32 8-bit codes and one fp16 scale per plane
    wo = dict(workloads.workload("long", B=1, tail=0), outliers=32)
    assert bench.cache_bytes_per_step(wo, [64]) == 8 * 64 * (208 + 2 * (32 + 2))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_for_the_profiled_sources(monkeypatch):
    # the committed counters belong to the long workload and to the current
    # sources; any other workload or source hash reports no traffic
    assert bench.measured_traffic("mid") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("long") is None

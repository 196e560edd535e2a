"""Host-side logic of bench.py (no GPU): the counter records it reports
traffic from, and its refusal of multi-GPU runs."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RECORDS = [
    ("gemv_4096_traffic.md", bench.GEMV_SOURCES),
    ("ffn_4096_traffic.md", bench.MFMA_SOURCES),
    ("chain_65536_traffic.md", bench.CHAIN_SOURCES),
    ("signw_gemv_4096_traffic.md", bench.SIGNW_SOURCES),
    ("signw_16384_traffic.md", bench.SIGNW_SOURCES),
]


def test_digest_covers_every_named_source():
    d = bench.kernel_sources_digest(["gemv.hip", "bnn_internal.h"])
    assert d != bench.kernel_sources_digest(["gemv.hip"])
    assert d != bench.kernel_sources_digest(["bnn_internal.h", "gemv.hip"])  # order matters
    assert d == bench.kernel_sources_digest(["gemv.hip", "bnn_internal.h"])


@pytest.mark.parametrize("name,sources", RECORDS)
def test_traffic_record_reported_only_for_its_sources(name, sources):
    path = os.path.join(ROOT, "profiles", name)
    text = open(path).read()
    assert "kernel_sources_sha256:" in text and "traffic_bytes_per_launch:" in text
    assert "FETCH_SIZE" in text and "WRITE_SIZE" in text  # both passes named
    got = bench.recorded_traffic(name, sources)
    if got is None:  # record taken with older sources: must say so by digest
        assert bench.kernel_sources_digest(sources) not in text
    else:
        assert got > 0
    # a different source set never matches the record
    assert bench.recorded_traffic(name, sources + ["pack.hip"]) is None


def test_missing_record_is_none():
    assert bench.recorded_traffic("no_such_record.md", bench.GEMV_SOURCES) is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


@pytest.mark.parametrize("R", [2, 3, 17, 384])
@pytest.mark.parametrize("steps", [1, 2, 5, 20, 383, 384, 385, 1024])
@pytest.mark.parametrize("warmup", [0, 1, 5, 64])
def test_ring_plan_keeps_timed_weights_cold(R, steps, warmup):
    plan = bench.ring_plan(R, steps, warmup)
    phases = [p for p, _ in plan]
    assert phases[-1] == "timed" and phases[0] == "warm"
    timed = plan[-1][1]
    assert timed == [i % R for i in range(steps)]          # step i reads entry i mod R
    warm = dict(plan)["warm"]
    assert len(warm) == warmup
    if steps + warmup <= R:
        # eager warm-up never reads an entry the timed replay reads
        assert not set(warm) & set(timed)
    # between a timed read and the previous read of the same entry, every
    # other ring entry is read once: R - 1 entries
    assert bench.cold_gap_entries(plan) == R - 1


def test_headline_ring_exceeds_the_infinity_cache():
    # a short run (--steps 20 --warmup 5): each timed 2 MiB weight copy was
    # last read before 383 other copies (766 MiB > 2 x 256 MB) were read
    plan = bench.ring_plan(bench.GEMV_RING, 20, 5)
    gap_bytes = bench.cold_gap_entries(plan) * 4096 * 64 * 8
    assert gap_bytes >= 2 * bench.MALL_BYTES
    assert "evict" in dict(plan)


def test_cold_gap_detects_a_warm_replay():
    # the protocol of the previous bench (no eviction pass between the graph
    # warm-up replay and the timed replay) re-read the timed entries after
    # steps - 1 others only; the checker must see that
    plan = [("warm", [0, 1, 2]), ("graph", list(range(20))), ("timed", list(range(20)))]
    assert bench.cold_gap_entries(plan) == 19


def test_bench_parses_step_flags():
    a = bench.parse(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert (a.gpus, a.steps, a.warmup, a.workload) == (1, 20, 5, "gemv_4096")

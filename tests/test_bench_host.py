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

"""bench.py's host-side contract, on the CPU: more than one GPU is refused
with a message and a non-zero status before any GPU work, and the figures it
takes from the committed counter summary are found there (the prefill
sources have not changed since the summary was taken)."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_counters_match_the_prefill_sources():
    if bench._stored_counters() is None:
        pytest.skip("the counter summary was taken on another prefill source")
    busy = bench.stored_mfma_busy()
    assert set(busy) >= {"intra_16k", "cross_window_16k", "cross_full_32k", "intra_32k"}
    for rec in busy.values():
        assert 0 < rec["mfma_busy"] <= 100 and 0.5 < rec["clock_ghz"] < 3.0
    traffic = bench.stored_traffic()
    assert traffic is not None and traffic > 0

"""Host-side checks of bench.py: the one-GPU contract and the stored counters.

bench.py reports `roofline.traffic` (and, for prefill and fp8, MFMA counters)
from rocprofv3 figures stored with a digest of the sources each workload's
gate/up kernel is built from; a stale digest makes the default line carry
null.  These tests check the stored figures and report (as a skip) any that
the committed sources have outdated.
"""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_kernel_source_lists_name_existing_files():
    for workload, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.isfile(os.path.join(ROOT, "sparse_moe_layer_group_amd", "csrc", f)), (workload, f)


def test_stored_traffic_counters_match_the_sources():
    stale = [w for w in bench.MEASURED_TRAFFIC if bench.measured_traffic(w) is None]
    for w in bench.MEASURED_TRAFFIC:
        if w not in stale:
            assert bench.measured_traffic(w) > 0
    if stale:  # a kernel changed since its counters were taken: the bench reports null
        pytest.skip(f"traffic counters to re-take for {stale}")


def test_stored_mfma_counters_match_the_sources():
    stale = [w for w in bench.MEASURED_MFMA if bench.measured_mfma(w) is None]
    for w in bench.MEASURED_MFMA:
        if w not in stale:
            m = bench.measured_mfma(w)
            assert 0.0 < m["busy"] < 1.0 and 0.5 < m["clock_ghz"] < 2.5
    if stale:
        pytest.skip(f"MFMA counters to re-take for {stale}")

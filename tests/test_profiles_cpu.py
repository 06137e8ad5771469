"""The committed rocprofv3 summaries agree with the sources they describe.

Each `profiles/traffic_*.json` records the sha256 of the kernel source and
device header its counters were taken from; `bench.py` reports that record's
HBM bytes as `roofline.traffic` only while the hash still matches.  These
checks fail when a kernel changes without its profile being taken again, and
when a summary stops naming the command that produced it."""
from __future__ import annotations

import glob
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))
TRACES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_trace.md")))


def _sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def test_profiles_exist():
    assert TRAFFIC and TRACES


@pytest.mark.parametrize("path", TRAFFIC, ids=[os.path.basename(p) for p in TRAFFIC])
def test_traffic_record_matches_current_sources(path):
    rec = json.load(open(path))
    covers = rec["kernel_source_sha256_covers"]
    assert covers and all(os.path.exists(os.path.join(ROOT, p)) for p in covers), covers
    assert rec["kernel_source_sha256"] == _sha(covers), (
        f"{os.path.basename(path)} was taken from other sources than {covers}: profile the workload again")
    assert rec["hbm_bytes_per_launch"] > 0
    cal = rec["copy_calibration"]
    assert 1.5 < cal["fetch_scale"] < 2.5 and 0.5 < cal["write_scale"] < 1.5


@pytest.mark.parametrize("path", TRACES, ids=[os.path.basename(p) for p in TRACES])
def test_trace_summary_names_its_command(path):
    text = open(path).read()
    assert "rocprofv3 --kernel-trace --stats" in text and "bench.py" in text
    assert "_work" not in text, "a summary's command must run committed files only"


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

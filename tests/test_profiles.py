"""The committed HBM-traffic summaries (profiles/*traffic*.json) are
self-consistent: bytes per launch are the counters scaled by the plain-copy
calibration, every file names the two counter commands it came from, and
no launch moves fewer bytes than its algorithmic minimum (a counter or
scaling slip would show as a launch beating the bytes it must read)."""
import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.json")))


def test_there_are_traffic_summaries():
    assert len(FILES) >= 8


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(p) for p in FILES])
def test_traffic_summary_is_consistent(path):
    with open(path) as f:
        t = json.load(f)
    cal = t["copy_calibration"]
    assert (cal["fetch_scale"], cal["write_scale"]) == (2.0, 1.0)
    if "bytes_copied" in cal:
        # a plain copy of N bytes reads N and writes N: the scales map the
        # counters' KiB to bytes moved
        assert cal["fetch_scale"] * cal["fetch_size_kib"] * 1024 == pytest.approx(
            cal["bytes_copied"], rel=1e-3)
        assert cal["write_scale"] * cal["write_size_kib"] * 1024 == pytest.approx(
            cal["bytes_copied"], rel=1e-3)
    moved = (t["fetch_size_kib_per_dispatch"] * 1024 * cal["fetch_scale"]
             + t["write_size_kib_per_dispatch"] * 1024 * cal["write_scale"])
    assert t["bytes_per_launch"] == pytest.approx(moved, rel=1e-5)
    # prefill counts the distinct bytes it must touch (its K/V tiles are
    # re-read through L2 by design)
    floor = t.get("algorithmic_bytes_per_launch", t.get("distinct_bytes_per_launch"))
    assert floor and t["bytes_per_launch"] >= 0.99 * floor
    assert t["dispatches_sampled"] >= 1
    assert len(t["kernel_source_hash"]) == 16
    cmds = t["commands"]
    assert any("--pmc FETCH_SIZE" in c for c in cmds) and any("--pmc WRITE_SIZE" in c for c in cmds)

"""The committed measurement records under profiles/ (no GPU).

counters_*.json hold rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch, scaled by
what the same counters read for a plain copy of known size, with the hash of
the kernel sources they were taken on; bench.py reports them as `traffic`
only while that hash still matches.  Each one names sources that exist, adds
up, and sits beside a kernel-trace summary of the same kernel and workload
that gives its command.  The default bench workload (the 3x3 layer) must
keep valid counters, so its line carries traffic.
"""
import glob
import hashlib
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COUNTERS = sorted(glob.glob(os.path.join(ROOT, "profiles", "counters_*.json")))


def _sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def test_counters_present():
    assert COUNTERS, "no counters_*.json under profiles/"


@pytest.mark.parametrize("path", COUNTERS, ids=os.path.basename)
def test_counters_record(path):
    with open(path) as fh:
        c = json.load(fh)
    for f in c["sources"]:
        assert os.path.isfile(os.path.join(ROOT, f)), f
    cal = c["copy_calibration"]
    assert cal["fetch_scale"] > 0 and cal["write_scale"] > 0
    fetch = c["fetch_kib_per_dispatch"] * 1024 * cal["fetch_scale"]
    write = c["write_kib_per_dispatch"] * 1024 * cal["write_scale"]
    assert abs(c["hbm_fetch_bytes_per_dispatch"] - fetch) <= 1e-3 * fetch + 1024
    assert abs(c["hbm_write_bytes_per_dispatch"] - write) <= 1e-3 * write + 1024
    # each figure is truncated to whole bytes on its own
    assert abs(c["hbm_bytes_per_dispatch"] - c["hbm_fetch_bytes_per_dispatch"] - c["hbm_write_bytes_per_dispatch"]) <= 1
    assert c["dispatches"] >= 1
    summary = os.path.join(ROOT, "profiles", "%s_%s.md" % (c["kernel"], c["workload"]))
    assert os.path.isfile(summary), "no kernel-trace summary %s" % os.path.basename(summary)
    with open(summary) as fh:
        text = fh.read()
    assert "rocprofv3 --kernel-trace --stats" in text and "bench.py" in text


def test_headline_counters_current():
    hits = []
    for path in COUNTERS:
        with open(path) as fh:
            c = json.load(fh)
        if c["workload"] == "conv3x3_bf16" and c["route"] == "auto":
            hits.append(c)
    assert len(hits) == 1
    assert _sha(hits[0]["sources"]) == hits[0]["sources_sha256"], \
        "the 3x3 kernel changed since its counters were taken: retake FETCH_SIZE / WRITE_SIZE"

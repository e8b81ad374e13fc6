"""The recorded measurements still describe the sources: the recurrence's HBM counters were taken
on the current recurrence kernel (else bench.py reports no traffic), and the b32 kernel-trace
summary's dominant-kernel duration agrees with the plan's own events in the same run."""

import json
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_recorded_traffic_matches_the_recurrence_sources():
    with open(os.path.join(ROOT, "profiles", "recurrence_traffic.json")) as f:
        rec = json.load(f)
    assert rec["source_sha256"] == bench.kernel_source_digest(), \
        "the recurrence kernel changed since its HBM counters were taken: retake them"
    assert rec["workload"] == "b32"
    total = rec["fetch_bytes"] + rec["write_bytes"]
    # within 10 % of the algorithmic bytes (gates read, h written, R once per XCD)
    assert rec["algorithmic_bytes"] <= total <= 1.1 * rec["algorithmic_bytes"]


def test_b32_trace_agrees_with_the_plans_events():
    with open(os.path.join(ROOT, "profiles", "b32_kernel_trace.md")) as f:
        text = f.read()
    m = re.search(r"launches, median ([0-9.]+) us, mean ([0-9.]+) us;.*against ([0-9.]+) us from the plan's HIP "
                  r"events", text)
    assert m, "dominant-kernel line missing from the b32 summary"
    median, mean, events = (float(v) for v in m.groups())
    # the events bracket the timed region, so they also hold the few microseconds between launches
    assert mean <= events <= 1.05 * mean
    assert abs(median - mean) <= 0.05 * mean

"""The HBM counter summaries under profiles/ that bench.py reads for its
roofline's `traffic` figure stay tied to the kernel sources they were taken
on: each record's digest must equal the digest of today's sources, so that a
kernel change without a fresh counter run fails here instead of turning the
bench line's traffic into null unnoticed.  No GPU needed.
"""
from __future__ import annotations

import glob
import json
import os
import re

import pytest

import bench
from routed_expert_ffn_flint_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_gate_up.*.hbm_counters.md")))


def record(path):
    with open(path) as f:
        text = f.read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    assert m, f"{path}: no json record"
    return text, json.loads(m.group(1))


def test_every_bench_workload_has_a_counter_summary():
    names = {os.path.basename(p) for p in SUMMARIES}
    for wl in ("decode32", "prefill4096", "skew16384", "stack47", "decode32_mx4", "dense32", "dense4096"):
        assert any(n.endswith(f"_gate_up.{wl}.hbm_counters.md") for n in names), wl


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_counter_summary_matches_current_sources(path):
    text, rec = record(path)
    kernel, wl = os.path.basename(path).split("_gate_up.")
    wl = wl[: -len(".hbm_counters.md")]
    assert kernel in bench.KERNEL_SOURCES
    assert wl in inputs.WORKLOADS
    assert rec["workload"] == wl
    assert rec["sources_sha256"] == bench.sources_digest(kernel), (
        f"{os.path.basename(path)} was taken on other sources of {kernel}: take the counters again")
    assert bench.counters_traffic(kernel, wl, bench.sources_digest(kernel)) == rec["traffic_bytes_per_launch"]
    # measured traffic never falls below what the kernel must move
    assert rec["traffic_bytes_per_launch"] >= 0.95 * rec["algorithmic_bytes_per_launch"]
    # the summary states the commands that made it, on committed files only
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    assert "_work" not in text


def test_profiles_hold_text_only():
    for p in glob.glob(os.path.join(ROOT, "profiles", "*")):
        assert os.path.splitext(p)[1] in (".md", ".txt"), p

"""The committed rocprofv3 summaries: complete, named for a known workload,
and made by commands that run the committed benchmark only.

Whether a summary matches the current kernel sources is decided at run time
by bench.py (its HBM traffic figure is reported only when the recorded source
hash matches), so a kernel edit does not fail this test.
"""
import glob
import json
import os

from accelerator_programming_amd.inputs import GEMM_WORKLOADS, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
KNOWN = {w.name for w in WORKLOADS.values()} | {w.name for w in GEMM_WORKLOADS.values()} | {
    "R1_rope_B1_H32_N16384_d128"}


def traffic_files():
    return sorted(glob.glob(os.path.join(PROFILES, "*_traffic.json")))


def test_every_summary_has_trace_counters_and_traffic():
    files = traffic_files()
    assert files, "no profiles committed"
    for f in files:
        tag = os.path.basename(f)[: -len("_traffic.json")]
        for part in ("kernel_trace.txt", "counters.txt"):
            assert os.path.exists(os.path.join(PROFILES, "%s_%s" % (tag, part))), (tag, part)


def test_traffic_summaries_are_well_formed():
    for f in traffic_files():
        with open(f) as fh:
            t = json.load(fh)
        assert t["workload"] in KNOWN, (f, t["workload"])
        assert t["kernel"] and len(t["kernel_sha"]) == 16
        # HBM bytes: calibrated against a copy of known size, positive
        assert t["fetch_scale"] > 0 and t["write_scale"] > 0
        assert t["bytes_per_launch"] == t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
        assert t["bytes_per_launch"] > 0
        for cmd in t["commands"]:
            assert cmd.startswith("rocprofv3 ") and " -- python3 bench.py" in cmd, cmd
            # counters are collected in their own runs, never beside a trace domain
            if "--pmc" in cmd:
                assert "--sys-trace" not in cmd and "--runtime-trace" not in cmd


def test_kernel_trace_summaries_name_their_command():
    for f in sorted(glob.glob(os.path.join(PROFILES, "*_kernel_trace.txt"))):
        with open(f) as fh:
            text = fh.read()
        assert "rocprofv3 --kernel-trace --stats" in text, f
        assert "avg ns" in text, f

"""Host-side pieces of bench.py: the multi-GPU refusal and the counter-derived traffic record."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_records_are_well_formed():
    for wl in ("w4a16", "w8a8", "w4a8", "w4a4", "w4a16mx", "fp8block", "w8a16", "f8a16", "w2a16", "moe", "moe_mx",
               "moe_fp8b", "moe_layer", "moe_layer_w4a8", "w3a16"):
        path = os.path.join(ROOT, "profiles", f"traffic_{wl}.json")
        rec = json.load(open(path))
        cal = rec["copy_calibration"]
        fetch = rec["fetch_size_kib_per_dispatch"] * 1024 * cal["fetch_factor"]
        write = rec["write_size_kib_per_dispatch"] * 1024 * cal["write_factor"]
        assert abs(fetch + write - rec["hbm_bytes_per_launch"]) <= 1e-4 * rec["hbm_bytes_per_launch"]
        assert len(rec["kernel_sources_sha256"]) == 64 and rec["kernel_files"]


def test_committed_bench_lines_name_their_workload():
    """Every committed bench line's config.workload is the label bench.py gives that workload."""
    configs = list(bench.WORKLOADS) + ["moe", "moe_mx", "moe_fp8b", "moe_layer", "moe_layer_w4a8"]
    paths = [os.path.join(ROOT, "profiles", f"bench_{wl}.json") for wl in configs]
    if not all(os.path.exists(p) for p in paths):
        pytest.skip("the bench records are not in this copy of the tree (they stay off the GPU box)")
    for wl, path in zip(configs, paths):
        line = json.load(open(path))
        assert line["config"]["workload"] == bench.workload_name(wl), path
    assert len({bench.workload_name(wl) for wl in configs}) == len(configs)


def test_traffic_is_dropped_when_sources_change(monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_w4a16.json")))
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda files=None: rec["kernel_sources_sha256"])
    assert bench.measured_traffic("w4a16", rec["point"]) == rec["hbm_bytes_per_launch"]
    assert bench.measured_traffic("w4a16", "M=0") is None
    if rec.get("plan") is not None:      # another configuration at that point: dropped too
        other = [rec["plan"][0], rec["plan"][1] + 1, rec["plan"][2]]
        assert bench.measured_traffic("w4a16", rec["point"], plan=other) is None
        assert bench.measured_traffic("w4a16", rec["point"], plan=rec["plan"]) == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda files=None: "0" * 64)
    assert bench.measured_traffic("w4a16", rec["point"]) is None


def test_kernel_sources_sha_covers_the_named_files_only(tmp_path):
    full = bench.kernel_sources_sha()
    part = bench.kernel_sources_sha(["gemm_pingpong.hip", "device_ops.h"])
    assert len(full) == len(part) == 64 and full != part
    assert part == bench.kernel_sources_sha(["device_ops.h", "gemm_pingpong.hip"])   # order-free


def test_traffic_records_reach_the_gpu_box():
    """bench.py resolves `roofline.traffic` from profiles/traffic_*.json on the machine it runs on,
    so no line of .gpurunignore may keep those records from being shipped with the tree."""
    import fnmatch
    lines = [ln.strip() for ln in open(os.path.join(ROOT, ".gpurunignore")) if ln.strip() and not ln.startswith("#")]
    for rec in ("./profiles/traffic_w4a16.json", "./profiles/traffic_moe.json"):
        for pat in lines:
            anchored = pat.startswith("./")
            name = rec if anchored else os.path.basename(rec)
            assert not fnmatch.fnmatch(name, pat) and not rec.startswith(pat.rstrip("/") + "/"), (pat, rec)


def test_current_records_resolve():
    """A record whose kernel sources are unchanged must give a number: a null traffic field in the
    measured line then means the kernel changed, never that the record was not found."""
    for path in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not (path.startswith("traffic_") and path.endswith(".json")):
            continue
        rec = json.load(open(os.path.join(ROOT, "profiles", path)))
        if rec["kernel_sources_sha256"] != bench.kernel_sources_sha(rec["kernel_files"]):
            continue
        assert bench.measured_traffic(rec["workload"], rec["point"]) == rec["hbm_bytes_per_launch"], path

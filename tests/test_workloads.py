"""The frozen workload parameters agree with the oracle calibration that produced them
(tests/golden/calibrate_tau.py -> tests/golden/tau_calibration.json)."""
import json
import os

from entropy_adaptive_sparse_amd import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tau_calibration.json")


def test_frozen_tau_matches_calibration():
    cal = json.load(open(GOLDEN))["workloads"]
    for wid in (2, 3, 4):
        wl = workloads.get(wid)
        c = cal[wl.name]
        assert wl.tau == c["tau"], wl.name
        assert abs(c["density"] - wl.density_target) < 0.005, wl.name


def test_static_mask_workload_matches_calibration():
    # one entropy constant per head, each matched to the density of the same head of workload 3
    cal = json.load(open(GOLDEN))["workloads"]
    wl = workloads.get(5)
    c = cal[wl.name]
    assert wl.static_mask and wl.tau == c["tau"] and wl.tau == workloads.get(3).tau
    assert len(wl.static_entropy) == wl.outer == len(c["static_entropy"])
    assert list(wl.static_entropy) == c["static_entropy"]
    for d, t in zip(c["density"], c["target"]):
        assert abs(d - t) < 0.005


def test_density_variants_match_calibration():
    cal = json.load(open(GOLDEN))["workloads"]
    wl = workloads.get(3)
    var = cal[wl.name]["density_variants"]
    for d, tau in workloads.DENSITY_TAU[3].items():
        if abs(d - 0.15) < 1e-9:
            assert tau == wl.tau
            continue
        c = var["%.2f" % d]
        assert tau == c["tau"] and abs(c["density"] - d) < 0.005


def test_traffic_profile_is_current():
    """bench.py reports the sparse kernel's HBM traffic from the committed counter summary only
    while that summary was taken on the present kernel source; this keeps the two in step."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    src = os.path.join(root, "entropy_adaptive_sparse_amd", "csrc", "attention.hip")
    traffic = bench.profiled_traffic(workloads.get(3).name, src)
    assert traffic is not None, "profiles/attn_sparse_hbm_traffic.md was taken on another attention.hip"
    assert traffic > 3.0e9  # at least q, k, v and o once


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU and says so for --gpus N > 1 (exit status 2, before any GPU work)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in (r.stdout + r.stderr)

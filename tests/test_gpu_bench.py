"""GPU: bench.py keeps its one-line JSON contract (metric, value, roofline with the sparse
kernel's HBM traffic from the committed counter summary of the present kernel source) on a
short run, with the fp8 and 1D-distance rows."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    print("bench.py --steps 1 --warmup 0 --no-cpu", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0", "--no-cpu"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 0 and d["cpu_baseline"] is None
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["value"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == 2500.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # the counter summary under profiles/ was taken on this kernel source: traffic is live (at least
    # q, k, v and o once)
    assert isinstance(rf["traffic"], int) and rf["traffic"] > 3.0e9
    assert d["config"]["workload"] == "wan2.1-14b-720p-21x45x80"
    assert all(v > 0 for v in d["ms_per_call"].values())
    assert set(d["ms_per_call"]) == {"permute_qkv", "dense_entropy", "build_mask", "schedule", "sparse_attn",
                                     "unpermute"}
    f8 = d["fp8_sparse"]
    assert f8["ms"] > 0 and abs(f8["frac_blended"] - f8["achieved"] / f8["peak_blended"]) < 1e-3
    m1 = d["mask_1d"]
    assert m1["ms_mask"] > 0 and 0.0 < m1["density"] <= 1.0 and m1["ms_sparse"] > 0
    rl = d["rooflines"]
    assert rl["device_copy"]["achieved"] > 0
    for name in ("permute_qkv", "unpermute"):
        assert abs(rl[name]["vs_device_copy"] - rl[name]["achieved"] / rl["device_copy"]["achieved"]) < 2e-3

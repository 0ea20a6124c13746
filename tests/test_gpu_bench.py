"""The benchmark's JSON line: one short run of the default workload (zigzag 128K
rank-0 share) must print the fields the metric is reported with, and its
numbers must agree with each other (value from the step time and the credited
pairs, the roofline fraction from its achieved rate and peak)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    from gpu_util import log
    log("bench.py --steps 2 --warmup 1 --no-cpu-baseline --also contiguous --also-steps 1")
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                          "--no-cpu-baseline", "--also", "contiguous", "--also-steps", "1"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 2 and r["warmup"] == 1
    assert r["unit"] == "TFLOP/s" and r["higher_is_better"] is True and r["dtype"] == "bf16"
    assert r["vs_baseline"] is None and r["cpu_baseline"] is None
    assert "workload" in r["config"] and r["config"]["layout"] == "zigzag"
    # value = 3.5 x forward FLOP of the visible pairs over the step time
    pairs = r["visible_pairs_per_head"]
    assert pairs == 1073750016  # zigzag 128K, rank 0 of 8: 16 C^2 + C pairs per head with C = 8192
    fb_flop = 3.5 * 4 * 128 * 32 * pairs
    assert abs(r["value"] - fb_flop / (r["ms_per_step"] / 1e3) / 1e12) <= 0.01 * r["value"]
    assert 0 < r["value"] < 2516.6
    rf = r["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2516.6
    assert rf["kernel"] in r["kernels"] and rf["launches"] == 2 * 8
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert rf["traffic"] is None or rf["traffic"] > 0
    # the per-kernel launches: 8 ring steps per timed step for each block kernel
    for name in ("block_fwd", "block_bwd_dkdv", "block_bwd_dq_ds"):
        assert r["kernels"][name]["launches"] == 2 * 8, name
    # step statistics, ring efficiency and the compact line of a further workload
    assert r["step_ms_min"] <= r["step_ms_median"] and r["fwd_ms_min"] <= r["fwd_ms_median"]
    re_ = r["ring_efficiency_fwd"]
    assert re_ is not None and 0 < re_["value"] < 2 and re_["ring_fwd_ms"] == pytest.approx(r["ms_fwd"], rel=1e-3)
    o = r["other_workloads"]["contiguous"]
    assert o["visible_pairs_per_head"] == 32768 * 32769 // 2  # all 8 ranks: every causal pair once
    assert o["steps"] == 1 and o["min_ms"] <= o["median_ms"]
    assert abs(o["tflops"] - 3.5 * 4 * 128 * 32 * o["visible_pairs_per_head"] / (o["ms_per_step"] / 1e3) / 1e12) \
        <= 0.01 * o["tflops"]

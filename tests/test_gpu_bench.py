"""The benchmark's output line, run in this process on the toy workload with
a few steps: one JSON line with the metric, the step time, the roofline of the
dominant kernel and the oracle baseline, in the shape the benchmark promises."""

import json
import sys

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_bench_json_line(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "toy", "--steps", "3",
                                      "--warmup", "1", "--cpu-seconds", "0.5", "--no-clocks",
                                      "--extra-workloads", "none"])
    print("[bench] toy, 3 steps", file=sys.stderr, flush=True)
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "tokens/s"
    assert d["config"]["workload"].startswith("toy")
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma") and r["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < r["frac"] <= 1.0 and r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    assert c["single_thread"]["cores"] == 1
    assert set(d["kernels"]) >= {"route", "dispatch_layout", "permute", "ffn_up", "ffn_down",
                                 "combine", "bias_update"}
    assert "H excluded" in r["algorithmic"]
    f = d["routed_ffn"]
    assert 0 < f["frac_of_floor"] <= 1.0 and f["weight_floor_us"] > 0
    ld = d["load"]
    assert ld["drop_rate"] == 0.0 and ld["rank_load_max_over_mean"] >= 1.0

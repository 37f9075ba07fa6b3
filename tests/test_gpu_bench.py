"""bench.py's output contract on the GPU: one JSON line with the metric, the
whole-job value, the roofline of the dominant kernel (with the per-launch
timing taken with every launch queued ahead) and the oracle's CPU baseline,
on the small fp32 workload with a few steps."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


def test_bench_line_contract(monkeypatch, capsys):
    import bench
    print("[case] bench.py --workload 1 --steps 5 --warmup 2 --sets 1 --no-configs", flush=True)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "1", "--steps", "5", "--warmup", "2",
                                      "--sets", "1", "--no-configs"])
    bench.main()
    out = capsys.readouterr().out.strip().splitlines()
    lines = [l for l in out if l.startswith("{")]
    assert len(lines) == 1, out
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 5 and rec["warmup"] == 2
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["config"]["workload"].startswith("tiny_fp32")
    rf = rec["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["launches_queued_ahead"] is True
    cb = rec["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]

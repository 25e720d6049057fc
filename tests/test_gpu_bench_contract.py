"""bench.py's output contract, on a short run of the headline workload: exactly one
JSON line on stdout, with the fields and types its consumers read (throughput,
timing protocol, workload, roofline of the dominant kernel with its counter
traffic, and the CPU oracle baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line(gpu):
    print("\n[case] bench.py --steps 3 --warmup 1 --repeats 2 --compare-steps 2 --cpu-seqs 1 --extra ''", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--repeats",
                        "2", "--compare-steps", "2", "--cpu-seqs", "1", "--extra", ""], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[key], typ), key
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["value"] > 0 and abs(d["value"] - d["config"]["tokens"] / (d["ms_per_step"] * 1e-3)) <= 1e-3 * d["value"]
    assert d["config"]["workload"].startswith("c3")
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["peak"] > 0 and 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"] and cb["unit"]
    assert d["path_compare"]["steps"] == 2

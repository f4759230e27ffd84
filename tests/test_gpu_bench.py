"""The bench.py JSON line on an MI355X: one small run as a child process,
checked field by field against the contract the line documents (metric,
timing, config, roofline, CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    print(f"[bench] bench.py {' '.join(args)}", file=sys.stderr, flush=True)
    p = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_line_contract():
    d = _run("--config", "c1", "--steps", "50", "--warmup", "3", "--cpu-seconds", "1",
             "--no-probe")
    for k, t in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                 ("steps", int), ("warmup", int), ("ms_per_step", float),
                 ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                 ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[k], t), (k, d[k])
    assert d["n_gpus"] == 1 and d["steps"] == 50 and d["warmup"] == 3
    assert d["unit"] == "us/call" and d["higher_is_better"] is False
    assert d["vs_baseline"] is None
    assert abs(d["ms_per_step"] * 1e3 - d["value"]) <= 1e-3 * d["value"] + 1e-6
    assert d["config"]["id"] == "c1" and "workload" in d["config"]
    assert d["config"]["untimed_calls_before_timed_region"] == 3
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    # achieved = algorithmic bytes per launch / the launch time the line reports
    assert abs(r["achieved"] - r["alg_bytes_per_launch"] / (d["value"] * 1e-6) / 1e9) <= (
        1e-3 * r["achieved"] + 0.1)
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-3
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "us/call" and c["cores"] >= 1
    assert c["value"] > 0 and "c1" in c["sample"]
    assert d["extra"]["sets_consistent"] is True


@pytest.mark.parametrize("args,what", [
    (("--epilogue",), "bias + RMSNorm"),
    (("--two-shot",), "two-shot"),
    (("--slot-dtype", "bf16", "--out-dtype", "bf16"), '"slots": "bf16"'),
    (("--epilogue-unfused",), "second kernel"),
])
def test_bench_other_entry_points_run(args, what):
    d = _run("--config", "c1", "--steps", "20", "--warmup", "2", "--cpu-seconds", "0",
             "--no-probe", *args)
    assert d["value"] > 0 and d["extra"]["sets_consistent"] is True, args
    assert d["cpu_baseline"] is None
    assert what in json.dumps(d["config"]), (args, d["config"])

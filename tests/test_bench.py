"""The benchmark's command-line contract: one GPU only, and the one JSON line
it prints (fields, types, the roofline and CPU-baseline objects)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one MI355X" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_bench_json_line_contract():
    r = _bench("--steps", "5", "--warmup", "2", "--no-cold", "--workload", "small")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool),
                     ("scaling", str), ("dtype", str), ("data", str), ("config", dict),
                     ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["clock_settle"]["steps"] > 0 and d["clock_settle"]["ms"] >= 300.0
    assert d["value"] > 0 and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["config"]["workload"]
    rl = d["roofline"]
    assert rl["bound"] in ("hbm", "mfma", "alu") and rl["unit"] in ("GB/s", "TOP/s", "TFLOP/s")
    assert rl["achieved"] > 0 and rl["peak"] > 0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert "traffic" in rl
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    cal = d["calibration"]
    assert cal["mfma_i8"]["tops"] > 0 and cal["epilogue_valu"]["tops"] > 0
    assert cal["epilogue_valu_q4k"]["tops"] > 0 and rl["epilogue_roof"]["measured"] > 0
    # the chunk-step ceilings: below the MFMA peak, and the kernel below them
    assert 0 < cal["chunk_q4k"]["tops"] < cal["mfma_i8"]["tops"]
    assert 0 < cal["chunk_q6k"]["tops"] < cal["mfma_i8"]["tops"]
    assert 0 < rl["chunk_roof"]["frac_of_measured"] < 1.05
    ov = cal["mfma_valu_overlap"]
    assert ov["both_cycles"] >= max(ov["mfma_cycles"], ov["fma_cycles"]) * 0.95

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
    assert all(cal[k]["schedule"] in ("default", "max-ilp") for k in ("mfma_i8", "chunk_q4k", "chunk_q6k"))
    # power and clock samples (null where amd-smi is missing or the run too short to sample)
    assert "telemetry" in d
    if d["telemetry"] is not None:
        assert d["telemetry"]["samples"] > 0 and d["telemetry"]["gfx_mhz_median"] > 0
    # per weight type: its GEMMs' rate against the int8 peak and its own chunk-step roof
    pt = rl["per_type"]
    assert pt and set(pt) <= {"q4_K", "q6_K", "q4_K packed"}, pt
    for v in pt.values():
        assert v["tops"] > 0 and abs(v["frac"] - v["tops"] / rl["peak"]) < 1e-3
        assert 0 < v["chunk_roof_frac"] < 1.05
    ov = cal["mfma_valu_overlap"]
    assert ov["both_cycles"] >= max(ov["mfma_cycles"], ov["fma_cycles"]) * 0.95


def test_step_roof_weights_each_gemm_by_its_ops():
    """The roof of a step of several GEMMs (epilogue and chunk-step roofs) is
    its total ops over the sum of each GEMM's time at its own type's roof: a
    harmonic mean weighted by ops, checked on hand-computed cases (CPU)."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    g = [("a", synth.Q4_K, 4096, 4096, "x"), ("b", synth.Q6_K, 4096, 11008, "y")]
    roofs = {synth.Q4_K: 1000.0, synth.Q6_K: 500.0}
    ops = [2.0 * 64 * 4096 * 4096, 2.0 * 64 * 4096 * 11008]
    want = sum(ops) / (ops[0] / 1000.0 + ops[1] / 500.0)
    assert abs(bench.epilogue_roof(g, 64, roofs.get) - want) < 1e-9 * want
    # one GEMM: its own roof; equal roofs: that roof
    assert bench.epilogue_roof(g[:1], 64, roofs.get) == 1000.0
    assert abs(bench.epilogue_roof(g, 64, lambda t: 700.0) - 700.0) < 1e-9
    # the nominal vector-ALU roofs: 256 CUs x 64 lanes x 2.4 GHz lane-instructions,
    # 64 int8 ops per (token, row, 32-block), 3 (q6_K) or 2.25 (q4_K) instructions each
    assert abs(bench.nominal_epilogue_tops(synth.Q6_K) - 256 * 64 * 2.4e9 * 64 / 3 / 1e12) < 1e-9
    assert abs(bench.nominal_epilogue_tops(synth.Q4_K) - 256 * 64 * 2.4e9 * 64 / 2.25 / 1e12) < 1e-9


def test_kernel_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    """The kernel hash that ties the committed counters to the MMQ code stays
    the same when only comments or blank space change, and changes with the
    code (CPU)."""
    sys.path.insert(0, ROOT)
    import bench
    src = open(bench.KERNEL_SRC).read()
    h0 = bench.kernel_hash()
    k = tmp_path / "k.hip"
    k.write_text("// a comment\n\n" + src.replace("namespace qmm {", "namespace qmm {  /* a note */", 1))
    monkeypatch.setattr(bench, "KERNEL_SRC", str(k))
    assert bench.kernel_hash() == h0
    assert "constexpr int kGroupRows = 8;" in src
    k.write_text(src.replace("constexpr int kGroupRows = 8;", "constexpr int kGroupRows = 4;"))
    assert bench.kernel_hash() != h0

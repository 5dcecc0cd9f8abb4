"""Benchmark of the q4_K/q6_K x q8 prefill MMQ on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the hot path over one batch of synthetic activations that
are already resident in HBM: the q8 quantize prepass of every distinct input,
then every MMQ of the workload.  Weight registration (the once-per-weight repack
into planes) happens before the timed region, as a deployment does it at model
load; its device memory is reported.

Prints one JSON line: effective int8 TOPS of the whole step (2*T*od*id summed
over the GEMMs, per step time); the spread of the step time and the roofline of
the dominant kernel (the MMQ) from HIP events on the stream the kernels run on,
at each step's start, between its prepass and its MMQs, and at its end, in a
second pass of K steps (so the timed steps carry nothing but the kernels); each
kernel's time alone (K back-to-back launches between two events, a third pass);
the MMQs with the weights cold (a fourth pass rotating over
copies of the weights whose planes together exceed the 256 MB last-level
cache); the measured roofs (the int8 MFMA rate and the vector-ALU rate of the
scale epilogue on calibration kernels, with the shader clock); and the CPU
oracle timed on the host as a reference (all host threads, and one thread).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import re
import importlib.util
import json
import os
import shutil
import subprocess
import threading
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

MFMA_INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA
# The vector-ALU roof of the scale epilogue: each (token, row, 32-block) takes 64
# int8 MFMA ops and, on the vector ALU, 3 instructions for q6_K (join the two
# plane dots, convert, FMA) or 2.25 for q4_K (remove the block dot's accumulator
# bias, FMA with the scale product that comes from the matrix core, and per
# super-block of 8 chunks two FMAs for d and the min term), at 256 CUs x 64
# lanes x 2.4 GHz lane-instructions/s.
EPILOGUE_INSTRS = {synth.Q6_K: 3, synth.Q4_K: 2.25,
                   # the packed-code registration: 4 more per 16 elements to unpack
                   synth.Q4_K_PACKED: 2.5}
VALU_LANE_OPS = 256 * 64 * 2.4e9


def epilogue_roof(gemms, T, tops_of_type):
    """The roof of a step whose GEMMs have different epilogue roofs: its total
    ops over the sum of each GEMM's time at its own type's roof."""
    ops = [2.0 * T * od * id_ for _, _, od, id_, _ in gemms]
    return sum(ops) / sum(o / tops_of_type(t) for o, (_, t, _, _, _) in zip(ops, gemms))


def nominal_epilogue_tops(type_):
    return VALU_LANE_OPS * 64 / EPILOGUE_INSTRS[type_] / 1e12
HBM_PEAK_GBS = 8000.0
COLD_BYTES = 512 << 20         # weight planes cycled per cold pass: twice the 256 MB cache

# workload name -> (description, tokens, inputs {name: id}, gemms [(name, type, od, id, input)],
#                   outliers)
def _single(cfg, inp="x"):
    name, type_, od, id_, T, outl = cfg
    return (name, T, {inp: id_}, [(name, type_, od, id_, inp)], outl)


WORKLOADS = {
    "ffn_down": _single(synth.FFN_DOWN),            # q6_K 4096 x 11008, 512 tokens
    "ffn_down_odd": _single(synth.FFN_DOWN_ODD),
    "attn": _single(synth.ATTN),
    "ffn_gate_up": _single(synth.GATE_UP),
    "head": _single(synth.HEAD),
    "small": _single(synth.SMALL_Q6K),
    # one GPU's share of ffn_down under 8-way tensor parallelism: a column slice
    # (512 of the 4096 rows) and a row slice (6 of the 43 super-blocks of id)
    "ffn_down_tp8_col": _single(("q6_K ffn_down column shard 512x11008 T=512", synth.Q6_K, 512, 11008, 512, False)),
    "ffn_down_tp8_row": _single(("q6_K ffn_down row shard 4096x1536 T=512", synth.Q6_K, 4096, 1536, 512, False)),
    "layer": ("LLaMA-7B q4_K_M-style layer, 3314 tokens (q,k,o,gate,up q4_K; v,down q6_K)",
              synth.LAYER_TOKENS,
              {"attn_in": 4096, "attn_out": 4096, "ffn_in": 4096, "ffn_mid": 11008},
              [("attn_q", synth.Q4_K, 4096, 4096, "attn_in"),
               ("attn_k", synth.Q4_K, 4096, 4096, "attn_in"),
               ("attn_v", synth.Q6_K, 4096, 4096, "attn_in"),
               ("attn_output", synth.Q4_K, 4096, 4096, "attn_out"),
               ("ffn_gate", synth.Q4_K, 11008, 4096, "ffn_in"),
               ("ffn_up", synth.Q4_K, 11008, 4096, "ffn_in"),
               ("ffn_down", synth.Q6_K, 4096, 11008, "ffn_mid")],
              False),
    # the same layer with the q4_K weights registered with their codes packed two
    # per byte (0.5 instead of 1 byte per weight of code plane)
    "layer_packed": ("LLaMA-7B q4_K_M-style layer, 3314 tokens, q4_K codes packed on the device",
                     synth.LAYER_TOKENS,
                     {"attn_in": 4096, "attn_out": 4096, "ffn_in": 4096, "ffn_mid": 11008},
                     [("attn_q", synth.Q4_K_PACKED, 4096, 4096, "attn_in"),
                      ("attn_k", synth.Q4_K_PACKED, 4096, 4096, "attn_in"),
                      ("attn_v", synth.Q6_K, 4096, 4096, "attn_in"),
                      ("attn_output", synth.Q4_K_PACKED, 4096, 4096, "attn_out"),
                      ("ffn_gate", synth.Q4_K_PACKED, 11008, 4096, "ffn_in"),
                      ("ffn_up", synth.Q4_K_PACKED, 11008, 4096, "ffn_in"),
                      ("ffn_down", synth.Q6_K, 4096, 11008, "ffn_mid")],
                     False),
    # the same layer with same-type GEMMs that share an input fused by row
    # concatenation at registration: q||k (od 8192) and gate||up (od 22016)
    "layer_fused": ("LLaMA-7B q4_K_M-style layer, 3314 tokens, q||k and gate||up fused",
                    synth.LAYER_TOKENS,
                    {"attn_in": 4096, "attn_out": 4096, "ffn_in": 4096, "ffn_mid": 11008},
                    [("attn_qk", synth.Q4_K, 8192, 4096, "attn_in"),
                     ("attn_v", synth.Q6_K, 4096, 4096, "attn_in"),
                     ("attn_output", synth.Q4_K, 4096, 4096, "attn_out"),
                     ("ffn_gate_up", synth.Q4_K, 22016, 4096, "ffn_in"),
                     ("ffn_down", synth.Q6_K, 4096, 11008, "ffn_mid")],
                    False),
}

# Counter summaries committed under profiles/ (HBM bytes per MMQ launch from
# rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a plain copy's reading); valid
# only while the kernel source is the one they were taken with.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mmq_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "quant_q8_gemm_amd", "csrc", "qmm_mmq.hip")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up steps, run untimed steps for at least this long so the "
                         "shader clock has left its idle state (0: none)")
    ap.add_argument("--workload", default="layer", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-weights pass")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="do not sample power and clock (never sampled under rocprofv3)")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the measured MFMA and epilogue roofs (calibration kernels)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (default: the job's CPU share, OMP_NUM_THREADS where the "
                         "machine sets it, else every CPU this process may run on)")
    ap.add_argument("--cpu-macs", type=float, default=2.4e10,
                    help="multiply-accumulates of the oracle sample (about 20 s of CPU work)")
    return ap.parse_args()


class Telemetry:
    """Socket power and shader clock of GPU 0 while the benchmark runs, from
    `amd-smi metric` started as a child process in a background thread (about
    three samples per second); absent tool or unparsable output: no samples."""

    def __init__(self, enabled=True):
        exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
        exe = os.path.realpath(exe) if os.path.exists(exe) else None
        # the tool is a Python script: run it with this interpreter rather than
        # through its "#!/usr/bin/env" line, one program start fewer
        self.cmd = None if exe is None or not enabled else ([sys.executable, exe] if exe.endswith(".py") else [exe])
        self.samples = []
        self.stop = threading.Event()
        self.thread = None

    def start(self):
        if self.cmd is not None:
            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()

    def _run(self):
        while not self.stop.is_set():
            t = time.perf_counter()
            try:
                r = subprocess.run(self.cmd + ["metric", "-g", "0", "--power", "--clock", "--json"],
                                   capture_output=True, text=True, timeout=10)
                d = json.loads(r.stdout)
                d = d[0] if isinstance(d, list) else d
                g = d["gpu_data"][0] if "gpu_data" in d else d
                watts = float(g["power"]["socket_power"]["value"])
                clks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                        if k.startswith("gfx_") and isinstance(v, dict)
                        and isinstance(v.get("clk", {}).get("value"), (int, float))]
                if clks:
                    self.samples.append((t, watts, float(np.median(clks))))
            except (OSError, ValueError, KeyError, TypeError, IndexError, subprocess.SubprocessError):
                pass
            self.stop.wait(0.2)

    def summary(self, t_from, t_to):
        """Medians over the samples taken in [t_from, t_to] (perf_counter
        seconds), or None; stops the sampling."""
        self.stop.set()
        if self.thread is not None:
            self.thread.join(timeout=15)
        sel = [(w, c) for t, w, c in self.samples if t_from <= t <= t_to]
        if not sel:
            return None
        return {"socket_w_median": round(float(np.median([w for w, _ in sel])), 1),
                "gfx_mhz_median": round(float(np.median([c for _, c in sel])), 1),
                "samples": len(sel),
                "source": "amd-smi metric, GPU 0: socket power; shader clock, median over the XCDs"}


def kernel_hash() -> str:
    """The MMQ kernel's code (its source without comments and blank space, so
    that a comment edit keeps counters taken on the same code valid) and the
    device compiler flags it is built with."""
    spec = importlib.util.spec_from_file_location("qmm_build", os.path.join(ROOT, "quant_q8_gemm_amd", "_build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", open(KERNEL_SRC).read(), flags=re.S)
    h = hashlib.sha256(" ".join(code.split()).encode())
    h.update(" ".join(build.LIB_FLAGS).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes of the MMQ launches of one step from the committed counter
    summary (per launch for single-GEMM workloads), or None if
    there is none for this workload or the kernel changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else w.get("bytes_per_step")


def calibrate(torch, stream):
    """Measured roofs on this GPU: the int8 MFMA rate, the vector-ALU rates of
    the MMQ's scale epilogues (q6_K 3 and q4_K 2.25 instructions per (token,
    row, 32-block), 64 int8 ops each), the rates of the MMQ's whole chunk
    steps without their memory traffic, and MFMAs with and without independent
    FMAs beside them; from the calibration kernels in libqmm_peak.so, with the
    shader clock (s_memtime against the 100 MHz s_memrealtime) during each run.
    Each is the best over a few occupancies and over the kernels built with the
    backend's default and its max-ILP scheduling strategy, timed with HIP
    events on `stream`."""
    import ctypes
    libs = []
    for so in ("libqmm_peak.so", "libqmm_peak_ilp.so"):  # the two scheduling strategies
        lib = ctypes.CDLL(os.path.join(ROOT, "quant_q8_gemm_amd", so))
        lib.qmm_peak_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        libs.append(lib)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    sink = torch.empty(8 * n_cu * 256, dtype=torch.int32, device="cuda")
    out = {}
    # kind, name, work-groups per CU tried, SIMD cycles per wave-iteration, int8 ops per wave-iteration
    for kind, name, per_cu, cyc, ops_it in ((0, "mfma_i8", (1, 2, 3), 128, 4 * 65536),
                                            (1, "epilogue_valu", (2, 4, 8), 192, 65536),
                                            (2, "epilogue_valu_q4k", (2, 4, 8), 1152, 8 * 65536),
                                            (3, "chunk_q4k", (2, 4), 1600, 8 * 65536),
                                            (4, "chunk_q6k", (2, 4), 1700, 8 * 65536),
                                            (5, "mfma_with_fma", (1, 2, 3), 256, 4 * 65536),
                                            (6, "fma_only", (1, 2, 3), 128, 0)):
        best = None
        for lib_i, g in ((li, g) for li in range(len(libs)) for g in per_cu):
            lib = libs[lib_i]
            grid = g * n_cu
            iters = int(8e6 / (g * cyc))  # ~4 ms per launch
            def launch():
                rc = lib.qmm_peak_launch(kind, iters, grid, ctypes.c_void_p(clk.data_ptr()),
                                         ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"qmm_peak_launch({kind}) failed: hipError {rc}")
            launch()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            times = []
            for _ in range(3):
                e[0].record(stream)
                launch()
                e[1].record(stream)
                torch.cuda.synchronize()
                times.append(e[0].elapsed_time(e[1]) / 1e3)
            t = float(np.median(times))
            cycles, ticks = (int(v) for v in clk.cpu())
            tops = grid * 4 * iters * ops_it / t / 1e12
            ghz = cycles / (ticks / 100e6) / 1e9 if ticks > 0 else None
            rec = {"tops": round(tops, 1), "work_groups_per_cu": g, "ms": round(t * 1e3, 3),
                   "clock_ghz": round(ghz, 3) if ghz else None,
                   "schedule": ("default", "max-ilp")[lib_i]}
            if ghz:  # SIMD cycles per wave-iteration: the launch's SIMD cycles over its wave-iterations
                rec["simd_cycles_per_iteration"] = round(t * ghz * 1e9 * 4 * n_cu / (grid * 4 * iters), 1)
            rate = tops if ops_it else -rec.get("simd_cycles_per_iteration", t)
            if best is None or rate > best["_rate"]:
                best = dict(rec, _rate=rate)
        best.pop("_rate")
        if not ops_it:
            best.pop("tops")
        out[name] = best
    mf = out["mfma_i8"]
    mf["pct_of_spec"] = round(100 * mf["tops"] / MFMA_INT8_PEAK_TOPS, 1)
    if mf["clock_ghz"]:
        # 8192 int8 ops per clock per CU (4 SIMDs x 32x32x32 MAC x 2 / 32 cycles)
        mf["spec_at_clock_tops"] = round(n_cu * mf["clock_ghz"] * 1e9 * 8192 / 1e12, 1)
    # do the matrix core and the vector ALU overlap?  Cycles per wave-iteration
    # of 4 MFMAs alone, 64 FMAs alone, and both: overlap 1 means the longer of
    # the two, 0 their sum
    c = [out[k].get("simd_cycles_per_iteration") for k in ("mfma_i8", "fma_only", "mfma_with_fma")]
    if all(c):
        out["mfma_valu_overlap"] = {"mfma_cycles": c[0], "fma_cycles": c[1], "both_cycles": c[2],
                                    "overlap": round((c[0] + c[1] - c[2]) / min(c[0], c[1]), 3)}
    return out


def cpu_threads(requested: int):
    """Oracle threads: the request, else the CPUs this job may use -- where the
    machine states the job's CPU share in OMP_NUM_THREADS that share, else every
    CPU in this process's affinity mask."""
    if requested > 0:
        return requested, "--cpu-threads"
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        return int(share), "OMP_NUM_THREADS (the job's CPU share)"
    return len(os.sched_getaffinity(0)), "all CPUs in the affinity mask"


def cpu_baseline(gemms, raws, xs, T, threads, macs_target):
    """The oracle, as it stands, on a bounded sample of the workload: all tokens,
    the first rows of every GEMM (same fraction for each), rows split over threads."""
    import oracle
    total = sum(T * od * id_ for _, _, od, id_, _ in gemms)
    frac = min(1.0, macs_target / total)
    t0 = time.perf_counter()
    quant = {name: oracle.quantize(x) for name, x in xs.items()}
    t1 = time.perf_counter()
    jobs, macs = [], 0
    for (gname, type_, od, id_, inp) in gemms:
        rows = max(1, int(round(od * frac)))
        macs += T * rows * id_
        bounds = np.linspace(0, rows, threads + 1).astype(int)
        for i in range(threads):
            if bounds[i + 1] > bounds[i]:
                jobs.append((type_, raws[gname], od, id_, quant[inp], int(bounds[i]), int(bounds[i + 1])))

    def work(j):
        type_, raw, od, id_, (q, dh, s), a, b = j
        oracle.mmq_rows(type_, raw, od, id_, q, dh, s, a, b)

    reps = 0
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        while True:  # the whole sample, again until about 10 s have passed
            list(ex.map(work, jobs))
            reps += 1
            if time.perf_counter() - t1 >= 10.0 or reps >= 100:
                break
    t2 = time.perf_counter()
    macs *= reps
    return {
        "value": round(2.0 * macs / (t2 - t0) / 1e12, 6),
        "unit": "effective int8 TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"all {T} tokens x the first {frac * 100:.1f}% of the rows of each GEMM "
                   f"({macs / reps / 1e9:.1f} G multiply-accumulates), run {reps} time(s): q8 quantize "
                   f"of every input on 1 thread ({t1 - t0:.2f} s, once) + the f64 oracle MMQ over "
                   f"{threads} threads ({t2 - t1:.2f} s wall)"),
        "seconds": round(t2 - t0, 3),
    }


def cpu_single_thread(gemms, raws, xs, T, macs_target):
    """The oracle MMQ on one thread over a sample of macs_target multiply-accumulates
    (rows of the first GEMM, activations quantized outside the timing)."""
    import oracle
    gname, type_, od, id_, inp = gemms[0]
    q, dh, s = oracle.quantize(xs[inp])
    rows = max(1, min(od, int(round(macs_target / (T * id_)))))
    t0 = time.perf_counter()
    oracle.mmq_rows(type_, raws[gname], od, id_, q, dh, s, 0, rows)
    dt = time.perf_counter() - t0
    return {"value": round(2.0 * T * rows * id_ / dt / 1e12, 6), "unit": "effective int8 TOPS",
            "cores": 1, "sample": f"{gname}: all {T} tokens x the first {rows} rows", "seconds": round(dt, 3)}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quant_q8_gemm_amd as qmm

    desc, T, inputs, gemms, outliers = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    rng = np.random.default_rng(0)
    raws, weights = {}, {}
    for (gname, type_, od, id_, _) in gemms:
        raws[gname] = synth.weights(rng, type_, od, id_)
        weights[gname] = qmm.register_weights(type_, od, id_, raws[gname])
    xs = {name: synth.activations(rng, T, id_, outliers) for name, id_ in inputs.items()}
    xd = {name: torch.from_numpy(x).cuda() for name, x in xs.items()}
    qacts = {name: torch.empty(qmm.qact_bytes(T, id_), dtype=torch.uint8, device="cuda")
             for name, id_ in inputs.items()}
    outs = {g[0]: torch.empty((T, g[2]), dtype=torch.float32, device="cuda") for g in gemms}
    stream = torch.cuda.current_stream()
    n_in, n_g = len(inputs), len(gemms)

    def prepass(name):
        qmm.quantize_activations(xd[name], qacts[name], stream)

    def gemm(g, w=None):
        gname, _, _, _, inp = g
        qmm.mmq(w or weights[gname], qacts[inp], T, outs[gname], stream)

    def step():
        for name in inputs:
            prepass(name)
        for g in gemms:
            gemm(g)

    # Clock settling: from idle the step runs up to 35% slower for its first
    # ~40 ms while the GPU raises its clocks; the timed steps measure the rate a
    # loaded GPU sustains, whatever --warmup asks for.
    settle_steps = 0
    # no sampler under a profiler: its preloaded library would initialise the GPU
    # in every child process too
    profiled = any(k.startswith("ROCPROF") for k in os.environ)
    telemetry = Telemetry(enabled=not (args.no_telemetry or profiled))
    telemetry.start()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by device synchronization, with
    # nothing but the kernels on the stream (an event record between two kernels
    # costs several microseconds here)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def event_pair():
        return [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    # step spread and the MMQs' time inside the step: K more steps with HIP events
    # (on the stream the kernels run on) at each step's start, between its
    # prepass and its MMQs, and at its end
    evs = [event_pair() + [torch.cuda.Event(enable_timing=True)] for _ in range(args.steps)]
    for k in range(args.steps):
        evs[k][0].record(stream)
        for name in inputs:
            prepass(name)
        evs[k][2].record(stream)
        for g in gemms:
            gemm(g)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    # power and clock over the timed steps and the event-timed ones
    power = telemetry.summary(t0, time.perf_counter())
    span = np.array([e[0].elapsed_time(e[1]) for e in evs])
    mmq_in_step = np.array([e[2].elapsed_time(e[1]) for e in evs])

    # per-kernel durations: every kernel of the step launched K times back to
    # back between two events (an event pair around each single launch would add
    # the event's own cost to every launch)
    kev = [event_pair() for _ in range(n_in + n_g)]
    for i, name in enumerate(inputs):
        kev[i][0].record(stream)
        for _ in range(args.steps):
            prepass(name)
        kev[i][1].record(stream)
    for k, g in enumerate(gemms):
        kev[n_in + k][0].record(stream)
        for _ in range(args.steps):
            gemm(g)
        kev[n_in + k][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([e[0].elapsed_time(e[1]) / args.steps for e in kev])  # [kernel] ms per launch

    # cold weights: copies of every weight, enough that the planes cycled through
    # exceed the last-level cache, one copy per step in turn
    plane_total = sum(w.plane_bytes for w in weights.values())
    n_copies = int(min(8, max(1, -(-COLD_BYTES // plane_total))))
    cold = None
    if n_copies > 1 and not args.no_cold:
        copies = [weights] + [{g: qmm.register_weights(t, od, id_, raws[g]) for g, t, od, id_, _ in gemms}
                              for _ in range(n_copies - 1)]
        for k in range(n_copies):  # one untimed round over the copies
            for g in gemms:
                gemm(g, copies[k][g[0]])
        torch.cuda.synchronize()
        cev = event_pair()
        cev[0].record(stream)
        for k in range(args.steps):
            for g in gemms:
                gemm(g, copies[k % n_copies][g[0]])
        cev[1].record(stream)
        torch.cuda.synchronize()
        cold_ms = cev[0].elapsed_time(cev[1]) / args.steps
        for c in copies[1:]:
            for w in c.values():
                w.release()
        cold = {"copies": n_copies, "planes_cycled_bytes": n_copies * plane_total,
                "mmq_avg_ms": round(float(cold_ms), 4)}
    pre_ms = float(per[:n_in].sum())
    mmq_b2b_ms = float(per[n_in:].sum())
    mmq_ms = float(mmq_in_step.mean())
    ms_per_step = wall * 1e3 / args.steps
    ops = sum(2.0 * T * od * id_ for _, _, od, id_, _ in gemms)
    mmq_avg_s = mmq_ms / 1e3
    mmq_tops = ops / mmq_avg_s / 1e12
    epi_nominal = epilogue_roof(gemms, T, nominal_epilogue_tops)
    pre_bytes = sum(T * id_ * 4 + qmm.qact_bytes(T, id_) for id_ in inputs.values())
    alg_bytes = sum(weights[g].plane_bytes + T * id_ * 9 // 8 + T * od * 4
                    for g, _, od, id_, _ in gemms)
    traffic = measured_traffic(args.workload)
    if cold is not None:
        cold["effective_tops"] = round(ops / (cold["mmq_avg_ms"] / 1e3) / 1e12, 2)

    result = {
        "metric": "effective int8 TOPS (q6_K/q4_K x q8 MMQ, prepass + GEMM per step)",
        "value": round(ops / (ms_per_step / 1e3) / 1e12, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"steps": settle_steps, "ms": round(settle_ms, 1)},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": desc, "n_tok": T,
                   "gemms": [{"name": g, "type": synth.TYPE_NAMES[t], "od": od, "id": id_}
                             for g, t, od, id_, _ in gemms],
                   "parallelism": "single GPU"},
        "pct_int8_mfma_peak": round(100.0 * ops / (ms_per_step / 1e3) / 1e12 / MFMA_INT8_PEAK_TOPS, 2),
        "token_rows_per_s": round(sum(T * g[2] for g in gemms) / (ms_per_step / 1e3), 1),
        "tokens_per_s": round(T / (ms_per_step / 1e3), 1),
        "step_ms_events": {"median": round(float(np.median(span)), 4), "min": round(float(span.min()), 4),
                           "max": round(float(span.max()), 4)},
        "mmq": {"avg_ms": round(mmq_ms, 4), "median_ms": round(float(np.median(mmq_in_step)), 4),
                "min_ms": round(float(mmq_in_step.min()), 4), "max_ms": round(float(mmq_in_step.max()), 4),
                "effective_tops": round(mmq_tops, 2),
                "back_to_back_ms": round(mmq_b2b_ms, 4),
                "back_to_back_tops": round(ops / (mmq_b2b_ms / 1e3) / 1e12, 2),
                "per_gemm_ms": {g[0]: round(float(per[n_in + k]), 4) for k, g in enumerate(gemms)},
                "algorithmic_gb_per_s": round(alg_bytes / mmq_avg_s / 1e9, 1),
                "cold_weights": cold},
        "prepass": {"avg_ms": round(pre_ms, 4),
                    "bytes": pre_bytes,
                    "gb_per_s": round(pre_bytes / (pre_ms / 1e3) / 1e9, 1),
                    "pct_hbm_peak": round(100 * pre_bytes / (pre_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 1),
                    "per_input_ms": {name: round(float(per[i]), 4) for i, name in enumerate(inputs)}},
        "roofline": {
            "kernel": "mmq_kernel",
            "bound": "mfma",
            "achieved": round(mmq_tops, 2),
            "peak": MFMA_INT8_PEAK_TOPS,
            "unit": "TOP/s",
            "frac": round(mmq_tops / MFMA_INT8_PEAK_TOPS, 4),
            "traffic": traffic,
            "algorithmic_ops_per_step": ops,
            "algorithmic_bytes_per_step": alg_bytes,
            "kernel_sha256_16": kernel_hash(),
            # the roof that binds by design: the per-32-block scale epilogue
            "epilogue_roof": {"bound": "alu", "peak": round(epi_nominal, 1),
                              "unit": "TOP/s (int8-equivalent)",
                              "frac": round(mmq_tops / epi_nominal, 4)},
        },
        "plane_bytes": sum(w.plane_bytes for w in weights.values()),
        "raw_weight_bytes": sum(w.raw_bytes for w in weights.values()),
        "telemetry": power,
    }
    # per weight type (registration type): its GEMMs' ops over their
    # back-to-back times, against the int8 peak (and below, its chunk-step roof)
    per_type = {}
    for k, (_, t, od, id_, _) in enumerate(gemms):
        e = per_type.setdefault(synth.TYPE_NAMES[t], {"type": t, "ops": 0.0, "ms": 0.0})
        e["ops"] += 2.0 * T * od * id_
        e["ms"] += float(per[n_in + k])
    result["roofline"]["per_type"] = {
        name: {"ops_per_step": e["ops"], "ms_back_to_back": round(e["ms"], 4),
               "tops": round(e["ops"] / (e["ms"] / 1e3) / 1e12, 2),
               "frac": round(e["ops"] / (e["ms"] / 1e3) / 1e12 / MFMA_INT8_PEAK_TOPS, 4)}
        for name, e in per_type.items()}
    if not args.no_calib:
        # the measured roofs are context for the MMQ's figures: a failure here
        # is reported in the line, not allowed to lose the measurement above
        try:
            cal = calibrate(torch, stream)
        except (OSError, RuntimeError) as e:
            result["calibration"] = {"error": f"{type(e).__name__}: {e}"}
        else:
            result["calibration"] = cal
            rl = result["roofline"]
            rl["measured_peak"] = cal["mfma_i8"]["tops"]
            rl["frac_of_measured_peak"] = round(mmq_tops / cal["mfma_i8"]["tops"], 4)
            measured = {synth.Q6_K: cal["epilogue_valu"]["tops"], synth.Q4_K: cal["epilogue_valu_q4k"]["tops"],
                        synth.Q4_K_PACKED: cal["epilogue_valu_q4k"]["tops"] * EPILOGUE_INSTRS[synth.Q4_K]
                        / EPILOGUE_INSTRS[synth.Q4_K_PACKED]}
            epi_measured = epilogue_roof(gemms, T, measured.get)
            rl["epilogue_roof"]["measured"] = round(epi_measured, 1)
            rl["epilogue_roof"]["frac_of_measured"] = round(mmq_tops / epi_measured, 4)
            # the MMQ's own chunk step (MFMAs, LDS operand reads, vector
            # epilogue) without its global copies and barriers: on this GPU the
            # matrix core's and the vector ALU's times add (mfma_valu_overlap),
            # so this, not the epilogue alone, is the compute ceiling of the
            # kernel's instruction mix.  The packed registration takes q4_K's
            # (its unpack is not in it: a higher roof, a lower fraction).
            chunk = {synth.Q6_K: cal["chunk_q6k"]["tops"], synth.Q4_K: cal["chunk_q4k"]["tops"],
                     synth.Q4_K_PACKED: cal["chunk_q4k"]["tops"]}
            chunk_roof = epilogue_roof(gemms, T, chunk.get)
            rl["chunk_roof"] = {"bound": "mfma+alu", "measured": round(chunk_roof, 1),
                                "unit": "TOP/s (int8-equivalent)",
                                "frac_of_measured": round(mmq_tops / chunk_roof, 4)}
            for name, e in per_type.items():
                rl["per_type"][name]["chunk_roof_frac"] = round(rl["per_type"][name]["tops"] / chunk[e["type"]], 4)
            # the same roofs at the shader clock the steps ran at (the chunk-step
            # kernels run near 2.3 GHz; a loaded GPU at its power limit runs
            # lower): each type's roof scaled by the clock ratio
            cal_ghz = {synth.Q6_K: cal["chunk_q6k"].get("clock_ghz"), synth.Q4_K: cal["chunk_q4k"].get("clock_ghz"),
                       synth.Q4_K_PACKED: cal["chunk_q4k"].get("clock_ghz")}
            if power is not None and all(cal_ghz[t] for _, t, _, _, _ in gemms):
                f = power["gfx_mhz_median"] / 1e3
                at_clock = {t: chunk[t] * f / cal_ghz[t] for t in chunk if cal_ghz[t]}
                roof_f = epilogue_roof(gemms, T, at_clock.get)
                rl["chunk_roof"]["at_step_clock"] = {"clock_ghz": round(f, 3), "measured": round(roof_f, 1),
                                                     "frac": round(mmq_tops / roof_f, 4)}
                for name, e in per_type.items():
                    rl["per_type"][name]["chunk_roof_frac_at_step_clock"] = round(
                        rl["per_type"][name]["tops"] / at_clock[e["type"]], 4)
    if not args.no_cpu:
        threads, rule = cpu_threads(args.cpu_threads)
        result["cpu_baseline"] = cpu_baseline(gemms, raws, xs, T, threads, args.cpu_macs)
        result["cpu_baseline"]["host"] = {"cpu_count": os.cpu_count(),
                                          "affinity_cpus": len(os.sched_getaffinity(0)),
                                          "threads_rule": rule}
        result["cpu_baseline"]["single_thread"] = cpu_single_thread(gemms, raws, xs, T,
                                                                    args.cpu_macs / 4)
    for w in weights.values():
        w.release()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the q4_K/q6_K x q8 prefill MMQ on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the hot path over one batch of synthetic activations that
are already resident in HBM: the q8 quantize prepass followed by the MMQ.  The
weight registration (the once-per-weight repack into planes) happens before the
timed region, as a deployment does it once at model load.

Prints one JSON line: effective int8 TOPS of the whole step (2*T*od*id per step
time), the roofline of the dominant kernel (the MMQ) measured with HIP events on
the stream it runs on, and the CPU oracle timed on the host as a reference.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

WORKLOADS = {
    "ffn_down": synth.C2,       # q6_K 4096 x 11008, 512 tokens
    "ffn_down_odd": synth.C2_ODD,
    "attn": synth.C3_QKVO,
    "ffn_gate_up": synth.C3_GU,
    "head": synth.C4,
    "c1": synth.C1,
}

MFMA_INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA
HBM_PEAK_GBS = 8000.0


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ffn_down", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-threads", type=int, default=0)
    return ap.parse_args()


def algorithmic_bytes(type_, od, id_, T, w):
    """Compulsory HBM bytes of one MMQ launch: the weight planes once, the q8
    activations once, the f32 output once."""
    qact = T * id_ * 9 // 8
    return w.plane_bytes + qact + T * od * 4


def cpu_baseline(type_, od, id_, T, raw, x, threads):
    import oracle
    t0 = time.perf_counter()
    q, dh, s = oracle.quantize(x)
    t1 = time.perf_counter()
    bounds = np.linspace(0, od, threads + 1).astype(int)

    def work(i):
        oracle.mmq_rows(type_, raw, od, id_, q, dh, s, int(bounds[i]), int(bounds[i + 1]))

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(work, range(threads)))
    t2 = time.perf_counter()
    ops = 2.0 * T * od * id_
    return {
        "value": round(ops / (t2 - t0) / 1e12, 6),
        "unit": "effective int8 TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"the whole workload ({T} tokens x {od} rows x {id_}): q8 quantize on 1 thread "
                   f"({t1 - t0:.2f} s) + the f64 oracle MMQ over {threads} threads of row slices "
                   f"({t2 - t1:.2f} s wall)"),
        "seconds": round(t2 - t0, 3),
    }


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quant_q8_gemm_amd as qmm

    name, type_, od, id_, T, outliers = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    raw, x = synth.case(type_, od, id_, T, seed=0, outliers=outliers)
    w = qmm.register_weights(type_, od, id_, raw)
    xd = torch.from_numpy(x).cuda()
    qact = torch.empty(qmm.qact_bytes(T, id_), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, od), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        qmm.quantize_activations(xd, qact, stream)
        if ev is not None:
            ev[1].record(stream)
        qmm.mmq(w, qact, T, out, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by device synchronization
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    mmq_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps
    ops = 2.0 * T * od * id_
    mmq_avg_s = float(mmq_ms.mean()) / 1e3
    mmq_tops = ops / mmq_avg_s / 1e12
    pre_bytes = T * id_ * 4 + qmm.qact_bytes(T, id_)

    result = {
        "metric": "effective int8 TOPS (q6_K/q4_K x q8 MMQ, prepass + GEMM per step)",
        "value": round(ops / (ms_per_step / 1e3) / 1e12, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": name, "type": synth.TYPE_NAMES[type_], "od": od, "id": id_,
                   "n_tok": T, "parallelism": "single GPU"},
        "pct_int8_mfma_peak": round(100.0 * ops / (ms_per_step / 1e3) / 1e12 / MFMA_INT8_PEAK_TOPS, 2),
        "token_rows_per_s": round(T * od / (ms_per_step / 1e3), 1),
        "tokens_per_s": round(T / (ms_per_step / 1e3), 1),
        "mmq": {"avg_ms": round(float(mmq_ms.mean()), 4), "median_ms": round(float(np.median(mmq_ms)), 4),
                "min_ms": round(float(mmq_ms.min()), 4), "max_ms": round(float(mmq_ms.max()), 4),
                "effective_tops": round(mmq_tops, 2)},
        "prepass": {"avg_ms": round(float(pre_ms.mean()), 4),
                    "gb_per_s": round(pre_bytes / (float(pre_ms.mean()) / 1e3) / 1e9, 1),
                    "pct_hbm_peak": round(100 * pre_bytes / (float(pre_ms.mean()) / 1e3) / 1e9 / HBM_PEAK_GBS, 1)},
        "roofline": {
            "kernel": "mmq_kernel",
            "bound": "mfma",
            "achieved": round(mmq_tops, 2),
            "peak": MFMA_INT8_PEAK_TOPS,
            "unit": "TOP/s",
            "frac": round(mmq_tops / MFMA_INT8_PEAK_TOPS, 4),
            "traffic": None,
            "algorithmic_bytes": algorithmic_bytes(type_, od, id_, T, w),
            "algorithmic_ops": ops,
        },
        "plane_bytes": w.plane_bytes,
        "raw_weight_bytes": w.raw_bytes,
    }
    if not args.no_cpu:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        result["cpu_baseline"] = cpu_baseline(type_, od, id_, T, raw, x, threads)
    w.release()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Build libqmm.so (the C-ABI library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
KERNELS = ["qmm_repack.hip", "qmm_prepass.hip", "qmm_mmq.hip"]
SOURCES = [os.path.join(CSRC, "qmm_api.cpp")] + [os.path.join(CSRC, k) for k in KERNELS]
LIB = os.path.join(HERE, "libqmm.so")
# calibration kernels for the benchmark's measured rooflines (not part of the ABI),
# built under the backend's default scheduling strategy and under max-ILP: a
# roof is the better of the two rates
PEAK_SRC = os.path.join(CSRC, "qmm_peak.hip")
PEAK_LIB = os.path.join(HERE, "libqmm_peak.so")
PEAK_LIB_ILP = os.path.join(HERE, "libqmm_peak_ilp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU forms are disabled for the device code on purpose (the host
# pass warns that it does not know the feature; that is harmless).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The MMQ's instruction schedule is set by its sched_group_barriers; the
# backend's max-ILP scheduling strategy orders the rest 1-2% faster on the q4_K
# shapes and equal on the q6_K ones, with bit-identical results.
MAX_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
LIB_FLAGS = DEVICE_FLAGS + MAX_ILP


def _hipcc(sources, out: str, verbose: bool, flags=None) -> str:
    cmd = [HIPCC, *(LIB_FLAGS if flags is None else flags), "-fPIC", "-shared", "-Wall", "-I",
           os.path.join(ROOT, "include"), *sources, "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    _hipcc(SOURCES, LIB, verbose)
    _hipcc([PEAK_SRC], PEAK_LIB, verbose, DEVICE_FLAGS)
    _hipcc([PEAK_SRC], PEAK_LIB_ILP, verbose, DEVICE_FLAGS + MAX_ILP)
    return LIB


def device_asm(out_path: str) -> str:
    """gfx950 assembly of all kernels (for inspection: instruction mix, VGPRs,
    scratch), concatenated into out_path."""
    parts = []
    for k in KERNELS + ["qmm_peak.hip"]:
        tmp = out_path + "." + k + ".s"
        cmd = [HIPCC, *(DEVICE_FLAGS if k == "qmm_peak.hip" else LIB_FLAGS), "--cuda-device-only", "-S", "-I",
               os.path.join(ROOT, "include"), os.path.join(CSRC, k), "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc -S failed:\n" + r.stderr)
        parts.append(open(tmp).read())
        os.remove(tmp)
    with open(out_path, "w") as f:
        f.write("\n".join(parts))
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))

"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code, on the CPU:

* the oracle (plain C) built with gcc -fsanitize=address,undefined runs its
  own pin tests; a copy with a planted out-of-bounds read (one block's d read
  from two bytes past the block) must be reported, which shows the harness
  catches what it is for;
* libqmm with its host code (argument validation, handle accounting, the error
  messages) instrumented -- the device code is compiled as usual -- runs every
  validation path of the C ABI (tests/sanitize/abi_driver.py).

Word/byte stride mistakes in block and plane indexing are the bugs these guard
against.  Neither build is the product: both live in a temporary directory.
"""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
PIN_TESTS = ["tests/test_oracle_f16.py", "tests/test_oracle_decode.py",
             "tests/test_oracle_quantize.py", "tests/test_oracle_mmq.py"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _gcc_asan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build_oracle(src_text, out_dir):
    src = os.path.join(out_dir, "oracle_san.c")
    open(src, "w").write(src_text)
    lib = os.path.join(out_dir, "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "oracle"), src, "-o", lib, "-lm"], check=True)
    return lib


def _run_pins(lib, runtime):
    env = dict(os.environ, QMM_ORACLE_LIB=lib, LD_PRELOAD=runtime, **ENV)
    # --capture=no: a sanitizer report is written to the process's stderr, which
    # pytest's own capture would lose when the report aborts the process
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "--capture=no",
                           *PIN_TESTS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    runtime = _gcc_asan()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = _build_oracle(open(ORACLE_SRC).read(), str(tmp_path))
    r = _run_pins(lib, runtime)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out, out[-3000:]


def test_planted_out_of_bounds_read_is_reported(tmp_path):
    runtime = _gcc_asan()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(ORACLE_SRC).read()
    anchor = "*d = oracle_f16_to_f32((uint16_t)(B[208] | (B[209] << 8)));"
    assert src.count(anchor) == 1
    lib = _build_oracle(src.replace(anchor, "*d = oracle_f16_to_f32((uint16_t)(B[210] | (B[211] << 8)));"),
                        str(tmp_path))
    r = _run_pins(lib, runtime)
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in r.stdout + r.stderr


def test_library_validation_paths_under_asan_and_ubsan(tmp_path):
    runtime = _clang_asan()
    if runtime is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    # the library's own source list (the build module, loaded without importing the package)
    spec = importlib.util.spec_from_file_location("qmm_build", os.path.join(ROOT, "quant_q8_gemm_amd", "_build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    lib = str(tmp_path / "libqmm_san.so")
    # the sanitizers go to the host compilation only (each right after -Xarch_host)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           *build.SOURCES,
           "-o", lib]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, **ENV)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "abi_driver.py"), lib],
                       env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out, out[-3000:]

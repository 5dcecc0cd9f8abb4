"""CPU check that __graft_entry__.build() works on a tree where nothing is built
yet: the package refuses to import without its library, so the build must not
go through the package import."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_from_a_tree_with_no_built_library(tmp_path):
    def no_built(_dir, names):
        return [n for n in names if n.endswith((".so", ".tmp")) or n == "__pycache__"]

    for sub in ("quant_q8_gemm_amd", "include", "oracle"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub, ignore=no_built)
    for f in ("__graft_entry__.py", "synth.py"):
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    assert not (tmp_path / "quant_q8_gemm_amd" / "libqmm.so").exists()
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert (tmp_path / "quant_q8_gemm_amd" / "libqmm.so").exists()
    assert (tmp_path / "oracle" / "liboracle.so").exists()

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Build the C-ABI library and the oracle only if nothing is built yet.
if not os.path.exists(os.path.join(ROOT, "quant_q8_gemm_amd", "libqmm.so")):
    import __graft_entry__
    __graft_entry__._load_build_module().build()
if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
    import oracle
    oracle.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")

"""The allocation-free MMQ entry point (qmm_mmq_noalloc) through the C ABI: its
output equals qmm_mmq's bit for bit and lies within 1e-4 * sum|terms| of the
oracle, on two calls in a row whose launches split tail tiles along K (so the
static tail scratch is used), the second with a smaller input; then a launch
with no tail."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import quant_q8_gemm_amd as qmm  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(entry, w, qact, T):
    out = torch.full((T, w.od), float("nan"), dtype=torch.float32, device="cuda")
    entry(w, qact, T, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_mmq_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    # a ragged second wave (264 tiles on 256 CUs: the tail split 21 ways), then
    # a smaller launch that splits every one of its 24 tiles, then no tail
    cases = [(synth.Q6_K, 4200, 768, 500, 41), (synth.Q4_K, 512, 3072, 300, 42), (synth.Q4_K, 96, 512, 40, 43)]
    for type_, od, id_, T, seed in cases:
        print(f"noalloc {synth.TYPE_NAMES[type_]} {od}x{id_} T={T}", flush=True)
        sys.stdout.flush()
        raw, x = synth.case(type_, od, id_, T, seed=seed)
        w = qmm.register_weights(type_, od, id_, raw)
        qact = qmm.quantize_activations(torch.from_numpy(x).cuda())
        got = _run(qmm.mmq_noalloc, w, qact, T)
        ref = _run(qmm.mmq, w, qact, T)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        q, dh, s = oracle.quantize(x)
        exact, A = oracle.mmq(type_, raw, od, id_, q, dh, s)
        assert np.all(np.abs(got.astype(np.float64) - exact) <= 1e-4 * A)
        w.release()

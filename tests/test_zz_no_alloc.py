"""The allocation-free MMQ entry point (qmm_mmq_noalloc) through the C ABI: its
output equals qmm_mmq's bit for bit and lies within 1e-4 * sum|terms| of the
oracle, on two calls in a row whose launches split tail tiles along K (so the
static tail scratch is used), the second with a smaller input; then a ragged
second wave's split tail and a launch with no tail."""
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
    # every tile split along K (24 tiles of 64 x 128, 6 slices each), then a
    # smaller input that splits the same tiles 2 ways into a prefix of the
    # scratch still holding the first call's partials, then a ragged second wave
    # (260 tiles on 256 CUs: the 4 tail tiles split 4 ways), then no tail
    cases = [(synth.Q4_K, 512, 3072, 300, 42), (synth.Q4_K, 512, 1024, 300, 44), (synth.Q6_K, 4160, 2048, 512, 41),
             (synth.Q4_K, 96, 512, 40, 43)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    scratch = [qmm.mmq_plan(t, od, id_, T, cus).scratch_bytes for t, od, id_, T, _ in cases]
    if cus == 256:  # MI355X: the plans above use the static scratch as described
        assert scratch[0] > scratch[1] > scratch[2] > 0 and scratch[3] == 0, scratch
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

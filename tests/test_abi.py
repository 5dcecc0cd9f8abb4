"""CPU-only checks of the C ABI: the library loads, exports every entry point the
header declares, sizes the qact buffer as documented, and rejects invalid
arguments before touching HIP (so these run on machines without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import quant_q8_gemm_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert _declared() == sorted(qmm.EXPORTS)


@pytest.mark.parametrize("name", _declared())
def test_library_exports_every_declared_symbol(name):
    lib = ctypes.CDLL(qmm.LIB_PATH)
    assert hasattr(lib, name)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (QMM_[A-Z0-9_]+) \(?(-?\d+)\)?", text))
    assert int(consts["QMM_Q4_K"]) == qmm.Q4_K and int(consts["QMM_Q6_K"]) == qmm.Q6_K
    assert int(consts["QMM_Q4_K_PACKED"]) == qmm.Q4_K_PACKED
    assert int(consts["QMM_EINVAL"]) == qmm.EINVAL and int(consts["QMM_ESHAPE"]) == qmm.ESHAPE
    assert int(consts["QMM_ENOMEM"]) == qmm.ENOMEM and int(consts["QMM_EHIP"]) == qmm.EHIP
    assert int(consts["QMM_TOKEN_PAD"]) == qmm.TOKEN_PAD


@pytest.mark.parametrize("n_tok,id_,expect", [
    (1, 256, 128 * 256 * 9 // 8), (128, 256, 128 * 256 * 9 // 8), (129, 512, 256 * 512 * 9 // 8),
    (509, 11008, 512 * 11008 * 9 // 8), (3314, 4096, 3328 * 4096 * 9 // 8),
    (0, 256, 0), (5, 100, 0), (5, 288, 0), (5, 0, 0), (-1, 256, 0)])
def test_qact_bytes(n_tok, id_, expect):
    assert qmm.qact_bytes(n_tok, id_) == expect


def _reg(type_, od, id_, nbytes=None, ptr=True):
    L = qmm._lib
    buf = np.zeros(max(nbytes or 0, 1), np.uint8)
    h = ctypes.c_void_p()
    rc = L.qmm_register_weights(type_, od, id_, buf.ctypes.data_as(ctypes.c_void_p) if ptr else None,
                                nbytes if nbytes is not None else 0, None, ctypes.byref(h))
    return rc, h.value


@pytest.mark.parametrize("type_,od,id_,nbytes", [
    (5, 4, 256, 4 * 210), (qmm.Q6_K, 0, 256, 0), (qmm.Q6_K, 4, 255, 4 * 210),
    (qmm.Q6_K, 4, 384, 4 * 210), (qmm.Q4_K, 4, 256, 4 * 210), (qmm.Q6_K, 4, 256, 4 * 210 - 1),
    (qmm.Q6_K, (1 << 21) + 1, 256, 0), (qmm.Q4_K, 3, 1 << 21, 0)])
def test_register_rejects_bad_arguments(type_, od, id_, nbytes):
    rc, h = _reg(type_, od, id_, nbytes)
    assert rc == qmm.EINVAL and h is None
    assert qmm.last_error()


def test_register_rejects_null_pointers():
    rc, _ = _reg(qmm.Q6_K, 1, 256, 210, ptr=False)
    assert rc == qmm.EINVAL
    buf = np.zeros(210, np.uint8)
    rc = qmm._lib.qmm_register_weights(qmm.Q6_K, 1, 256, buf.ctypes.data_as(ctypes.c_void_p), 210,
                                       None, None)
    assert rc == qmm.EINVAL


def test_memory_cap_fails_before_allocating():
    qmm.set_memory_cap(1000)
    try:
        rc, h = _reg(qmm.Q6_K, 4, 256, 4 * 210)
        assert rc == qmm.ENOMEM and h is None
        assert "cap" in qmm.last_error()
    finally:
        qmm.set_memory_cap(0)


def test_memory_cap_reservation_is_given_back_on_failure():
    """With the cap at exactly one registration's bytes, two registrations in a
    row must both get past the cap: a failed one (no GPU here) returns what it
    reserved, a successful one is released before the next."""
    qmm.set_memory_cap(1000)
    try:
        rc, _ = _reg(qmm.Q6_K, 4, 256, 4 * 210)
        assert rc == qmm.ENOMEM
        need = int(re.search(r"needs (\d+) device bytes", qmm.last_error()).group(1))
        qmm.set_memory_cap(need)
        for _ in range(2):
            rc, h = _reg(qmm.Q6_K, 4, 256, 4 * 210)
            assert rc != qmm.ENOMEM, qmm.last_error()
            if rc == qmm.OK:
                qmm._lib.qmm_release_weights(ctypes.c_void_p(h))
            else:
                assert rc == qmm.EHIP and h is None
    finally:
        qmm.set_memory_cap(0)


def test_quantize_rejects_bad_arguments():
    L = qmm._lib
    good = ctypes.c_void_p(4096)
    n = qmm.qact_bytes(4, 256)
    assert L.qmm_quantize_activations(good, 0, 256, good, n, None) == qmm.EINVAL
    assert L.qmm_quantize_activations(good, 4, 300, good, n, None) == qmm.EINVAL
    assert L.qmm_quantize_activations(None, 4, 256, good, n, None) == qmm.EINVAL
    assert L.qmm_quantize_activations(good, 4, 256, None, n, None) == qmm.EINVAL
    assert L.qmm_quantize_activations(ctypes.c_void_p(4100), 4, 256, good, n, None) == qmm.EINVAL
    assert L.qmm_quantize_activations(good, 4, 256, ctypes.c_void_p(4104), n, None) == qmm.EINVAL
    assert L.qmm_quantize_activations(good, 4, 256, good, n - 1, None) == qmm.EINVAL
    assert "qact_bytes" in qmm.last_error()
    assert L.qmm_quantize_activations(good, -1, 256, good, 0, None) == qmm.EINVAL


def test_quantize_empty_batch_is_a_no_op():
    """n_tok = 0 is valid: nothing to write, no pointer or device is touched (so
    it succeeds without a GPU); a non-zero qact_bytes or a bad id still fails."""
    L = qmm._lib
    assert L.qmm_quantize_activations(None, 0, 256, None, 0, None) == qmm.OK
    assert qmm.last_error() == ""
    assert L.qmm_quantize_activations(None, 0, 256, None, 16, None) == qmm.EINVAL
    assert L.qmm_quantize_activations(None, 0, 300, None, 0, None) == qmm.EINVAL


@pytest.mark.parametrize("entry", ["qmm_mmq", "qmm_mmq_noalloc"])
def test_mmq_rejects_bad_arguments(entry):
    """Both MMQ entry points share their validation: a null handle fails before
    any HIP call, and an empty batch with a null handle still fails."""
    f = getattr(qmm._lib, entry)
    good = ctypes.c_void_p(4096)
    assert f(None, good, 100, 4, good, None) == qmm.EINVAL
    assert "handle" in qmm.last_error()
    assert f(None, None, 0, 0, None, None) == qmm.EINVAL


def test_info_and_export_reject_null():
    L = qmm._lib
    info = qmm.Info()
    assert L.qmm_weights_info(None, ctypes.byref(info)) == qmm.EINVAL
    assert L.qmm_weights_export(None, ctypes.c_void_p(4096), 10) == qmm.EINVAL
    L.qmm_release_weights(None)  # no-op


def test_info_struct_matches_header():
    """The binding's qmm_info mirror has the header's fields, in order."""
    import re
    hdr = open(os.path.join(ROOT, "include", "qmm.h")).read()
    body = re.search(r"typedef struct \{(.*?)\} qmm_info;", hdr, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"(\w+)\s*;", body)
    assert names == [f[0] for f in qmm.Info._fields_]


@pytest.mark.parametrize("so", ["libqmm_peak.so", "libqmm_peak_ilp.so"])
def test_calibration_library_loads_and_validates(so):
    """The benchmark's calibration kernels (measured MFMA and epilogue roofs)
    live in their own library, built under two scheduling strategies; invalid
    arguments are refused before any HIP call (hipErrorInvalidValue = 1)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "quant_q8_gemm_amd", so))
    f = lib.qmm_peak_launch
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    good = ctypes.c_void_p(4096)
    assert f(7, 10, 1, good, good, None) == 1
    assert f(-1, 10, 1, good, good, None) == 1
    assert f(0, 0, 1, good, good, None) == 1
    assert f(1, 10, 0, good, good, None) == 1
    assert f(0, 10, 1, None, good, None) == 1


def test_binding_rejects_wrong_qact_tensors():
    """The binding passes byte counts from the tensor: a qact that is not a flat
    uint8 device tensor is refused before any library call."""
    import torch
    with pytest.raises(qmm.QmmError):
        qmm._check_qact(torch.zeros(16, dtype=torch.float32))
    with pytest.raises(qmm.QmmError):
        qmm._check_qact(torch.zeros(16, dtype=torch.uint8))  # host memory


def test_stream_release_of_a_stream_without_scratch_is_a_no_op():
    """No scratch was allocated for these streams: the call returns QMM_OK
    before any HIP call (so it works without a GPU)."""
    freed = ctypes.c_size_t(7)
    assert qmm._lib.qmm_stream_release(ctypes.c_void_p(0x1234), ctypes.byref(freed)) == 0
    assert freed.value == 0
    assert qmm._lib.qmm_stream_release(None, None) == 0

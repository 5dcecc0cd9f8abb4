"""Python binding of libqmm (include/qmm.h): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; PyTorch is used
only to hold device memory and to name the stream.  If libqmm.so has not been
built, importing this package raises immediately -- there is no other path.

    import quant_q8_gemm_amd as qmm
    w = qmm.register_weights(qmm.Q6_K, od, id, raw_bytes)      # numpy uint8
    qact = qmm.quantize_activations(x)                          # x: cuda f32 [T][id]
    out = qmm.mmq(w, qact, n_tok)                               # cuda f32 [T][od]
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python quant_q8_gemm_amd/_build.py or "
        "__graft_entry__.build()); there is no fallback implementation")

# One HIP runtime per process: PyTorch ships its own libamdhip64 under the same
# soname.  Loading torch first makes libqmm bind to that runtime; loading libqmm
# first would pull in a second runtime that cannot see the device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# keep in step with include/qmm.h
Q4_K = 4
Q6_K = 6
Q4_K_PACKED = 14  # q4_K blocks, codes kept two per byte on the device
OK = 0
EINVAL = -1
ESHAPE = -2
ENOMEM = -3
EHIP = -4
TOKEN_PAD = 128
BLOCK_BYTES = {Q4_K: 144, Q4_K_PACKED: 144, Q6_K: 210}

# The full list of entry points include/qmm.h declares.
EXPORTS = ("qmm_register_weights", "qmm_weights_info", "qmm_weights_export", "qmm_release_weights",
           "qmm_set_memory_cap", "qmm_qact_bytes", "qmm_quantize_activations", "qmm_mmq",
           "qmm_mmq_noalloc", "qmm_stream_release", "qmm_mmq_plan", "qmm_mmq_plan_work", "qmm_last_error")
MAX_CUS = 65536


class Info(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("od", ctypes.c_int64), ("id", ctypes.c_int64),
                ("od_pad", ctypes.c_int64), ("raw_bytes", ctypes.c_size_t),
                ("plane_bytes", ctypes.c_size_t), ("wd_offset", ctypes.c_size_t),
                ("sm_offset", ctypes.c_size_t)]


class Plan(ctypes.Structure):
    _fields_ = [("work_groups", ctypes.c_int64), ("scratch_bytes", ctypes.c_size_t),
                ("threads", ctypes.c_int32), ("many", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("k_groups", ctypes.c_int32), ("per_cu", ctypes.c_int32),
                ("row_tiles", ctypes.c_int32), ("tok_tiles", ctypes.c_int32), ("dp_row_tiles", ctypes.c_int32),
                ("n_tail", ctypes.c_int32), ("split", ctypes.c_int32), ("nsb", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_lib.qmm_register_weights.argtypes = [ctypes.c_int, _I64, _I64, _P, _SZ, _P, ctypes.POINTER(_P)]
_lib.qmm_register_weights.restype = ctypes.c_int
_lib.qmm_weights_info.argtypes = [_P, ctypes.POINTER(Info)]
_lib.qmm_weights_info.restype = ctypes.c_int
_lib.qmm_weights_export.argtypes = [_P, _P, _SZ]
_lib.qmm_weights_export.restype = ctypes.c_int
_lib.qmm_release_weights.argtypes = [_P]
_lib.qmm_release_weights.restype = None
_lib.qmm_set_memory_cap.argtypes = [_SZ]
_lib.qmm_set_memory_cap.restype = None
_lib.qmm_qact_bytes.argtypes = [_I64, _I64]
_lib.qmm_qact_bytes.restype = _SZ
_lib.qmm_quantize_activations.argtypes = [_P, _I64, _I64, _P, _SZ, _P]
_lib.qmm_quantize_activations.restype = ctypes.c_int
_lib.qmm_mmq.argtypes = [_P, _P, _SZ, _I64, _P, _P]
_lib.qmm_mmq.restype = ctypes.c_int
_lib.qmm_mmq_noalloc.argtypes = [_P, _P, _SZ, _I64, _P, _P]
_lib.qmm_mmq_noalloc.restype = ctypes.c_int
_lib.qmm_stream_release.argtypes = [_P, ctypes.POINTER(_SZ)]
_lib.qmm_stream_release.restype = ctypes.c_int
_lib.qmm_mmq_plan.argtypes = [ctypes.c_int, _I64, _I64, _I64, ctypes.c_int, ctypes.POINTER(Plan)]
_lib.qmm_mmq_plan.restype = ctypes.c_int
_I32P = ctypes.POINTER(ctypes.c_int32)
_lib.qmm_mmq_plan_work.argtypes = [ctypes.POINTER(Plan), _I64, _I32P, _I32P, _I32P, _I32P]
_lib.qmm_mmq_plan_work.restype = ctypes.c_int
_lib.qmm_last_error.argtypes = []
_lib.qmm_last_error.restype = ctypes.c_char_p


class QmmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"qmm error {code}: {message}")
        self.code = code


def last_error() -> str:
    return _lib.qmm_last_error().decode()


def _check(rc: int) -> None:
    if rc != OK:
        raise QmmError(rc, last_error())


def _check_qact(qact) -> None:
    import torch
    if qact.dtype != torch.uint8 or not qact.is_cuda or qact.dim() != 1 or not qact.is_contiguous():
        raise QmmError(EINVAL, "qact must be a contiguous one-dimensional cuda uint8 tensor")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def set_memory_cap(nbytes: int) -> None:
    _lib.qmm_set_memory_cap(int(nbytes))


def qact_bytes(n_tok: int, id_: int) -> int:
    return int(_lib.qmm_qact_bytes(int(n_tok), int(id_)))


class Weights:
    """A registered weight matrix (device planes owned by the library)."""

    def __init__(self, handle: int):
        self._h = handle
        info = Info()
        _check(_lib.qmm_weights_info(ctypes.c_void_p(handle), ctypes.byref(info)))
        self.type = info.type
        self.od = info.od
        self.id = info.id
        self.od_pad = info.od_pad
        self.raw_bytes = info.raw_bytes
        self.plane_bytes = info.plane_bytes
        self.wd_offset = info.wd_offset
        self.sm_offset = info.sm_offset

    @property
    def handle(self) -> int:
        if self._h is None:
            raise QmmError(EINVAL, "weights already released")
        return self._h

    def export(self) -> np.ndarray:
        """Host copy of the device planes (layout: include/qmm.h, qmm_weights_export)."""
        buf = np.empty(self.plane_bytes, np.uint8)
        _check(_lib.qmm_weights_export(ctypes.c_void_p(self.handle),
                                       buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes))
        return buf

    def release(self) -> None:
        if self._h is not None:
            _lib.qmm_release_weights(ctypes.c_void_p(self._h))
            self._h = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


def register_weights(type_: int, od: int, id_: int, raw, stream=None) -> Weights:
    """Copy k-quant bytes (host numpy/bytes, od x (id/256) blocks) to the device and
    expand them into the library's planes."""
    buf = np.ascontiguousarray(np.frombuffer(raw, np.uint8) if isinstance(raw, (bytes, bytearray))
                               else np.asarray(raw, np.uint8).reshape(-1))
    h = ctypes.c_void_p()
    _check(_lib.qmm_register_weights(int(type_), int(od), int(id_),
                                     buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes,
                                     _stream(stream), ctypes.byref(h)))
    return Weights(h.value)


def quantize_activations(x, qact=None, stream=None):
    """x: cuda float32 [n_tok][id] contiguous -> qact (cuda uint8, qact_bytes)."""
    import torch
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise QmmError(EINVAL, "x must be a contiguous cuda float32 [n_tok][id] tensor")
    n_tok, id_ = x.shape
    nb = qact_bytes(n_tok, id_)
    if qact is None:
        if nb == 0 and n_tok != 0:
            raise QmmError(EINVAL, f"bad shape n_tok={n_tok} id={id_}")
        qact = torch.empty(nb, dtype=torch.uint8, device=x.device)
    _check_qact(qact)
    _check(_lib.qmm_quantize_activations(ctypes.c_void_p(x.data_ptr()), n_tok, id_,
                                         ctypes.c_void_p(qact.data_ptr()), qact.numel(),
                                         _stream(stream)))
    return qact


def _mmq_args(w: Weights, qact, n_tok: int, out):
    import torch
    _check_qact(qact)
    if out is None:
        out = torch.empty((n_tok, w.od), dtype=torch.float32, device=qact.device)
    elif (out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous()
          or tuple(out.shape) != (n_tok, w.od)):
        raise QmmError(EINVAL, "out must be a contiguous cuda float32 [n_tok][od] tensor")
    return out


def mmq(w: Weights, qact, n_tok: int, out=None, stream=None):
    """out[t][j] (cuda float32 [n_tok][od]) from a handle and a qact buffer."""
    out = _mmq_args(w, qact, n_tok, out)
    _check(_lib.qmm_mmq(ctypes.c_void_p(w.handle), ctypes.c_void_p(qact.data_ptr()), qact.numel(),
                        int(n_tok), ctypes.c_void_p(out.data_ptr()), _stream(stream)))
    return out


def mmq_noalloc(w: Weights, qact, n_tok: int, out, stream=None):
    """mmq through the allocation-free entry point (the caller passes out)."""
    out = _mmq_args(w, qact, n_tok, out)
    _check(_lib.qmm_mmq_noalloc(ctypes.c_void_p(w.handle), ctypes.c_void_p(qact.data_ptr()), qact.numel(),
                                int(n_tok), ctypes.c_void_p(out.data_ptr()), _stream(stream)))
    return out


def stream_release(stream=None) -> int:
    """Free the MMQ scratch the library keeps for `stream` (torch's current
    stream if None); synchronizes the stream first.  Returns the bytes freed."""
    freed = _SZ(0)
    _check(_lib.qmm_stream_release(_stream(stream), ctypes.byref(freed)))
    return int(freed.value)


def mmq_plan(type_: int, od: int, id_: int, n_tok: int, num_cus: int) -> Plan:
    """The launch plan qmm_mmq follows for this shape on a GPU with num_cus
    compute units (host arithmetic only; no device needed)."""
    plan = Plan()
    _check(_lib.qmm_mmq_plan(int(type_), int(od), int(id_), int(n_tok), int(num_cus), ctypes.byref(plan)))
    return plan


def mmq_plan_work(plan: Plan, wg: int):
    """(row tile, token tile, first super-block, end super-block) that
    work-group wg of the plan's launch computes."""
    out = [ctypes.c_int32() for _ in range(4)]
    _check(_lib.qmm_mmq_plan_work(ctypes.byref(plan), int(wg), *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)

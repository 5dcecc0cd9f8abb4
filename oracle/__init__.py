"""Python access to the plain C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark import this module; the product library never
does, and the product path must never route through it.

Every function takes and returns numpy arrays.  The C side is compiled with gcc
(``build()``) into ``liboracle.so`` next to this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A different build of the same source may be named here (used by the test that
# plants mistakes in copies of oracle.c to show the pins catch them).
_LOAD_PATH = os.environ.get("QMM_ORACLE_LIB", _LIB_PATH)

Q4_K = 4
Q6_K = 6
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}

_lib = None


def build() -> str:
    """Compile liboracle.so with plain gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LOAD_PATH == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LOAD_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_decode_q6k.argtypes = [P, I64, I64, P, P, P]
    lib.oracle_decode_q6k.restype = None
    lib.oracle_decode_q4k.argtypes = [P, I64, I64, P, P, P, P, P]
    lib.oracle_decode_q4k.restype = None
    lib.oracle_quantize.argtypes = [P, I64, I64, P, P, P]
    lib.oracle_quantize.restype = ctypes.c_int
    lib.oracle_dots_q6k.argtypes = [P, I64, I64, P, I64, P, P]
    lib.oracle_dots_q6k.restype = None
    lib.oracle_dots_q4k.argtypes = [P, I64, I64, P, I64, P]
    lib.oracle_dots_q4k.restype = None
    lib.oracle_mmq.argtypes = [ctypes.c_int, P, I64, I64, P, P, P, I64, P, P]
    lib.oracle_mmq.restype = ctypes.c_int
    lib.oracle_mmq_at.argtypes = [ctypes.c_int, P, I64, I64, P, P, P, I64, I64, P, P, P, P]
    lib.oracle_mmq_at.restype = ctypes.c_int
    lib.oracle_mmq_rows.argtypes = [ctypes.c_int, P, I64, I64, P, P, P, I64, I64, I64, P, P]
    lib.oracle_mmq_rows.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _raw_check(type_: int, raw: np.ndarray, od: int, id_: int) -> np.ndarray:
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    if type_ not in BLOCK_BYTES or id_ % 256 or od < 1:
        raise ValueError("bad type or shape")
    if raw.size != od * (id_ // 256) * BLOCK_BYTES[type_]:
        raise ValueError("raw byte count does not match od x id")
    return raw


# --- binary16 --------------------------------------------------------------

def f16_to_f64(h: int) -> float:
    return _load().oracle_f16_to_f64(int(h))


def f32_to_f16(f: float) -> int:
    return int(_load().oracle_f32_to_f16(float(np.float32(f))))


def f32_to_f16_array(x: np.ndarray) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.oracle_f32_to_f16(float(v)) for v in x], dtype=np.uint16)


def f16_to_f64_array(h: np.ndarray) -> np.ndarray:
    lib = _load()
    h = np.asarray(h, dtype=np.uint16).ravel()
    return np.array([lib.oracle_f16_to_f64(int(v)) for v in h], dtype=np.float64)


# --- O1 --------------------------------------------------------------------

def decode_q6k(raw: np.ndarray, od: int, id_: int):
    """Returns (w = q - 32 [od][id] int8, sc [od][id/16] int8, d [od][id/256] f32)."""
    raw = _raw_check(Q6_K, raw, od, id_)
    w = np.empty((od, id_), np.int8)
    sc = np.empty((od, id_ // 16), np.int8)
    d = np.empty((od, id_ // 256), np.float32)
    _load().oracle_decode_q6k(_ptr(raw), od, id_, _ptr(w), _ptr(sc), _ptr(d))
    return w, sc, d


def decode_q4k(raw: np.ndarray, od: int, id_: int):
    """Returns (w = 4-bit codes [od][id] uint8, sc [od][id/32], mn [od][id/32],
    d [od][id/256] f32, dmin [od][id/256] f32)."""
    raw = _raw_check(Q4_K, raw, od, id_)
    w = np.empty((od, id_), np.uint8)
    sc = np.empty((od, id_ // 32), np.uint8)
    mn = np.empty((od, id_ // 32), np.uint8)
    d = np.empty((od, id_ // 256), np.float32)
    dm = np.empty((od, id_ // 256), np.float32)
    _load().oracle_decode_q4k(_ptr(raw), od, id_, _ptr(w), _ptr(sc), _ptr(mn), _ptr(d), _ptr(dm))
    return w, sc, mn, d, dm


# --- O2 --------------------------------------------------------------------

def quantize(x: np.ndarray):
    """x [n_tok][id] f32 -> (q [n_tok][id] int8, dh [n_tok][id/32] uint16 (f16 bits),
    s [n_tok][id/32] uint16 (f16 bits))."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n_tok, id_ = x.shape
    q = np.empty((n_tok, id_), np.int8)
    dh = np.empty((n_tok, id_ // 32), np.uint16)
    s = np.empty((n_tok, id_ // 32), np.uint16)
    rc = _load().oracle_quantize(_ptr(x), n_tok, id_, _ptr(q), _ptr(dh), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_quantize: input not finite, out of range or bad shape")
    return q, dh, s


# --- O3 --------------------------------------------------------------------

def dots_q6k(raw: np.ndarray, od: int, id_: int, q: np.ndarray):
    """Returns (D16 [T][od][id/16] int32, J [T][od][id/32] int32)."""
    raw = _raw_check(Q6_K, raw, od, id_)
    q = np.ascontiguousarray(q, dtype=np.int8)
    T = q.shape[0]
    D16 = np.empty((T, od, id_ // 16), np.int32)
    J = np.empty((T, od, id_ // 32), np.int32)
    _load().oracle_dots_q6k(_ptr(raw), od, id_, _ptr(q), T, _ptr(D16), _ptr(J))
    return D16, J


def dots_q4k(raw: np.ndarray, od: int, id_: int, q: np.ndarray):
    """Returns D32 [T][od][id/32] int32."""
    raw = _raw_check(Q4_K, raw, od, id_)
    q = np.ascontiguousarray(q, dtype=np.int8)
    T = q.shape[0]
    D32 = np.empty((T, od, id_ // 32), np.int32)
    _load().oracle_dots_q4k(_ptr(raw), od, id_, _ptr(q), T, _ptr(D32))
    return D32


# --- O4 --------------------------------------------------------------------

def _act_check(q, dh, s, id_):
    q = np.ascontiguousarray(q, dtype=np.int8)
    dh = np.ascontiguousarray(dh, dtype=np.uint16)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    T = q.shape[0]
    if q.shape != (T, id_) or dh.shape != (T, id_ // 32) or s.shape != (T, id_ // 32):
        raise ValueError("activation shapes do not match id")
    return q, dh, s, T


def mmq(type_: int, raw: np.ndarray, od: int, id_: int, q, dh, s):
    """Full result: (out [T][od] f64, A [T][od] f64 = sum of |terms|)."""
    raw = _raw_check(type_, raw, od, id_)
    q, dh, s, T = _act_check(q, dh, s, id_)
    out = np.empty((T, od), np.float64)
    A = np.empty((T, od), np.float64)
    rc = _load().oracle_mmq(type_, _ptr(raw), od, id_, _ptr(q), _ptr(dh), _ptr(s), T,
                            _ptr(out), _ptr(A))
    if rc:
        raise ValueError("oracle_mmq failed")
    return out, A


def mmq_rows(type_: int, raw: np.ndarray, od: int, id_: int, q, dh, s, j0: int, j1: int):
    """Result for weight rows [j0, j1): (out [T][j1-j0], A [T][j1-j0])."""
    raw = _raw_check(type_, raw, od, id_)
    q, dh, s, T = _act_check(q, dh, s, id_)
    out = np.empty((T, j1 - j0), np.float64)
    A = np.empty((T, j1 - j0), np.float64)
    rc = _load().oracle_mmq_rows(type_, _ptr(raw), od, id_, _ptr(q), _ptr(dh), _ptr(s), T,
                                 j0, j1, _ptr(out), _ptr(A))
    if rc:
        raise ValueError("oracle_mmq_rows failed")
    return out, A


def mmq_parallel(type_: int, raw: np.ndarray, od: int, id_: int, q, dh, s, threads: int = 0):
    """mmq() with the rows split into blocks that oracle_mmq_rows computes on
    separate threads (the C call releases the GIL); the arithmetic of every
    element is mmq()'s.  threads = 0: OMP_NUM_THREADS, else the CPUs in this
    process's affinity mask."""
    import concurrent.futures as cf
    raw = _raw_check(type_, raw, od, id_)
    q, dh, s, T = _act_check(q, dh, s, id_)
    if threads <= 0:
        env = os.environ.get("OMP_NUM_THREADS", "")
        threads = int(env) if env.isdigit() and int(env) > 0 else len(os.sched_getaffinity(0))
    out = np.empty((T, od), np.float64)
    A = np.empty((T, od), np.float64)
    bounds = np.linspace(0, od, min(od, 4 * threads) + 1).astype(int)

    def work(i):
        j0, j1 = int(bounds[i]), int(bounds[i + 1])
        if j1 > j0:
            o, a = mmq_rows(type_, raw, od, id_, q, dh, s, j0, j1)
            out[:, j0:j1] = o
            A[:, j0:j1] = a

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(work, range(len(bounds) - 1)))
    return out, A


def mmq_at(type_: int, raw: np.ndarray, od: int, id_: int, q, dh, s, ts, js):
    """Result at the (ts[i], js[i]) pairs: (out [n], A [n]).  Pairs sorted by j
    decode each weight row once."""
    raw = _raw_check(type_, raw, od, id_)
    q, dh, s, T = _act_check(q, dh, s, id_)
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    js = np.ascontiguousarray(js, dtype=np.int64)
    n = ts.size
    out = np.empty(n, np.float64)
    A = np.empty(n, np.float64)
    rc = _load().oracle_mmq_at(type_, _ptr(raw), od, id_, _ptr(q), _ptr(dh), _ptr(s), T, n,
                               _ptr(ts), _ptr(js), _ptr(out), _ptr(A))
    if rc:
        raise ValueError("oracle_mmq_at failed")
    return out, A

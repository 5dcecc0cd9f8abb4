"""Drives the validation paths of a libqmm build through ctypes, with no GPU:
every call below must be refused (or, for n_tok = 0, succeed) before any HIP
call.  Run by tests/test_sanitizers.py against a build whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer; exits non-zero on a wrong
return code (a sanitizer report aborts the process by itself).

    python abi_driver.py <path to libqmm build>
"""
import ctypes
import math
import random
import sys

EINVAL, ESHAPE, ENOMEM = -1, -2, -3
Q4_K, Q6_K, Q4_K_PACKED = 4, 6, 14


def main(path):
    L = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.qmm_register_weights.argtypes = [ctypes.c_int, I64, I64, P, SZ, P, ctypes.POINTER(P)]
    L.qmm_weights_info.argtypes = [P, P]
    L.qmm_weights_export.argtypes = [P, P, SZ]
    L.qmm_release_weights.argtypes = [P]
    L.qmm_release_weights.restype = None
    L.qmm_set_memory_cap.argtypes = [SZ]
    L.qmm_set_memory_cap.restype = None
    L.qmm_qact_bytes.argtypes = [I64, I64]
    L.qmm_qact_bytes.restype = SZ
    L.qmm_quantize_activations.argtypes = [P, I64, I64, P, SZ, P]
    L.qmm_mmq.argtypes = [P, P, SZ, I64, P, P]
    L.qmm_mmq_noalloc.argtypes = [P, P, SZ, I64, P, P]
    L.qmm_stream_release.argtypes = [P, P]
    L.qmm_last_error.restype = ctypes.c_char_p
    bad = []

    def expect(what, got, want):
        if got != want:
            bad.append(f"{what}: got {got}, want {want} ({L.qmm_last_error().decode()})")

    buf = ctypes.create_string_buffer(1 << 16)
    good = ctypes.cast(buf, P)
    h = P()
    # registration: every argument check, with the long error messages formatted
    expect("null out", L.qmm_register_weights(Q6_K, 4, 256, good, 840, None, None), EINVAL)
    expect("bad type", L.qmm_register_weights(5, 4, 256, good, 840, None, ctypes.byref(h)), EINVAL)
    expect("od 0", L.qmm_register_weights(Q6_K, 0, 256, good, 0, None, ctypes.byref(h)), EINVAL)
    expect("od huge", L.qmm_register_weights(Q6_K, 1 << 40, 256, good, 840, None, ctypes.byref(h)), EINVAL)
    expect("id 300", L.qmm_register_weights(Q6_K, 4, 300, good, 840, None, ctypes.byref(h)), EINVAL)
    expect("id huge", L.qmm_register_weights(Q4_K, 4, 1 << 40, good, 840, None, ctypes.byref(h)), EINVAL)
    expect("null bytes", L.qmm_register_weights(Q6_K, 4, 256, None, 840, None, ctypes.byref(h)), EINVAL)
    expect("nbytes", L.qmm_register_weights(Q6_K, 4, 256, good, 841, None, ctypes.byref(h)), EINVAL)
    expect("nbytes q4", L.qmm_register_weights(Q4_K, 3, 512, good, 3 * 2 * 210, None, ctypes.byref(h)), EINVAL)
    # the memory cap refuses before allocating
    L.qmm_set_memory_cap(1000)
    expect("cap", L.qmm_register_weights(Q6_K, 4, 256, good, 840, None, ctypes.byref(h)), ENOMEM)
    L.qmm_set_memory_cap(0)
    # sizes
    for n_tok, id_, want in ((1, 256, 128 * 256 * 9 // 8), (129, 512, 256 * 512 * 9 // 8), (0, 256, 0),
                             (-1, 256, 0), (4, 255, 0), (1 << 40, 256, 0)):
        expect(f"qact_bytes({n_tok}, {id_})", L.qmm_qact_bytes(n_tok, id_), want)
    # the prepass
    expect("quantize null", L.qmm_quantize_activations(None, 4, 256, good, 4608, None), EINVAL)
    expect("quantize misaligned", L.qmm_quantize_activations(ctypes.c_void_p(buf_addr(buf) + 4), 4, 256, good,
                                                             128 * 256 * 9 // 8, None), EINVAL)
    expect("quantize bytes", L.qmm_quantize_activations(good, 4, 256, good, 100, None), EINVAL)
    expect("quantize tokens", L.qmm_quantize_activations(good, -1, 256, good, 0, None), EINVAL)
    expect("quantize empty", L.qmm_quantize_activations(None, 0, 256, None, 0, None), 0)
    expect("quantize empty bytes", L.qmm_quantize_activations(None, 0, 256, None, 16, None), EINVAL)
    # both MMQ entry points
    for name in ("qmm_mmq", "qmm_mmq_noalloc"):
        f = getattr(L, name)
        expect(f"{name} null handle", f(None, good, 100, 4, good, None), EINVAL)
        expect(f"{name} null handle, empty", f(None, None, 0, 0, None, None), EINVAL)
    # the handle queries
    expect("info null", L.qmm_weights_info(None, good), EINVAL)
    expect("export null", L.qmm_weights_export(None, good, 10), EINVAL)
    L.qmm_release_weights(None)
    # a stream that holds no scratch: nothing to free, no HIP call
    expect("stream release, nothing held", L.qmm_stream_release(good, good), 0)
    expect("stream release, freed count", ctypes.cast(good, ctypes.POINTER(SZ))[0], 0)
    expect("stream release, null stream", L.qmm_stream_release(None, None), 0)
    # the launch planner, host arithmetic only: seeded shapes over the accepted
    # range on several GPU sizes, every work-group of the small launches mapped
    # (undefined behaviour -- a division by zero, an overflow -- aborts)
    L.qmm_mmq_plan.argtypes = [ctypes.c_int, I64, I64, I64, ctypes.c_int, ctypes.POINTER(Plan)]
    I32P = ctypes.POINTER(ctypes.c_int32)
    L.qmm_mmq_plan_work.argtypes = [ctypes.POINTER(Plan), I64, I32P, I32P, I32P, I32P]
    rng = random.Random(7)
    plan = Plan()
    out = [ctypes.c_int32() for _ in range(4)]
    mapped = 0
    for i in range(3000):
        type_ = (Q4_K, Q6_K, Q4_K_PACKED)[i % 3]
        od = int(math.exp(rng.uniform(0, math.log(1 << 21))))
        id_ = 256 * int(math.exp(rng.uniform(0, math.log(4096))))
        n_tok = int(math.exp(rng.uniform(0, math.log(20000))))
        cus = rng.choice((1, 3, 80, 256, 304))
        rc = L.qmm_mmq_plan(type_, od, id_, n_tok, cus, ctypes.byref(plan))
        expect(f"plan {type_} {od}x{id_} T={n_tok} cus={cus}", rc, 0)
        if rc == 0 and plan.work_groups <= 4000:
            for wg in range(plan.work_groups):
                expect("plan work", L.qmm_mmq_plan_work(ctypes.byref(plan), wg, *[ctypes.byref(o) for o in out]), 0)
            mapped += 1
    expect("plans mapped", mapped > 100, True)
    expect("plan bad cus", L.qmm_mmq_plan(Q4_K, 4096, 4096, 512, 0, ctypes.byref(plan)), EINVAL)
    expect("plan too big", L.qmm_mmq_plan(Q4_K, 1 << 21, 256, 1 << 20, 256, ctypes.byref(plan)), EINVAL)
    expect("plan null", L.qmm_mmq_plan(Q4_K, 4096, 4096, 512, 256, None), EINVAL)
    expect("plan work null", L.qmm_mmq_plan_work(None, 0, *[ctypes.byref(o) for o in out]), EINVAL)
    if bad:
        print("\n".join(bad))
        return 1
    print("abi driver: all validation paths returned the documented codes")
    return 0


class Plan(ctypes.Structure):  # qmm_plan
    _fields_ = [("work_groups", ctypes.c_int64), ("scratch_bytes", ctypes.c_size_t)] + [
        (n, ctypes.c_int32) for n in ("threads", "many", "tile_rows", "tile_tokens", "k_groups", "per_cu",
                                      "row_tiles", "tok_tiles", "dp_row_tiles", "n_tail", "split", "nsb")]


def buf_addr(buf):
    return ctypes.addressof(buf)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))

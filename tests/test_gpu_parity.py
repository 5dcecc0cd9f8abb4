"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* prepass bytes (q codes, dh, s) bit-exact, padded tokens zero;
* registration planes byte-exact against the oracle's decode;
* integer dots bit-exact through the production kernel (unit super-scales and
  integer activations make every output an exact integer below 2^24);
* f32 results within 1e-4 * sum|terms| of the oracle on every element: at small
  sizes spanning several tiles and a ragged tail, and at the full workload
  sizes in the same launch configuration the benchmark times, and on row
  subsets of seeded random shapes at any size;
* odd row counts / token tails are bit-identical prefixes, repeat runs are
  bit-identical, nothing outside the output is written.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import quant_q8_gemm_amd as qmm  # noqa: E402
import synth  # noqa: E402
from tests import layouts  # noqa: E402
from tests.kq_blocks import q4k_block, q6k_block  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def gpu_quantize(x: np.ndarray):
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    qact = qmm.quantize_activations(xt)
    return qact


def check_prepass(x: np.ndarray, qact):
    n_tok, id_ = x.shape
    q, dh, s = layouts.read_qact(qact.cpu().numpy(), n_tok, id_)
    oq, odh, os_ = oracle.quantize(x)
    assert np.array_equal(q[:n_tok], oq), "q codes differ"
    assert np.array_equal(dh[:n_tok], odh), "dh differs"
    assert np.array_equal(s[:n_tok], os_), "s differs"
    assert not q[n_tok:].any() and not dh[n_tok:].any() and not s[n_tok:].any(), "padding not zero"
    return oq, odh, os_


def run_mmq(w, qact, n_tok, poison=True):
    out = torch.empty((n_tok, w.od), dtype=torch.float32, device="cuda")
    if poison:
        out.fill_(float("nan"))
    qmm.mmq(w, qact, n_tok, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_close(got, ref, A, where=""):
    err = np.abs(got.astype(np.float64) - ref)
    bad = ~(err <= TOL * A)
    assert not np.isnan(got).any(), f"NaN in output {where}"
    assert not bad.any(), (f"{bad.sum()} elements beyond tolerance {where}; worst "
                           f"err={err[bad].max():.3e} A={A[bad][np.argmax(err[bad])]:.3e}")


# --------------------------------------------------------------------------
# prepass
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n_tok,id_,outliers", [(64, 512, False), (13, 768, True), (1, 256, False),
                                                (509, 11008, False), (130, 4096, True)])
def test_prepass_bytes_exact(n_tok, id_, outliers):
    say(f"prepass n_tok={n_tok} id={id_}")
    x = synth.activations(np.random.default_rng(n_tok), n_tok, id_, outliers)
    check_prepass(x, gpu_quantize(x))


def test_prepass_special_values():
    say("prepass special values")
    x = np.zeros((6, 256), np.float32)
    step = np.float32(0.0625)
    x[0, 0] = 127 * step                                   # exact scale, then half-way ties
    x[0, 1:9] = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 126.5], np.float32) * step
    x[1, :32] = 1e-6                                       # scale rounds to zero
    x[1, 32] = 2e-5                                        # subnormal f16 scale
    x[1, 33] = -1e-5
    x[2, :] = 2046.0 * np.sign(np.random.default_rng(1).standard_normal(256)).astype(np.float32)
    x[3, :] = -0.0
    x[4, ::2] = 1.0
    x[5, :] = np.random.default_rng(2).uniform(-2046, 2046, 256).astype(np.float32)
    check_prepass(x, gpu_quantize(x))


def test_prepass_near_ties():
    """Quotients x/dh a few f32 ulps either side of half-integers (and exactly on
    them): the rounding decision must match the correctly rounded division."""
    say("prepass near ties")
    rng = np.random.default_rng(11)
    T, id_ = 64, 1024
    x = np.zeros((T, id_), np.float32)
    xb = x.reshape(T, -1, 32)
    steps = (np.abs(rng.standard_normal(xb.shape[:2])) * 0.05 + 1e-3).astype(np.float16).astype(np.float32)
    # element 0 of each block fixes amax = 127 * step, so dh = f16(step * 127 / 127) = step
    xb[:, :, 0] = 127 * steps
    k = rng.integers(-126, 126, size=xb[:, :, 1:].shape).astype(np.float32)
    ulps = rng.integers(-3, 4, size=k.shape)
    target = ((k + 0.5) * steps[:, :, None]).astype(np.float32)
    xb[:, :, 1:] = np.nextafter(target, np.where(ulps > 0, np.inf, -np.inf).astype(np.float32))
    xb[:, :, 1:] = np.where(ulps == 0, target, xb[:, :, 1:])
    check_prepass(x, gpu_quantize(x))


# --------------------------------------------------------------------------
# registration planes
# --------------------------------------------------------------------------

def _full_range_q6k(rng, od, id_):
    raw = synth.q6k_weights(rng, od, id_).reshape(-1, 210).copy()
    raw[:, 192:208] = rng.integers(-128, 128, size=(raw.shape[0], 16), dtype=np.int8).view(np.uint8)
    return raw.reshape(-1)


def expected_planes(type_, raw, od, id_):
    """The planes include/qmm.h documents, from the oracle's decode: q6_K the
    scale-folded weights and d; q4_K the codes, d*2^25 and -dmin (exact in
    binary32: an f16 value times a power of two), and the 6-bit scales and mins
    as binary16 integers (exact)."""
    if type_ == synth.Q6_K:
        w6, sc, d = oracle.decode_q6k(raw, od, id_)
        w = w6.astype(np.int32) * np.repeat(sc.astype(np.int32), 16, axis=1)
        return {"w": w, "d": d}
    w4, sc, mn, d, dm = oracle.decode_q4k(raw, od, id_)
    d25 = np.ldexp(d.astype(np.float64), 25)
    assert np.all(d25.astype(np.float32) == d25)
    return {"codes": w4.astype(np.int32), "d25": d25.astype(np.float32) + np.float32(0.0),
            "ndmin": (-dm.astype(np.float32)) + np.float32(0.0),
            "sc": sc.astype(np.float16).view(np.uint16), "mn": mn.astype(np.float16).view(np.uint16)}


def check_planes(w, type_, raw, od, id_):
    got = layouts.read_planes(w.export(), type_, w.od_pad, id_, w.wd_offset, w.sm_offset)
    exp = expected_planes(type_, raw, od, id_)
    assert set(got) == set(exp)
    for k, e in exp.items():
        g = got[k]
        if e.dtype == np.float32:  # compare bit patterns: -0 and +0 differ
            assert np.array_equal(g[:od].view(np.uint32), e.view(np.uint32)), f"plane {k} differs"
        else:
            assert np.array_equal(g[:od], e), f"plane {k} differs"
        assert not g[od:].view(np.uint8).any(), f"plane {k}: padding rows not zero"


@pytest.mark.parametrize("type_,od,id_,full", [(synth.Q6_K, 5, 512, False), (synth.Q6_K, 130, 768, True),
                                               (synth.Q4_K, 37, 512, False), (synth.Q4_K, 129, 1024, False),
                                               (synth.Q4_K_PACKED, 37, 512, False),
                                               (synth.Q4_K_PACKED, 129, 1024, False),
                                               # above the repack grid's 4M items: threads stride
                                               (synth.Q6_K, 16400, 8192, False), (synth.Q4_K, 16400, 8192, False),
                                               (synth.Q4_K_PACKED, 8193, 8192, False)])
def test_planes_byte_exact(type_, od, id_, full):
    say(f"planes type={type_} od={od} id={id_}")
    rng = np.random.default_rng(od)
    raw = _full_range_q6k(rng, od, id_) if full else synth.weights(rng, type_, od, id_)
    w = qmm.register_weights(type_, od, id_, raw)
    assert w.od_pad % 128 == 0 and w.od_pad >= od
    check_planes(w, type_, raw, od, id_)
    w.release()


def _set_f16(raw, lo, bits):
    """Overwrite the f16 field at byte offset lo of every block with bits."""
    nb = raw.shape[0]
    raw[:, lo:lo + 2] = np.asarray(bits, np.uint16).astype("<u2").view(np.uint8).reshape(nb, 2)


@pytest.mark.parametrize("type_", [synth.Q4_K, synth.Q6_K, synth.Q4_K_PACKED], ids=["q4_K", "q6_K", "q4_K packed"])
def test_extreme_block_scales(type_):
    """Super-block scales of either sign, huge (60000), subnormal (2^-24) and
    zero of either sign (a super-block that contributes nothing): the planes
    stay byte-exact and the MMQ stays within the tolerance.  Blocks are drawn
    as usual, then their f16 d (and q4_K dmin) bits are rewritten."""
    od, id_, T = 90, 1024, 70
    say(f"extreme block scales {synth.TYPE_NAMES[type_]}")
    rng = np.random.default_rng(9)
    bb = synth.BLOCK_BYTES[type_]
    raw = synth.weights(rng, type_, od, id_).reshape(-1, bb).copy()
    nb = raw.shape[0]
    fields = [0, 2] if type_ != synth.Q6_K else [208]
    for lo in fields:
        bits = raw[:, lo:lo + 2].copy().view("<u2").reshape(-1)
        pick = rng.random(nb)
        bits = np.where(pick < 0.3, bits | 0x8000, bits)                 # negative
        bits = np.where((pick >= 0.3) & (pick < 0.35), 0x7B53, bits)     # 60000
        bits = np.where((pick >= 0.35) & (pick < 0.40), 0x0001, bits)    # 2^-24
        bits = np.where((pick >= 0.40) & (pick < 0.44), 0x0000, bits)    # +0
        bits = np.where((pick >= 0.44) & (pick < 0.47), 0x8000, bits)    # -0
        _set_f16(raw, lo, bits)
    raw = raw.reshape(-1)
    w = qmm.register_weights(type_, od, id_, raw)
    check_planes(w, type_, raw, od, id_)
    x = synth.activations(rng, T, id_, False)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    out = run_mmq(w, qact, T)
    ref, A = oracle.mmq(synth.block_format(type_), raw, od, id_, q, dh, s)
    check_close(out, ref, A, "extreme block scales")
    w.release()


# Shapes for the wide-scale-range rows: both tile geometries, a ragged second
# wave whose tail tiles are split along K, and an under-filled launch where
# every tile is split.
WIDE = [("few-tile 96x2048 T=70", 96, 2048, 70), ("many-tile 1030x1024 T=4000", 1030, 1024, 4000),
        ("ragged tail 4160x1024 T=512", 4160, 1024, 512), ("all split 512x3072 T=300", 512, 3072, 300)]


@pytest.mark.parametrize("type_", [synth.Q4_K, synth.Q4_K_PACKED], ids=["q4_K", "q4_K packed"])
@pytest.mark.parametrize("case", WIDE, ids=[c[0] for c in WIDE])
def test_q4k_wide_scale_range_rows(case, type_):
    """q4_K rows whose super-block scales span the whole f16 range: super-block
    0 of every row has d = 60000 (and dmin = 60000 on a third of the rows), the
    others d = k * 2^-24 for k in [1, 1023] (subnormal) and dmin either tiny
    (k * 2^-24), zero or 60000.  Half of the tokens are zero over super-block 0,
    so their outputs are made of the tiny terms alone; a quarter are non-zero in
    one small super-block only.  Every element must land within 1e-4 of the sum
    of its terms' magnitudes -- which a scale stored relative to the row's
    largest value cannot do."""
    name, od, id_, T = case
    say(f"{synth.TYPE_NAMES[type_]} wide scale range {name}")
    rng = np.random.default_rng(31)
    nsb = id_ // 256
    raw = synth.q4k_weights(rng, od, id_).reshape(od, nsb, 144).copy()
    d = rng.integers(1, 1024, size=(od, nsb)).astype(np.uint16)           # k * 2^-24
    kind = rng.integers(0, 3, size=(od, nsb))
    dmin = np.where(kind == 0, rng.integers(1, 1024, size=(od, nsb)), np.where(kind == 1, 0, 0x7B53))
    d[:, 0] = 0x7B53
    dmin[:, 0] = np.where(np.arange(od) % 3 == 0, 0x7B53, dmin[:, 0])
    raw[:, :, 0:2] = d.astype("<u2").view(np.uint8).reshape(od, nsb, 2)
    raw[:, :, 2:4] = dmin.astype(np.uint16).astype("<u2").view(np.uint8).reshape(od, nsb, 2)
    raw = raw.reshape(-1)
    x = synth.activations(rng, T, id_)
    x[0::2, :256] = 0.0                                   # zero over the d = 60000 block
    one = 1 + (np.arange(T) % max(1, nsb - 1))            # one small super-block only
    for t in range(1, T, 4):
        keep = x[t, 256 * one[t]: 256 * one[t] + 256].copy()
        x[t] = 0.0
        x[t, 256 * one[t]: 256 * one[t] + 256] = keep
    w = qmm.register_weights(type_, od, id_, raw)
    check_planes(w, type_, raw, od, id_)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    got = run_mmq(w, qact, T)
    ref, A = oracle.mmq(synth.Q4_K, raw, od, id_, q, dh, s)
    check_close(got, ref, A, f"wide scale range {name}")
    w.release()


# --------------------------------------------------------------------------
# integer dots through the production kernel
# --------------------------------------------------------------------------

def _int_acts(rng, T, id_):
    x = rng.integers(-127, 128, size=(T, id_)).astype(np.float32)
    x.reshape(T, -1, 32)[:, :, 0] = np.where(rng.random((T, id_ // 32)) < 0.5, 127, -127)
    return x


@pytest.mark.parametrize("type_", [synth.Q6_K, synth.Q4_K, synth.Q4_K_PACKED])
def test_int_dots_exact_unit_scale(type_):
    od, id_, T = 200, 512, 77
    say(f"int dots unit type={type_} od={od} T={T}")
    rng = np.random.default_rng(5)
    nb = od * id_ // 256
    if type_ == synth.Q6_K:
        blocks = [q6k_block(ql=rng.integers(0, 256, 128, dtype=np.uint8),
                            qh=rng.integers(0, 256, 64, dtype=np.uint8),
                            sc=rng.integers(-2, 3, 16).astype(np.int8)) for _ in range(nb)]
    else:
        blocks = []
        for _ in range(nb):
            sc = np.zeros(12, np.uint8)
            sc[0:4] = rng.integers(0, 4, 4)          # scales 0..3 of sub-blocks 0..3, mins 0
            sc[8:12] = rng.integers(0, 4, 4)         # scales of sub-blocks 4..7
            blocks.append(q4k_block(dmin_bits=0x3C00, scales=sc,
                                    qs=rng.integers(0, 256, 128, dtype=np.uint8)))
    raw = np.concatenate(blocks)
    x = _int_acts(rng, T, id_)
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    assert np.all(dh == 0x3C00)
    got = run_mmq(w, qact, T)
    ref, _ = oracle.mmq(synth.block_format(type_), raw, od, id_, q, dh, s)
    assert np.all(np.abs(ref) < 2 ** 24)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("type_", [synth.Q6_K, synth.Q4_K, synth.Q4_K_PACKED])
def test_int_dots_exact_full_range_one_chunk(type_):
    """Full-range scales; each token is non-zero in one 32-block only, so every
    output equals one scale-folded block dot J exactly."""
    od, id_, T = 160, 768, 96
    say(f"int dots full range type={type_}")
    rng = np.random.default_rng(6)
    nb = od * id_ // 256
    if type_ == synth.Q6_K:
        raw = _full_range_q6k(rng, od, id_).reshape(nb, 210)
        raw[:, 208:210] = np.array([0x00, 0x3C], np.uint8)  # d = 1
    else:
        raw = synth.q4k_weights(rng, od, id_).reshape(nb, 144)
        raw[:, 0:4] = np.array([0x00, 0x3C, 0x00, 0x00], np.uint8)  # d = 1, dmin = 0
    raw = raw.reshape(-1)
    nchunk = id_ // 32
    x = np.zeros((T, id_), np.float32)
    chunk = np.arange(T) % nchunk
    for t in range(T):
        blk = rng.integers(-127, 128, 32).astype(np.float32)
        blk[rng.integers(0, 32)] = 127 if t % 2 else -127
        x[t, 32 * chunk[t]: 32 * chunk[t] + 32] = blk
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    got = run_mmq(w, qact, T)
    if type_ == synth.Q6_K:
        _, J = oracle.dots_q6k(raw, od, id_, q)
        ref = J[np.arange(T), :, chunk].astype(np.float64)
    else:
        D32 = oracle.dots_q4k(raw, od, id_, q)
        _, sc, _, _, _ = oracle.decode_q4k(raw, od, id_)
        ref = (D32[np.arange(T), :, chunk].astype(np.int64) * sc[:, chunk].T.astype(np.int64)).astype(np.float64)
    assert np.array_equal(got.astype(np.float64), ref)


# --------------------------------------------------------------------------
# f32 results
# --------------------------------------------------------------------------

SMALL = [("q6_K 256x512 T=64", synth.Q6_K, 256, 512, 64, False),
         ("q4_K 300x768 T=77", synth.Q4_K, 300, 768, 77, True),
         ("q6_K 129x1280 T=200", synth.Q6_K, 129, 1280, 200, True),
         ("q4_K 1x256 T=1", synth.Q4_K, 1, 256, 1, False),
         # one super-block: the first k-group of the few-tile geometry has none
         ("q6_K 70x256 T=33", synth.Q6_K, 70, 256, 33, True),
         ("q6_K 33x2304 T=130", synth.Q6_K, 33, 2304, 130, False),
         ("q4_K 520x1536 T=257", synth.Q4_K, 520, 1536, 257, False),
         # a ragged last wave on 256 CUs (260 tiles of 64 x 128 each): the
         # tail tiles are split along K (4 super-blocks: 2 slices) and added by
         # the fixup kernel; with 3 super-blocks (4200x768, 264 tiles) the two
         # k-groups leave no room to split, and the tail runs whole
         ("q4_K 4160x1024 T=512", synth.Q4_K, 4160, 1024, 512, False),
         ("q6_K 4200x768 T=500", synth.Q6_K, 4200, 768, 500, True),
         # far fewer tiles than CUs (24): every tile split along K
         ("q6_K 512x2816 T=300", synth.Q6_K, 512, 2816, 300, False),
         # the same for q4_K (its d and dmin applied per super-block before the
         # partials leave a slice)
         ("q4_K 512x3072 T=300", synth.Q4_K, 512, 3072, 300, True),
         # enough 64 x 64 tiles (>= 1024) to select the many-tile geometry;
         # q6_K there runs 64 x 128 tiles two per CU: 528 tiles on 512 slots
         # (a split tail), and 1056 tiles (two full waves and a last of 32,
         # whole: one super-block leaves nothing to split)
         ("q6_K 1000x512 T=4100", synth.Q6_K, 1000, 512, 4100, True),
         ("q6_K 2100x256 T=4000", synth.Q6_K, 2100, 256, 4000, False),
         # three full waves of 512 tiles and a last wave of 89 (at most a quarter
         # of the slots, two work-groups per CU): the 100 tiles after the 61st
         # row tile split 4 ways along K, the last row tile and token tile ragged
         ("q6_K 4097x1024 T=3199", synth.Q6_K, 4097, 1024, 3199, True),
         # exactly three full waves (1536 tiles on 512 slots): no tail at all
         ("q6_K 4096x1024 T=3072", synth.Q6_K, 4096, 1024, 3072, False),
         # the same in the few-tile geometry (64 x 128 tiles, one work-group per
         # CU): 520 tiles on 256 slots, the 13 tiles after the 39th row tile
         # split 8 ways, the last row tile ragged
         ("q4_K 2527x4352 T=1572", synth.Q4_K, 2527, 4352, 1572, False),
         # one token against 70000 rows: the many-tile geometry with a single
         # token tile (1094 row tiles)
         ("q4_K 70000x256 T=1", synth.Q4_K, 70000, 256, 1, False),
         ("q6_K 70001x256 T=1", synth.Q6_K, 70001, 256, 1, True),
         ("q4_K 1030x256 T=4000", synth.Q4_K, 1030, 256, 4000, False),
         # the packed-code registration: few tiles, a ragged split tail, many tiles
         ("q4_K packed 300x768 T=77", synth.Q4_K_PACKED, 300, 768, 77, True),
         ("q4_K packed 4160x1024 T=512", synth.Q4_K_PACKED, 4160, 1024, 512, False),
         ("q4_K packed 1030x256 T=4000", synth.Q4_K_PACKED, 1030, 256, 4000, False)]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_all_elements(case):
    name, type_, od, id_, T, outl = case
    say(f"small {name}")
    raw, x = synth.case(type_, od, id_, T, seed=0, outliers=outl)
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    got = run_mmq(w, qact, T)
    ref, A = oracle.mmq(synth.block_format(type_), raw, od, id_, q, dh, s)
    check_close(got, ref, A, name)


@pytest.mark.parametrize("geometry", ["few", "many"])
@pytest.mark.parametrize("type_", [synth.Q4_K, synth.Q6_K, synth.Q4_K_PACKED], ids=["q4_K", "q6_K", "q4_K packed"])
def test_subnormal_activation_scales(type_, geometry):
    """Activation scales that are f16 subnormals (amax below 127 * 2^-14) reach
    the matrix core (q4_K's scale outer product and min term take dh and s as
    f16 operands) and the vector ALU (q6_K converts dh): every token's first
    chunks are tiny, some chunks are zero and the rest normal, and the first
    tokens are tiny throughout, so a flushed subnormal anywhere fails the
    relative tolerance.  Both tile geometries."""
    od, id_ = 200, 512
    T = 40 if geometry == "few" else 4100
    say(f"subnormal scales {synth.TYPE_NAMES[type_]} T={T}")
    raw, x = synth.case(type_, od, id_, T, seed=5)
    x = x.copy()
    x[:, :96] *= 1e-5                    # amax ~ 3e-5: dh ~ 2e-7, deep in the subnormals
    x[:, 96:128] *= 3e-3                 # dh near the smallest normal
    x[:, 128:160] = 0.0                  # zero blocks
    x[:8] *= 1e-4                        # tokens that are tiny everywhere
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    d16 = dh.view(np.float16).astype(np.float64)
    assert np.any((d16 > 0) & (d16 < 2.0 ** -14)), "no subnormal scale in the input"
    w = qmm.register_weights(type_, od, id_, raw)
    got = run_mmq(w, qact, T)
    ref, A = oracle.mmq(synth.block_format(type_), raw, od, id_, q, dh, s)
    check_close(got, ref, A, f"subnormal scales {geometry}")
    w.release()


def _random_shapes(n, seed=11):
    """Seeded random shapes: both types, odd row counts, 1..8 super-blocks; every
    other case with 2000..4200 tokens so that it takes the many-tile geometry.
    Small enough for the oracle on every element."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        type_ = synth.Q6_K if (i // 2) % 2 else synth.Q4_K
        if i % 2:
            id_ = 256 * int(rng.integers(1, 3))
            od = int(rng.integers(900, 1500))
            T = int(rng.integers(2000, 4201))
        else:
            id_ = 256 * int(rng.integers(1, 9))
            od = int(rng.integers(1, 3000))
            T = int(rng.integers(1, 701))
        out.append((f"random {synth.TYPE_NAMES[type_]} {od}x{id_} T={T}", type_, od, id_, T, bool(i % 3 == 0)))
    return out


RANDOM = _random_shapes(8)


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_shapes_all_elements(case):
    test_small_all_elements(case)


def _sweep_shapes(n, seed=29):
    """Seeded random shapes over the whole size range (up to 12000 rows, 12288
    inner, 4200 tokens, log-uniform), all three registration types: every
    geometry and tail plan turns up (many and few tiles, split ragged waves,
    split short last waves, whole tiles)."""
    rng = np.random.default_rng(seed)
    types = [synth.Q4_K, synth.Q6_K, synth.Q4_K_PACKED]
    out = []
    for i in range(n):
        type_ = types[i % 3]
        big = i % 2 == 1
        od = int(np.exp(rng.uniform(np.log(2000) if big else 0.0, np.log(12000))))
        id_ = 256 * int(rng.integers(1, 49))
        T = int(np.exp(rng.uniform(np.log(1000) if big else 0.0, np.log(4200))))
        while od * T * id_ > 6e10 and T > 1:
            T //= 2
        out.append((f"sweep {synth.TYPE_NAMES[type_]} {od}x{id_} T={T}", type_, od, id_, T, bool(rng.integers(0, 2))))
    return out


SWEEP = _sweep_shapes(24)


@pytest.mark.parametrize("case", SWEEP, ids=[c[0] for c in SWEEP])
def test_sweep_row_subsets(case):
    """Random shapes at any size: every token of the first and last 64 rows and
    of two random 32-row blocks against the oracle; every output written; the
    allocation-free entry point and a repeat call bit-identical to the first."""
    name, type_, od, id_, T, outl = case
    say(f"{name}: generating")
    raw, x = synth.case(type_, od, id_, T, seed=od * 7 + T, outliers=outl)
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    say(f"{name}: mmq")
    got = run_mmq(w, qact, T)
    again = run_mmq(w, qact, T)
    na = torch.full((T, od), float("nan"), dtype=torch.float32, device="cuda")
    qmm.mmq_noalloc(w, qact, T, na)
    torch.cuda.synchronize()
    w.release()
    assert np.array_equal(again.view(np.uint32), got.view(np.uint32)), "repeat call differs"
    assert np.array_equal(na.cpu().numpy().view(np.uint32), got.view(np.uint32)), "noalloc differs"
    rng = np.random.default_rng(od + T)
    blocks = {(0, min(64, od)), (max(0, od - 64), od)}
    for _ in range(2):
        j0 = int(rng.integers(0, od)) // 32 * 32
        blocks.add((j0, min(od, j0 + 32)))
    say(f"{name}: oracle on {len(blocks)} row blocks")
    for j0, j1 in sorted(blocks):
        ref, A = oracle.mmq_rows(synth.block_format(type_), raw, od, id_, q, dh, s, j0, j1)
        check_close(got[:, j0:j1], ref, A, f"{name} rows {j0}:{j1}")


def _stratified_pairs(rng, T, od):
    """One random (token, row) inside every 32 x 32 block of the output (each
    wave's output block), plus the four corners; sorted by row so the oracle
    decodes each weight row once."""
    tb, rb = np.meshgrid(np.arange(0, T, 32), np.arange(0, od, 32), indexing="ij")
    ts = np.minimum(tb + rng.integers(0, 32, tb.shape), T - 1).ravel()
    js = np.minimum(rb + rng.integers(0, 32, rb.shape), od - 1).ravel()
    ts = np.concatenate([ts, [0, 0, T - 1, T - 1]])
    js = np.concatenate([js, [0, od - 1, 0, od - 1]])
    order = np.argsort(js, kind="stable")
    return ts[order], js[order]


# the one-layer workload at 3314 tokens: its four distinct GEMM shapes
LAYER = [(f"layer {synth.TYPE_NAMES[t]} {od}x{id_} T={synth.LAYER_TOKENS}", t, od, id_, synth.LAYER_TOKENS, False)
         for t, od, id_ in sorted({(t, od, id_) for _, t, od, id_ in synth.LAYER_GEMMS})]
# one GPU's share of ffn_down under 8-way tensor parallelism (column and row slices)
SHARDS = [("q6_K ffn_down column shard 512x11008 T=512", synth.Q6_K, 512, 11008, 512, False),
          ("q6_K ffn_down row shard 4096x1536 T=512", synth.Q6_K, 4096, 1536, 512, False),
          ("q4_K ffn_gate column shard 1376x4096 T=512", synth.Q4_K, 1376, 4096, 512, False)]
# the q4_K shapes registered with packed codes
PACKED = [(c[0].replace("q4_K", "q4_K packed"), synth.Q4_K_PACKED) + tuple(c[2:])
          for c in [synth.ATTN, synth.GATE_UP] + LAYER if c[1] == synth.Q4_K]
# LLaMA-13B widths (hidden 5120, FFN 13824): other super-block counts (20 and 54 per
# row), other tile counts and odd token counts, in both types and both registrations
WIDER = [("13B attn q4_K 5120x5120 T=777", synth.Q4_K, 5120, 5120, 777, False),
         ("13B gate q4_K 13824x5120 T=1001", synth.Q4_K, 13824, 5120, 1001, True),
         ("13B down q6_K 5120x13824 T=301", synth.Q6_K, 5120, 13824, 301, False),
         ("13B v q6_K 5120x5120 T=2049", synth.Q6_K, 5120, 5120, 2049, True),
         ("13B attn q4_K packed 5120x5120 T=777", synth.Q4_K_PACKED, 5120, 5120, 777, False)]
FULL = [synth.FFN_DOWN, synth.FFN_DOWN_ODD, synth.ATTN, synth.GATE_UP, synth.HEAD] + LAYER + SHARDS + PACKED + WIDER


@pytest.mark.parametrize("cfg", FULL, ids=[c[0] for c in FULL])
def test_full_size_all_elements(cfg):
    """Every element of every full workload size, in the launch configuration
    the benchmark times, against the oracle (its rows split over the host's
    CPUs): ffn_down (also 4097 rows at 509 tokens), both attention/FFN q4_K
    shapes, the 2048-token output head, the four GEMM shapes of the 3314-token
    layer, the tensor-parallel shards, the packed-code q4_K shapes and five
    13B-width shapes."""
    name, type_, od, id_, T, outl = cfg
    say(f"full size {name}: generating")
    raw, x = synth.case(type_, od, id_, T, seed=0, outliers=outl)
    say(f"full size {name}: register + prepass")
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    say(f"full size {name}: mmq")
    got = run_mmq(w, qact, T)
    w.release()
    say(f"full size {name}: oracle on {T * od} elements")
    ref, A = oracle.mmq_parallel(synth.block_format(type_), raw, od, id_, q, dh, s)
    check_close(got, ref, A, name)


# The API's maximum sizes, each on every element: QMM_MAX_OD rows (32,768 row
# tiles), QMM_MAX_ID inner (4,096 super-blocks; one tile, split 256 ways along
# K, also through the allocation-free entry point), QMM_MAX_TOKENS tokens
# (16,384 token tiles).
MAXIMA = [("q6_K od=2^21 id=256 T=3", synth.Q6_K, 1 << 21, 256, 3),
          ("q4_K packed od=2^21 id=256 T=1", synth.Q4_K_PACKED, 1 << 21, 256, 1),
          ("q4_K od=33 id=2^20 T=5", synth.Q4_K, 33, 1 << 20, 5),
          ("q6_K od=33 id=2^20 T=5", synth.Q6_K, 33, 1 << 20, 5),
          ("q4_K od=1 id=256 T=2^20", synth.Q4_K, 1, 256, 1 << 20)]


@pytest.mark.parametrize("case", MAXIMA, ids=[c[0] for c in MAXIMA])
def test_maximum_sizes_all_elements(case):
    name, type_, od, id_, T = case
    assert max(od, 1) <= 1 << 21 and id_ <= 1 << 20 and T <= 1 << 20
    say(f"maximum size {name}: generating")
    raw, x = synth.case(type_, od, id_, T, seed=3)
    say(f"maximum size {name}: register + prepass")
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    say(f"maximum size {name}: mmq")
    got = run_mmq(w, qact, T)
    if id_ == 1 << 20:
        na = torch.full((T, od), float("nan"), dtype=torch.float32, device="cuda")
        qmm.mmq_noalloc(w, qact, T, na)
        torch.cuda.synchronize()
        assert np.array_equal(na.cpu().numpy().view(np.uint32), got.view(np.uint32)), "noalloc differs"
    w.release()
    say(f"maximum size {name}: oracle")
    ref, A = oracle.mmq_parallel(synth.block_format(type_), raw, od, id_, q, dh, s)
    check_close(got, ref, A, name)


# --------------------------------------------------------------------------
# properties
# --------------------------------------------------------------------------

@pytest.mark.parametrize("od,id_,T", [(300, 768, 77), (4160, 1024, 512), (1030, 256, 4000), (512, 3072, 300)])
def test_packed_codes_bit_identical_to_byte_codes(od, id_, T):
    """The packed-code registration feeds the matrix cores the same code bytes,
    so its results equal the byte-code registration's bit for bit (both tile
    geometries, a ragged split tail, an all-split launch)."""
    say(f"packed vs byte codes {od}x{id_} T={T}")
    raw, x = synth.case(synth.Q4_K, od, id_, T, seed=8)
    qact = gpu_quantize(x)
    w = qmm.register_weights(synth.Q4_K, od, id_, raw)
    wp = qmm.register_weights(synth.Q4_K_PACKED, od, id_, raw)
    assert wp.plane_bytes < w.plane_bytes
    a, b = run_mmq(w, qact, T), run_mmq(wp, qact, T)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    w.release()
    wp.release()


def test_odd_rows_and_token_tail_are_prefixes_and_repeatable():
    name, type_, od, id_, T, _ = synth.FFN_DOWN
    say("prefix properties at the ffn_down shape")
    raw, x = synth.case(type_, od + 1, id_, T, seed=3)
    w_odd = qmm.register_weights(type_, od + 1, id_, raw)
    w_even = qmm.register_weights(type_, od, id_, raw[: od * (id_ // 256) * 210])
    qact = gpu_quantize(x)
    out_odd = run_mmq(w_odd, qact, T)
    out_even = run_mmq(w_even, qact, T)
    assert np.array_equal(out_odd[:, :od], out_even)
    again = run_mmq(w_odd, qact, T)
    assert np.array_equal(again, out_odd)
    qact509 = gpu_quantize(x[:509])
    out509 = run_mmq(w_odd, qact509, 509)
    assert np.array_equal(out509, out_odd[:509])


@pytest.mark.parametrize("T", [512, 3314])
def test_fused_same_type_gemms_match_separate(T):
    """Row-concatenated registration (gate||up, q||k) on one shared qact: each
    column block of the fused result and the separate GEMM agree with the oracle
    on one random element of every 32 x 32 output block.  At 3314 tokens gate||up (22016 rows) and gate, up alone
    (11008 rows) use the same tile geometry and fill the GPU's work-group slots
    with no ragged last wave, so the per-element summation order is the same and
    the blocks are bit-identical.  Otherwise the geometry (one or two k-groups)
    or a K-split of a ragged last wave may differ between the two launches,
    which changes only the f32 summation order."""
    say(f"fused gate||up and q||k, T={T}")
    rng = np.random.default_rng(21)
    id_ = 4096
    x = synth.activations(rng, T, id_)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    for od in (11008, 4096):
        raw_a = synth.q4k_weights(rng, od, id_)
        raw_b = synth.q4k_weights(rng, od, id_)
        wa = qmm.register_weights(synth.Q4_K, od, id_, raw_a)
        wb = qmm.register_weights(synth.Q4_K, od, id_, raw_b)
        wf = qmm.register_weights(synth.Q4_K, 2 * od, id_, np.concatenate([raw_a, raw_b]))
        fused = run_mmq(wf, qact, T)
        ts, js = _stratified_pairs(np.random.default_rng(2), T, od)
        for half, (w, raw) in enumerate(((wa, raw_a), (wb, raw_b))):
            sep = run_mmq(w, qact, T)
            blk = fused[:, half * od:(half + 1) * od]
            ref, A = oracle.mmq_at(synth.Q4_K, raw, od, id_, q, dh, s, ts, js)
            check_close(blk[ts, js], ref, A, f"fused od={2 * od} half {half}")
            check_close(sep[ts, js], ref, A, f"separate od={od} half {half}")
            if od == 11008 and T == 3314:
                assert np.array_equal(blk, sep)
        for w in (wa, wb, wf):
            w.release()


def test_concurrent_streams_share_a_handle():
    """One handle used on two streams at once, on a shape whose ragged last wave
    needs the tail scratch (one buffer per stream): both results equal the
    single-stream result, repeatedly."""
    say("two streams, one handle, tail scratch")
    type_, od, id_, T = synth.Q6_K, 4097, 2048, 509  # 260 tiles on 256 CUs: the tail splits 4 ways
    raw, x = synth.case(type_, od, id_, T, seed=5)
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    ref = run_mmq(w, qact, T)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((T, od), float("nan"), device="cuda") for _ in streams]
    torch.cuda.synchronize()
    for _ in range(3):
        for st, o in zip(streams, outs):
            with torch.cuda.stream(st):
                qmm.mmq(w, qact, T, out=o, stream=st)
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(o.cpu().numpy(), ref)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    if qmm.mmq_plan(type_, od, id_, T, n_cu).scratch_bytes:  # each stream held its own scratch
        assert [qmm.stream_release(st) for st in streams] == [n_cu * 64 * 1024] * 2
    w.release()


def test_noalloc_under_graph_capture():
    """The allocation-free MMQ inside a captured HIP graph, the use it exists
    for: the prepass and a launch whose tail tiles are split into the static
    scratch, captured once and replayed three times, with eager work (poisoning
    the output and the qact buffer) and a synchronization between replays;
    every replay gives the eager result bit for bit."""
    say("noalloc under graph capture")
    type_, od, id_, T = synth.Q6_K, 4097, 2048, 509  # 260 tiles on 256 CUs: the tail splits 4 ways
    raw, x = synth.case(type_, od, id_, T, seed=61)
    w = qmm.register_weights(type_, od, id_, raw)
    xt = torch.from_numpy(x).cuda()
    qact = torch.empty(qmm.qact_bytes(T, id_), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, od), dtype=torch.float32, device="cuda")
    # eager reference; the first call on the device also looks up the static
    # scratch's address, outside the capture
    qmm.quantize_activations(xt, qact)
    qmm.mmq_noalloc(w, qact, T, out)
    torch.cuda.synchronize()
    ref = out.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capturing
        qmm.quantize_activations(xt, qact, stream=side)
        qmm.mmq_noalloc(w, qact, T, out, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qmm.quantize_activations(xt, qact)
        qmm.mmq_noalloc(w, qact, T, out)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        qact.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), f"replay {i} differs"
    del graph
    w.release()


def test_tail_scratch_shared_across_shapes():
    """Launches with different tail tile counts and splits (260 tiles on 256
    CUs with the tail split 4 ways, 24 tiles all split, a q4_K shape with its
    own geometry) share one stream's tail scratch in turn: each repeat gives
    its first result bit for bit, which agrees with the oracle."""
    say("tail scratch across shapes")
    cases = [(synth.Q6_K, 4097, 2048, 509, 21), (synth.Q6_K, 512, 2816, 300, 22),
             (synth.Q4_K, 4160, 1024, 512, 23)]
    runs = []
    for type_, od, id_, T, seed in cases:
        raw, x = synth.case(type_, od, id_, T, seed=seed)
        w = qmm.register_weights(type_, od, id_, raw)
        qact = gpu_quantize(x)
        first = run_mmq(w, qact, T)
        q, dh, sm = oracle.quantize(x)
        ref, A = oracle.mmq(synth.block_format(type_), raw, od, id_, q, dh, sm)
        check_close(first, ref, A, f"type {type_} od {od} T {T}")
        runs.append((w, qact, T, od, first))
    for _ in range(3):
        for w, qact, T, od, first in runs:
            assert np.array_equal(run_mmq(w, qact, T), first)
    for w, *_ in runs:
        w.release()


def test_stream_release_frees_the_scratch():
    """qmm_stream_release gives a stream's tail scratch back (64 KiB per CU,
    counted by the call), and a later MMQ on the same stream allocates it again
    and gives the same bits; a stream that holds nothing releases nothing."""
    say("stream release")
    type_, od, id_, T = synth.Q6_K, 4097, 2048, 509  # 260 tiles on 256 CUs: the tail splits 4 ways
    raw, x = synth.case(type_, od, id_, T, seed=31)
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = torch.empty((T, od), dtype=torch.float32, device="cuda")
        qmm.mmq(w, qact, T, out=out, stream=s)
    s.synchronize()
    first = out.cpu().numpy()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert qmm.stream_release(s) == n_cu * 64 * 1024
    assert qmm.stream_release(s) == 0                          # nothing left
    with torch.cuda.stream(s):
        qmm.mmq(w, qact, T, out=out, stream=s)
    s.synchronize()
    assert np.array_equal(out.cpu().numpy(), first)
    assert qmm.stream_release(s) == n_cu * 64 * 1024
    w.release()


def test_writes_stay_inside_output():
    type_, od, id_, T = synth.Q4_K, 77, 512, 45
    say("output bounds")
    raw, x = synth.case(type_, od, id_, T, seed=4)
    w = qmm.register_weights(type_, od, id_, raw)
    qact = gpu_quantize(x)
    big = torch.full((T * od + 4096,), 12345.0, dtype=torch.float32, device="cuda")
    big[: T * od].fill_(float("nan"))
    qmm.mmq(w, qact, T, out=big[: T * od].view(T, od))
    torch.cuda.synchronize()
    b = big.cpu().numpy()
    assert not np.isnan(b[: T * od]).any()
    assert np.all(b[T * od:] == 12345.0)


def test_shape_mismatch_and_memory_cap():
    say("error paths")
    raw, x = synth.case(synth.Q6_K, 8, 512, 4, seed=1)
    w = qmm.register_weights(synth.Q6_K, 8, 512, raw)
    x2 = np.zeros((4, 768), np.float32)
    qact = gpu_quantize(x2)
    out = torch.empty((4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.mmq(w, qact, 4, out=out)
    assert e.value.code == qmm.ESHAPE
    qmm.set_memory_cap(w.plane_bytes + 1)
    try:
        with pytest.raises(qmm.QmmError) as e:
            qmm.register_weights(synth.Q6_K, 8, 512, raw)
        assert e.value.code == qmm.ENOMEM
    finally:
        qmm.set_memory_cap(0)
    w2 = qmm.register_weights(synth.Q6_K, 8, 512, raw)
    w2.release()
    w.release()


def test_empty_batch_is_a_no_op():
    """n_tok = 0 through the binding: an empty qact and an empty output, nothing
    launched; the handle still serves a normal call afterwards."""
    say("empty batch")
    raw, x = synth.case(synth.Q4_K, 40, 512, 3, seed=2)
    w = qmm.register_weights(synth.Q4_K, 40, 512, raw)
    qa0 = qmm.quantize_activations(torch.empty((0, 512), dtype=torch.float32, device="cuda"))
    assert qa0.numel() == 0
    out0 = qmm.mmq(w, qa0, 0)
    assert tuple(out0.shape) == (0, 40)
    qact = gpu_quantize(x)
    q, dh, s = check_prepass(x, qact)
    ref, A = oracle.mmq(synth.Q4_K, raw, 40, 512, q, dh, s)
    check_close(run_mmq(w, qact, 3), ref, A, "after an empty batch")
    w.release()

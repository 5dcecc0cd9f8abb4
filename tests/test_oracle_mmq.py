"""Pins for the oracle's integer dots (O3) and result (O4).

* textbook special case: unit scales and integer activations whose blocks each
  reach 127 make the q8 scale exactly 1, so the whole product reduces to an exact
  integer matrix product, checked with numpy int64 matmul;
* brute force: dequantize in f64 and multiply with numpy (a different summation
  order and structure), agreement within the stated bound;
* closed forms and special cases: zero-scale blocks contribute exactly zero,
  constant inputs, odd row counts and token tails.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.kq_blocks import Q4K_UNIT_SCALES, q4k_block, q6k_block


def _int_acts(rng, T, id_):
    """Integer activations in [-127, 127] where every 32-block holds a +-127."""
    x = rng.integers(-127, 128, size=(T, id_)).astype(np.float32)
    x.reshape(T, -1, 32)[:, :, 0] = np.where(rng.random((T, id_ // 32)) < 0.5, 127, -127)
    return x


def _q6k_unit_raw(rng, od, id_):
    nb = od * (id_ // 256)
    blocks = [q6k_block(ql=rng.integers(0, 256, 128, dtype=np.uint8),
                        qh=rng.integers(0, 256, 64, dtype=np.uint8), sc=1) for _ in range(nb)]
    return np.concatenate(blocks)


def _q4k_unit_raw(rng, od, id_):
    nb = od * (id_ // 256)
    blocks = [q4k_block(scales=Q4K_UNIT_SCALES, qs=rng.integers(0, 256, 128, dtype=np.uint8))
              for _ in range(nb)]
    return np.concatenate(blocks)


def test_unit_q6k_is_integer_matmul():
    rng = np.random.default_rng(3)
    od, id_, T = 7, 512, 5
    raw = _q6k_unit_raw(rng, od, id_)
    x = _int_acts(rng, T, id_)
    q, dh, s = oracle.quantize(x)
    assert np.all(dh == 0x3C00) and np.array_equal(q, x.astype(np.int8))
    w, _, _ = oracle.decode_q6k(raw, od, id_)
    ref = x.astype(np.int64) @ w.astype(np.int64).T
    out, A = oracle.mmq(oracle.Q6_K, raw, od, id_, q, dh, s)
    assert np.array_equal(out, ref.astype(np.float64))
    D16, J = oracle.dots_q6k(raw, od, id_, q)
    ref16 = np.einsum("tgk,jgk->tjg", x.astype(np.int64).reshape(T, -1, 16),
                      w.astype(np.int64).reshape(od, -1, 16))
    assert np.array_equal(D16, ref16)
    assert np.array_equal(J, ref16.reshape(T, od, -1, 2).sum(axis=3))


def test_unit_q4k_is_integer_matmul():
    rng = np.random.default_rng(4)
    od, id_, T = 6, 768, 3
    raw = _q4k_unit_raw(rng, od, id_)
    x = _int_acts(rng, T, id_)
    q, dh, s = oracle.quantize(x)
    w, sc, mn, d, dm = oracle.decode_q4k(raw, od, id_)
    assert np.all(sc == 1) and np.all(mn == 0) and np.all(d == 1) and np.all(dm == 0)
    ref = x.astype(np.int64) @ w.astype(np.int64).T
    out, A = oracle.mmq(oracle.Q4_K, raw, od, id_, q, dh, s)
    assert np.array_equal(out, ref.astype(np.float64))
    D32 = oracle.dots_q4k(raw, od, id_, q)
    ref32 = np.einsum("tck,jck->tjc", x.astype(np.int64).reshape(T, -1, 32),
                      w.astype(np.int64).reshape(od, -1, 32))
    assert np.array_equal(D32, ref32)


def test_q6k_scale_folded_dots_at_full_range_scales():
    """J (the block dot carrying both 16-group scales) at full-range int8 scales
    against an independent numpy int64 product of the scale-folded weights
    sc[k/16] * (code - 32): per 32-block, and summed over the row (d = 1 and
    integer activations with dh = 1 make the result that exact integer matmul)."""
    rng = np.random.default_rng(12)
    od, id_, T = 6, 768, 5
    nb = od * (id_ // 256)
    blocks = [q6k_block(ql=rng.integers(0, 256, 128, dtype=np.uint8),
                        qh=rng.integers(0, 256, 64, dtype=np.uint8),
                        sc=rng.integers(-128, 128, 16).astype(np.int8)) for _ in range(nb)]
    raw = np.concatenate(blocks)
    x = _int_acts(rng, T, id_)
    q, dh, s = oracle.quantize(x)
    assert np.all(dh == 0x3C00)
    w, sc, d = oracle.decode_q6k(raw, od, id_)
    assert np.all(d == 1.0) and sc.min() < -100 and sc.max() > 100
    folded = w.astype(np.int64) * np.repeat(sc.astype(np.int64), 16, axis=1)     # [od][id]
    Jref = np.einsum("tck,jck->tjc", x.astype(np.int64).reshape(T, -1, 32), folded.reshape(od, -1, 32))
    D16, J = oracle.dots_q6k(raw, od, id_, q)
    assert np.array_equal(J, Jref)
    out, _ = oracle.mmq(oracle.Q6_K, raw, od, id_, q, dh, s)
    assert np.array_equal(out, (x.astype(np.int64) @ folded.T).astype(np.float64))


def _brute_force(type_, raw, od, id_, q, dh, s):
    """Dequantize both sides in f64 and multiply; returns (ref, extra bound)."""
    T = q.shape[0]
    dhv = np.asarray(dh, np.uint16).view(np.float16).astype(np.float64)
    a = q.astype(np.float64) * np.repeat(dhv, 32, axis=1)
    if type_ == oracle.Q6_K:
        w, sc, d = oracle.decode_q6k(raw, od, id_)
        y = (w.astype(np.float64) * np.repeat(sc.astype(np.float64), 16, axis=1)
             * np.repeat(d.astype(np.float64), 256, axis=1))
        return a @ y.T, np.zeros((T, od))
    w, sc, mn, d, dm = oracle.decode_q4k(raw, od, id_)
    y = (w.astype(np.float64) * np.repeat(sc.astype(np.float64), 32, axis=1)
         * np.repeat(d.astype(np.float64), 256, axis=1)
         - np.repeat(mn.astype(np.float64) * np.repeat(dm.astype(np.float64), 8, axis=1), 32, axis=1))
    ref = a @ y.T
    # the oracle's min term uses the stored f16 scaled sum s instead of dh * sum(q)
    sv = np.asarray(s, np.uint16).view(np.float16).astype(np.float64)
    S = q.reshape(T, -1, 32).astype(np.float64).sum(axis=2)
    ds = np.abs(sv - dhv * S)                       # [T][nchunk]
    wm = np.abs(mn.astype(np.float64) * np.repeat(dm.astype(np.float64), 8, axis=1))  # [od][nchunk]
    return ref, ds @ wm.T


@pytest.mark.parametrize("type_,od,id_,T", [(synth.Q6_K, 9, 512, 11), (synth.Q4_K, 10, 768, 7),
                                            (synth.Q6_K, 3, 1024, 2), (synth.Q4_K, 1, 256, 1)])
def test_matches_f64_brute_force(type_, od, id_, T):
    raw, x = synth.case(type_, od, id_, T, seed=11, outliers=True)
    q, dh, s = oracle.quantize(x)
    out, A = oracle.mmq(type_, raw, od, id_, q, dh, s)
    ref, extra = _brute_force(type_, raw, od, id_, q, dh, s)
    assert np.all(np.abs(out - ref) <= 1e-12 * A + extra)
    assert np.all(A >= np.abs(out)) and np.all(A > 0)


def test_per_pair_and_row_slices_agree_with_full():
    raw, x = synth.case(synth.Q4_K, 12, 512, 9, seed=5)
    q, dh, s = oracle.quantize(x)
    out, A = oracle.mmq(synth.Q4_K, raw, 12, 512, q, dh, s)
    o2, a2 = oracle.mmq_rows(synth.Q4_K, raw, 12, 512, q, dh, s, 3, 10)
    assert np.array_equal(o2, out[:, 3:10]) and np.array_equal(a2, A[:, 3:10])
    o4, a4 = oracle.mmq_parallel(synth.Q4_K, raw, 12, 512, q, dh, s, threads=3)
    assert np.array_equal(o4, out) and np.array_equal(a4, A)
    ts = np.array([0, 8, 4, 4]); js = np.array([0, 0, 11, 5])
    o3, a3 = oracle.mmq_at(synth.Q4_K, raw, 12, 512, q, dh, s, ts, js)
    assert np.array_equal(o3, out[ts, js]) and np.array_equal(a3, A[ts, js])


def test_odd_rows_and_token_tail_are_prefixes():
    raw, x = synth.case(synth.Q6_K, 5, 512, 16, seed=9)
    q, dh, s = oracle.quantize(x)
    out5, _ = oracle.mmq(synth.Q6_K, raw, 5, 512, q, dh, s)
    raw4 = raw[: 4 * 2 * 210]
    out4, _ = oracle.mmq(synth.Q6_K, raw4, 4, 512, q, dh, s)
    assert np.array_equal(out4, out5[:, :4])
    q13, dh13, s13 = oracle.quantize(x[:13])
    out13, _ = oracle.mmq(synth.Q6_K, raw, 5, 512, q13, dh13, s13)
    assert np.array_equal(out13, out5[:13])


@pytest.mark.parametrize("type_", [synth.Q6_K, synth.Q4_K])
def test_zero_scale_block_contributes_nothing(type_):
    od, id_, T = 4, 768, 6
    raw, x = synth.case(type_, od, id_, T, seed=2)
    q, dh, s = oracle.quantize(x)
    blk = synth.BLOCK_BYTES[type_]
    nsb = id_ // 256
    z = raw.copy().reshape(od * nsb, blk)
    row, b = 2, 1
    if type_ == synth.Q6_K:
        z[row * nsb + b, 208:210] = 0          # d = 0
    else:
        z[row * nsb + b, 0:4] = 0              # d = dmin = 0
    z = z.reshape(-1)
    out, _ = oracle.mmq(type_, z, od, id_, q, dh, s)
    # the same row with that block's 256 activations zeroed instead
    xz = x.copy()
    xz[:, 256 * b: 256 * (b + 1)] = 0
    qz, dhz, sz = oracle.quantize(xz)
    ref, _ = oracle.mmq(type_, raw, od, id_, qz, dhz, sz)
    assert np.array_equal(out[:, row], ref[:, row])
    # every block of a row at d = dmin = 0 gives exactly zero
    zz = z.reshape(od * nsb, blk).copy()
    for bb in range(nsb):
        if type_ == synth.Q6_K:
            zz[row * nsb + bb, 208:210] = 0
        else:
            zz[row * nsb + bb, 0:4] = 0
    out0, _ = oracle.mmq(type_, zz.reshape(-1), od, id_, q, dh, s)
    assert np.all(out0[:, row] == 0)


def test_q6k_closed_form_constant_inputs():
    # every code 48 (weight 16), every scale 5, d = 1/8; activations all 1.0
    od, id_, T = 2, 512, 3
    raw = np.concatenate([q6k_block(ql=0x00, qh=0xFF, sc=5, d_bits=0x3000)] * (od * 2))
    x = np.ones((T, id_), np.float32)
    q, dh, s = oracle.quantize(x)
    dhv = float(np.asarray(dh[0, 0], np.uint16).view(np.float16))
    qv = int(q[0, 0])
    assert np.all(q == qv) and abs(1.0 - dhv * qv) <= dhv / 2
    out, _ = oracle.mmq(synth.Q6_K, raw, od, id_, q, dh, s)
    assert np.all(out == id_ * 0.125 * 5 * 16 * dhv * qv)


def test_q4k_closed_form_constant_inputs():
    # codes all 3, scales 1, mins 0 except: dmin = 1/4 with min 2 on every sub-block
    scales = Q4K_UNIT_SCALES.copy()
    scales[4:8] = 2                      # min of sub-blocks 0..3
    scales[8:12] |= 2 << 4               # min of sub-blocks 4..7 (high nibble)
    od, id_, T = 3, 256, 2
    raw = np.concatenate([q4k_block(d_bits=0x3C00, dmin_bits=0x3400, scales=scales, qs=0x33)] * od)
    w, sc, mn, d, dm = oracle.decode_q4k(raw, od, id_)
    assert np.all(mn == 2) and np.all(sc == 1) and np.all(w == 3)
    x = np.full((T, id_), 2.0, np.float32)
    q, dh, s = oracle.quantize(x)
    dhv = float(np.asarray(dh[0, 0], np.uint16).view(np.float16))
    sv = float(np.asarray(s[0, 0], np.uint16).view(np.float16))
    qv = int(q[0, 0])
    out, _ = oracle.mmq(synth.Q4_K, raw, od, id_, q, dh, s)
    expect = 8 * (1.0 * 1 * dhv * (3 * qv * 32) - 0.25 * 2 * sv)
    assert np.all(out == expect)

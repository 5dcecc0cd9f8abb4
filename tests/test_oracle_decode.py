"""Pins for the oracle's weight decode (O1).

The block struct offsets come from the engineering log's r56 page (q6_K: ql, qh,
int8 scales at 192, f16 d at 208) and r58 page (q4_K: qs at 16; the 6-bit
scale/min unpack).  The element bit layouts inside ql/qh/qs and the 12-byte
scale/min packing are the public ggml conventions; no implementation of them is
available here to compare against, so they are pinned by literal spot values
taken from the format description and by structural properties (every bit used
exactly once), not cross-checked against llama.cpp.
"""
import numpy as np
import pytest

import oracle
from tests.kq_blocks import q4k_block, q6k_block


def _dec6(block):
    return oracle.decode_q6k(block, 1, 256)


def _dec4(block):
    return oracle.decode_q4k(block, 1, 256)


# --- q6_K ------------------------------------------------------------------

@pytest.mark.parametrize("ql,qh,code", [(0x00, 0x00, 0), (0x00, 0xFF, 48), (0xFF, 0x00, 15),
                                        (0xFF, 0xFF, 63), (0x55, 0xAA, 0x25)])
def test_q6k_constant_patterns(ql, qh, code):
    # qh = 0xAA sets bits 1,3,5,7 -> every element's 2-bit field is 0b10
    w, _, _ = _dec6(q6k_block(ql=ql, qh=qh))
    assert np.all(w == code - 32)


def _q6k_bit_map():
    base, _, _ = _dec6(q6k_block())
    hits = {}
    for byte in range(192):
        for bit in range(8):
            blk = q6k_block()
            blk[byte] |= 1 << bit
            w, _, _ = _dec6(blk)
            diff = w[0].astype(int) - base[0].astype(int)
            nz = np.nonzero(diff)[0]
            assert nz.size == 1, (byte, bit)
            hits[(byte, bit)] = (int(nz[0]), int(diff[nz[0]]))
    return hits


def test_q6k_every_code_bit_used_exactly_once():
    hits = _q6k_bit_map()
    per_elem = {}
    for (byte, bit), (e, inc) in hits.items():
        per_elem.setdefault(e, []).append(inc)
    assert sorted(per_elem) == list(range(256))
    for e, incs in per_elem.items():
        assert sorted(incs) == [1, 2, 4, 8, 16, 32], e


def test_q6k_spot_positions():
    hits = _q6k_bit_map()
    # ql low nibbles carry elements 0-31 / 32-63 of each half, high nibbles 64-95 / 96-127
    assert hits[(0, 0)] == (0, 1)
    assert hits[(0, 4)] == (64, 1)
    assert hits[(32, 0)] == (32, 1)
    assert hits[(32, 7)] == (96, 8)
    assert hits[(64, 0)] == (128, 1)
    assert hits[(127, 7)] == (255, 8)
    # qh bit pairs 0-1, 2-3, 4-5, 6-7 are the top bits of quarters 0..3 of a half
    assert hits[(128 + 0, 0)] == (0, 16)
    assert hits[(128 + 0, 3)] == (32, 32)
    assert hits[(128 + 0, 4)] == (64, 16)
    assert hits[(128 + 0, 6)] == (96, 16)
    assert hits[(128 + 32, 0)] == (128, 16)
    assert hits[(128 + 63, 7)] == (255, 32)


def test_q6k_scales_and_d():
    sc = np.arange(-8, 8, dtype=np.int8) * 16  # includes -128
    _, dsc, d = _dec6(q6k_block(sc=sc, d_bits=0x0001))
    assert np.array_equal(dsc[0], sc)
    assert d[0, 0] == np.float32(2.0 ** -24)  # smallest subnormal, exact
    _, _, d = _dec6(q6k_block(d_bits=0xB800))
    assert d[0, 0] == -0.5


def test_q6k_rows_and_blocks_are_row_major():
    b0 = q6k_block(ql=0x11, sc=1, d_bits=0x3C00)
    b1 = q6k_block(ql=0x22, sc=2, d_bits=0x4000)
    b2 = q6k_block(ql=0x33, sc=3, d_bits=0x4200)
    b3 = q6k_block(ql=0x44, sc=4, d_bits=0x4400)
    raw = np.concatenate([b0, b1, b2, b3])
    w, sc, d = oracle.decode_q6k(raw, 2, 512)
    assert np.all(w[0, :256] == 1 - 32) and np.all(w[0, 256:] == 2 - 32)
    assert np.all(w[1, :256] == 3 - 32) and np.all(w[1, 256:] == 4 - 32)
    assert np.array_equal(d, np.array([[1.0, 2.0], [3.0, 4.0]], np.float32))
    assert np.all(sc[1, 16:] == 4)


# --- q4_K ------------------------------------------------------------------

def _q4k_scale_bit_map():
    _, sc0, mn0, _, _ = _dec4(q4k_block(scales=0))
    hits = {}
    for byte in range(12):
        for bit in range(8):
            s = np.zeros(12, np.uint8)
            s[byte] = 1 << bit
            _, sc, mn, _, _ = _dec4(q4k_block(scales=s))
            dsc = np.nonzero(sc[0] != sc0[0])[0]
            dmn = np.nonzero(mn[0] != mn0[0])[0]
            assert dsc.size + dmn.size == 1, (byte, bit)
            if dsc.size:
                hits[(byte, bit)] = ("sc", int(dsc[0]), int(sc[0, dsc[0]]))
            else:
                hits[(byte, bit)] = ("mn", int(dmn[0]), int(mn[0, dmn[0]]))
    return hits


def test_q4k_scale_min_bits_each_used_once():
    hits = _q4k_scale_bit_map()
    fields = {}
    for (_, _), (kind, c, val) in hits.items():
        fields.setdefault((kind, c), []).append(val)
    assert len(fields) == 16
    for key, vals in fields.items():
        assert sorted(vals) == [1, 2, 4, 8, 16, 32], key


def test_q4k_scale_min_spot_values():
    hits = _q4k_scale_bit_map()
    assert hits[(0, 0)] == ("sc", 0, 1)      # byte 4+0, low 6 bits: scale of sub-block 0
    assert hits[(3, 5)] == ("sc", 3, 32)
    assert hits[(4, 0)] == ("mn", 0, 1)      # byte 4+4: min of sub-block 0
    assert hits[(0, 6)] == ("sc", 4, 16)     # top bits of byte 0 -> bits 4-5 of scale 4
    assert hits[(4, 7)] == ("mn", 4, 32)     # top bits of byte 4 -> bits 4-5 of min 4
    assert hits[(8, 0)] == ("sc", 4, 1)      # low nibble of byte 8: scale 4
    assert hits[(8, 4)] == ("mn", 4, 1)      # high nibble of byte 8: min 4
    assert hits[(11, 7)] == ("mn", 7, 8)


def test_q4k_code_layout_spots():
    base = _dec4(q4k_block())[0][0].astype(int)
    def hit(byte, bit):
        qs = np.zeros(128, np.uint8)
        qs[byte] = 1 << bit
        w = _dec4(q4k_block(qs=qs))[0][0].astype(int)
        nz = np.nonzero(w - base)[0]
        assert nz.size == 1
        return int(nz[0]), int((w - base)[nz[0]])
    assert hit(0, 0) == (0, 1)
    assert hit(0, 4) == (32, 1)
    assert hit(31, 7) == (63, 8)
    assert hit(32, 0) == (64, 1)
    assert hit(64, 4) == (160, 1)
    assert hit(127, 7) == (255, 8)
    seen = set()
    for byte in range(128):
        for bit in (0, 4):
            seen.add(hit(byte, bit)[0])
    assert seen == set(range(256))


def test_q4k_d_dmin():
    _, _, _, d, dm = _dec4(q4k_block(d_bits=0x3800, dmin_bits=0x0003))
    assert d[0, 0] == 0.5
    assert dm[0, 0] == np.float32(3 * 2.0 ** -24)

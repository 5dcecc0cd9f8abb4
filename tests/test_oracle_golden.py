"""Pins of the oracle against the format facts the pages print
(tests/golden/format_facts.txt, each with its citation): blocks are assembled
from those offsets alone, with every code field uniform so that the result does
not depend on the element bit layouts (readings pinned elsewhere), and the
oracle's full MMQ, driven with one-hot activations, must return each weight's
closed-form value d*sc*(code - 32) (q6_K) or d*sc*code - dmin*min (q4_K)."""
import os

import numpy as np

import oracle
import quant_q8_gemm_amd as qmm

HERE = os.path.dirname(os.path.abspath(__file__))


def _facts():
    facts = {}
    for line in open(os.path.join(HERE, "golden", "format_facts.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            key, value = (p.strip() for p in line.split("=", 1))
            facts[key] = int(value) if value.lstrip("-").isdigit() else value
    return facts


F = _facts()
SB = F["superblock_weights"]


def _f16(v):
    return np.array([v], np.float16).view(np.uint16)[0]


def _one_hot(id_):
    """Token t selects weight t: q = 1 there, dh = 1 in every chunk, s = dh*sum(q)."""
    T = id_
    q = np.eye(T, id_, dtype=np.int8)
    dh = np.full((T, id_ // 32), _f16(1.0), np.uint16)
    s = np.zeros((T, id_ // 32), np.uint16)
    s[np.arange(T), np.arange(T) // 32] = _f16(1.0)
    return q, dh, s


def test_q6k_weights_from_printed_offsets():
    nsb = 2
    block_bytes = F["q6k.d_offset"] + 2  # the f16 d closes the block
    raw = np.zeros(nsb * block_bytes, np.uint8)
    groups = F["q6k.chunks_per_superblock"] * F["q6k.scale_groups_per_chunk"]
    expect = np.zeros(nsb * SB)
    for b in range(nsb):
        blk = raw[b * block_bytes:(b + 1) * block_bytes]
        # every 6-bit code 33 (low nibbles 1, high 2-bit fields 0b10): code - 32 = 1
        blk[:F["q6k.scales_offset"] - 64] = 0x11
        blk[F["q6k.scales_offset"] - 64:F["q6k.scales_offset"]] = 0xAA
        sc = np.array([(g - 8) * (b + 1) for g in range(groups)], np.int8)  # signed, distinct
        blk[F["q6k.scales_offset"]:F["q6k.scales_offset"] + groups] = sc.view(np.uint8)
        d = 0.5 + 0.25 * b
        blk[F["q6k.d_offset"]:F["q6k.d_offset"] + 2] = np.array([_f16(d)]).view(np.uint8)
        for e in range(SB):
            chunk, half = divmod(e, 32)
            # chunk c uses the pair sc[2c], sc[2c+1]: the first 16 weights take sc[2c]
            expect[b * SB + e] = d * int(sc[2 * chunk + half // 16])
    q, dh, s = _one_hot(nsb * SB)
    out, _ = oracle.mmq(qmm.Q6_K, raw, 1, nsb * SB, q, dh, s)
    assert np.array_equal(out[:, 0], expect)


def test_q4k_weights_from_printed_offsets():
    nsb = 2
    raw = np.zeros(nsb * F["q4k.block_bytes"], np.uint8)
    expect = np.zeros(nsb * SB)
    sc, mn, code = 5, 7, 3
    for b in range(nsb):
        blk = raw[b * F["q4k.block_bytes"]:(b + 1) * F["q4k.block_bytes"]]
        d, dmin = 0.5 + 0.25 * b, 0.125 * (b + 1)
        blk[0:2] = np.array([_f16(d)]).view(np.uint8)
        blk[2:4] = np.array([_f16(dmin)]).view(np.uint8)
        # the 12 scale/min bytes between dmin and the codes: every sub-block
        # scale 5 and min 7 (values below 16 sit in the low bits of every
        # packing of 6-bit pairs into 12 bytes)
        scales = blk[4:F["q4k.qs_offset"]]
        assert len(scales) == 12
        scales[0:4], scales[4:8], scales[8:12] = sc, mn, (mn << 4) | sc
        qs = blk[F["q4k.qs_offset"]:F["q4k.qs_offset"] + F["q4k.qs_bytes"]]
        assert len(qs) == F["q4k.qs_bytes"] == SB // 2
        qs[:] = (code << 4) | code
        expect[b * SB:(b + 1) * SB] = d * sc * code - dmin * mn
    q, dh, s = _one_hot(nsb * SB)
    out, _ = oracle.mmq(qmm.Q4_K, raw, 1, nsb * SB, q, dh, s)
    assert np.allclose(out[:, 0], expect, rtol=0, atol=1e-12)


def test_a_misplaced_field_changes_the_result():
    """The pins above see the offsets: the same q4_K block with its codes moved
    four bytes down (into the scale bytes) decodes differently."""
    raw = np.zeros(F["q4k.block_bytes"], np.uint8)
    raw[0:2] = np.array([_f16(1.0)]).view(np.uint8)
    raw[4:16] = [5, 5, 5, 5, 7, 7, 7, 7, 0x75, 0x75, 0x75, 0x75]
    raw[F["q4k.qs_offset"]:] = 0x33
    q, dh, s = _one_hot(SB)
    good, _ = oracle.mmq(qmm.Q4_K, raw, 1, SB, q, dh, s)
    moved = raw.copy()
    moved[F["q4k.qs_offset"] - 4:F["q4k.qs_offset"] - 4 + 8] = 0x33
    bad, _ = oracle.mmq(qmm.Q4_K, moved, 1, SB, q, dh, s)
    assert not np.array_equal(good, bad)


def test_q8_chunk_bytes_match_the_qact_size():
    """32 code bytes and a 4-byte scale pair per 32-activation chunk."""
    per_chunk = F["q8.chunk_code_bytes"] + F["q8.chunk_pair_bytes"]
    for n_tok, id_ in [(1, 256), (300, 4096), (3314, 11008 // 256 * 256)]:
        t_pad = -(-n_tok // qmm.TOKEN_PAD) * qmm.TOKEN_PAD
        assert qmm.qact_bytes(n_tok, id_) == t_pad * (id_ // 32) * per_chunk
    assert qmm.qact_bytes(1, SB + 32) == 0  # whole super-blocks only

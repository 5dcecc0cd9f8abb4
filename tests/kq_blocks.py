"""Byte assembly of single k-quant blocks for hand-made test inputs.

Only the block struct offsets are encoded here (q6_K: ql at 0, qh at 128, the
sixteen int8 scales at 192, f16 d at 208; q4_K: f16 d at 0, f16 dmin at 2, the
twelve scale/min bytes at 4, qs at 16), as the engineering log's r56 and r58
pages state them.  No element bit layout lives here.
"""
import numpy as np

F16_ONE = 0x3C00


def q6k_block(ql=0, qh=0, sc=0, d_bits=F16_ONE) -> np.ndarray:
    b = np.zeros(210, np.uint8)
    b[0:128] = np.broadcast_to(np.asarray(ql, np.uint8), (128,))
    b[128:192] = np.broadcast_to(np.asarray(qh, np.uint8), (64,))
    b[192:208] = np.broadcast_to(np.asarray(sc, np.int8), (16,)).view(np.uint8)
    b[208] = d_bits & 0xFF
    b[209] = d_bits >> 8
    return b


def q4k_block(d_bits=F16_ONE, dmin_bits=0, scales=0, qs=0) -> np.ndarray:
    b = np.zeros(144, np.uint8)
    b[0] = d_bits & 0xFF
    b[1] = d_bits >> 8
    b[2] = dmin_bits & 0xFF
    b[3] = dmin_bits >> 8
    b[4:16] = np.broadcast_to(np.asarray(scales, np.uint8), (12,))
    b[16:144] = np.broadcast_to(np.asarray(qs, np.uint8), (128,))
    return b


# Twelve scale/min bytes that give every sub-block scale 1 and min 0.
Q4K_UNIT_SCALES = np.array([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1], np.uint8)

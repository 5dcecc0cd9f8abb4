"""Test-side readers of the byte layouts include/qmm.h documents (the qact buffer
and the exported weight planes), written from the header's formulas."""
import numpy as np

TOKEN_PAD = 128


def t_pad(n_tok: int) -> int:
    return (n_tok + TOKEN_PAD - 1) // TOKEN_PAD * TOKEN_PAD


def read_qact(buf: np.ndarray, n_tok: int, id_: int):
    """qact bytes -> (q [T_pad][id] int8, dh [T_pad][id/32] u16, s [T_pad][id/32] u16)."""
    tp = t_pad(n_tok)
    nchunk = id_ // 32
    buf = np.asarray(buf, np.uint8)
    assert buf.size == tp * id_ * 9 // 8
    qp = buf[: tp * id_].view(np.int8).reshape(tp // 32, nchunk, 2, 32, 16)
    q = qp.transpose(0, 3, 1, 2, 4).reshape(tp, id_)
    sp = buf[tp * id_:].view("<u2").reshape(tp // 32, nchunk, 32, 2)
    sp = sp.transpose(0, 2, 1, 3).reshape(tp, nchunk, 2)
    return q, sp[:, :, 0].copy(), sp[:, :, 1].copy()


def read_planes(buf: np.ndarray, type_: int, od_pad: int, id_: int, wd_offset: int, sm_offset: int) -> dict:
    """exported planes -> dict.  q6_K: w [od_pad][id] int32 folded weights
    64*hi + lo, d [od_pad][nsb] f32.  q4_K: codes [od_pad][id] int32, d25
    [od_pad][nsb] f32 (d times 2^25), ndmin [od_pad][nsb] f32 (-dmin), sc and mn
    [od_pad][nchunk] binary16 bit patterns (type 14, packed q4_K: the same, its
    codes read from the nibbles).  The q4_K values come from the stage records;
    the two records of a super-block must agree on its mins, d and dmin."""
    nchunk, nsb = id_ // 32, id_ // 256
    R = od_pad // 32
    buf = np.asarray(buf, np.uint8)
    if type_ == 6:
        assert sm_offset == buf.size
        wq = buf[: od_pad * id_ * 2].view(np.int8).reshape(R, nchunk, 2, 2, 32, 16)
        hi = wq[:, :, 0].transpose(0, 3, 1, 2, 4).reshape(od_pad, id_).astype(np.int32)
        lo = wq[:, :, 1].transpose(0, 3, 1, 2, 4).reshape(od_pad, id_).astype(np.int32)
        assert lo.min() >= 0 and lo.max() <= 63
        w = hi * 64 + lo
        d = buf[wd_offset: wd_offset + od_pad * nsb * 4].view("<f4").reshape(R, nsb, 32)
        return {"w": w, "d": d.transpose(0, 2, 1).reshape(od_pad, nsb)}
    assert wd_offset == buf.size
    if type_ == 14:  # packed: [R][nchunk][k-half h][row][8]: codes 16h + b (low nibble), + b + 8 (high)
        pk = buf[: od_pad * id_ // 2].reshape(R, nchunk, 2, 32, 8)
        both = np.concatenate([pk & 15, pk >> 4], axis=4)        # [..][16]: k%16 = 0..7 low, 8..15 high
        codes = both.transpose(0, 3, 1, 2, 4).reshape(od_pad, id_).astype(np.int32)
    else:  # [R][nchunk][k-half h][row][16]: code k = 16h + byte
        pk = buf[: od_pad * id_].view(np.int8).reshape(R, nchunk, 2, 32, 16)
        codes = pk.transpose(0, 3, 1, 2, 4).reshape(od_pad, id_).astype(np.int32)
    assert codes.min() >= 0 and codes.max() <= 15
    # stage records [R][nsb][stage of the super-block][1024 bytes]
    rec = buf[sm_offset: sm_offset + R * nsb * 2 * 1024].reshape(R, nsb, 2, 1024)
    # +0: scales [row][chunk%4] of the stage's chunks
    sc = rec[..., :256].copy().view("<u2").reshape(R, nsb, 2, 32, 4)
    sc = sc.transpose(0, 3, 1, 2, 4).reshape(od_pad, nchunk)
    # +256: mins [chunk%8 / 4][row][chunk%4] of the super-block, in both of its records
    mn2 = rec[..., 256:768].copy().view("<u2").reshape(R, nsb, 2, 2, 32, 4)
    assert np.array_equal(mn2[:, :, 0], mn2[:, :, 1]), "the two records of a super-block disagree on its mins"
    mn = mn2[:, :, 0].transpose(0, 3, 1, 2, 4).reshape(od_pad, nchunk)
    # +768: (d*2^25, -dmin) [part][row], in both records
    dd2 = rec[..., 768:].copy().view("<u4").reshape(R, nsb, 2, 2, 32)
    assert np.array_equal(dd2[:, :, 0], dd2[:, :, 1]), "the two records of a super-block disagree on d, dmin"
    dd = dd2[:, :, 0].copy().view("<f4").transpose(0, 3, 1, 2).reshape(od_pad, nsb, 2)
    return {"codes": codes, "d25": dd[..., 0].copy(), "ndmin": dd[..., 1].copy(), "sc": sc.copy(), "mn": mn.copy()}

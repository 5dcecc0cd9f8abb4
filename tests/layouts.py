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


def read_planes(buf: np.ndarray, type_: int, od_pad: int, id_: int, wd_offset: int, mn_offset: int,
                dm_offset: int, sc_offset: int):
    """exported planes -> (w [od_pad][id] int32 scale-carrying weights: q6_K the
    folded 64*hi + lo, q4_K scale * code; d [od_pad][nsb] f32; for q4_K the mins
    [od_pad][nchunk] (decoded from their f16 values) and dmin [od_pad][nsb] f32,
    else None, None)."""
    nchunk, nsb = id_ // 32, id_ // 256
    R = od_pad // 32
    buf = np.asarray(buf, np.uint8)
    if type_ == 6:
        wq = buf[: od_pad * id_ * 2].view(np.int8).reshape(R, nchunk, 2, 2, 32, 16)
        hi = wq[:, :, 0].transpose(0, 3, 1, 2, 4).reshape(od_pad, id_).astype(np.int32)
        lo = wq[:, :, 1].transpose(0, 3, 1, 2, 4).reshape(od_pad, id_).astype(np.int32)
        assert lo.min() >= 0 and lo.max() <= 63
        w = hi * 64 + lo
    else:
        # [R][nchunk][k-half h][row][16]: code k = 16h + byte
        pk = buf[: od_pad * id_].view(np.int8).reshape(R, nchunk, 2, 32, 16)
        codes = pk.transpose(0, 3, 1, 2, 4).reshape(od_pad, id_).astype(np.int32)
        assert codes.min() >= 0 and codes.max() <= 15
        # scales: binary16 [R][nsb][chunk/4][row][chunk%4], like the mins
        s16 = buf[sc_offset: sc_offset + od_pad * nchunk * 2].view("<f2").reshape(R, nsb, 2, 32, 4)
        sf = s16.astype(np.float64).transpose(0, 3, 1, 2, 4).reshape(od_pad, nchunk)
        assert np.all(sf == np.round(sf)) and sf.min() >= 0 and sf.max() <= 63
        sc = sf.astype(np.int32)
        w = codes * np.repeat(sc, 32, axis=1)
    d = buf[wd_offset: wd_offset + od_pad * nsb * 4].view("<f4").reshape(R, nsb, 32)
    d = d.transpose(0, 2, 1).reshape(od_pad, nsb)
    mn = dm = None
    if type_ == 4:
        # mins: binary16 [R][nsb][chunk/4][row][chunk%4] (chunk within the super-block)
        m16 = buf[mn_offset: mn_offset + od_pad * nchunk * 2].view("<f2").reshape(R, nsb, 2, 32, 4)
        mf = m16.astype(np.float64).transpose(0, 3, 1, 2, 4).reshape(od_pad, nchunk)
        assert np.all(mf == np.round(mf)) and mf.min() >= 0 and mf.max() <= 63
        mn = mf.astype(np.int32)
        dm = buf[dm_offset: dm_offset + od_pad * nsb * 4].view("<f4").reshape(R, nsb, 32)
        dm = dm.transpose(0, 2, 1).reshape(od_pad, nsb)
    return w, d, mn, dm

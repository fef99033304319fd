"""Record-format readers for the tests, written from the bit layouts defined
in include/turboquant.h. Independent of the oracle's packers (which write
records) and of the library (which also writes them)."""
from __future__ import annotations

import numpy as np


def _bits(words: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(words).astype("<u4", copy=False)
    return np.unpackbits(w.view(np.uint8).reshape(w.shape[0], -1), axis=1, bitorder="little")


def unpack_token_major(codes, signs, norms, dims, bits, mse_only=False):
    """codes [n, Wc], signs [n, Ws] uint32, norms [n, 2G] -> per group lists of
    codes [n, d_g] int64, sign bits [n, d_g] bool, n_g [n], gamma_g [n].
    MSE-only records have no sign words: their sign bits come back None."""
    cb, sb = _bits(codes), _bits(signs)
    out_c, out_s, out_n, out_g = [], [], [], []
    cw = sw = 0
    for g, (d, m) in enumerate(zip(dims, bits)):
        j = np.arange(d)
        val = np.zeros((codes.shape[0], d), np.int64)
        for p in range(m):
            val |= cb[:, 32 * cw + m * j + p].astype(np.int64) << p
        out_c.append(val)
        out_s.append(None if mse_only else sb[:, 32 * sw + j].astype(bool))
        out_n.append(np.asarray(norms)[:, 2 * g])
        out_g.append(np.asarray(norms)[:, 2 * g + 1])
        cw += (m * d + 31) // 32
        sw += (d + 31) // 32
    return out_c, out_s, out_n, out_g


def unpack_block32(codes, signs, norms, dims, bits, mse_only=False):
    """codes [n_blocks, BCW], signs [n_blocks, BSW] uint32, norms [32 n_blocks, 2G]
    -> per group codes [32 n_blocks, d_g], bits, n_g, gamma_g (rows in order)."""
    nb = codes.shape[0]
    cb, sb = _bits(codes), _bits(signs)
    t = np.arange(32)
    o, s = t // 8, t % 8
    out_c, out_s, out_n, out_g = [], [], [], []
    cw = sw = 0
    for g, (d, m) in enumerate(zip(dims, bits)):
        j = np.arange(d)
        pos = 8 * m * (o[:, None] * d + j[None, :]) + m * s[:, None]        # [32, d]
        val = np.zeros((nb, 32, d), np.int64)
        for p in range(m):
            val |= cb[:, 32 * cw + pos + p].astype(np.int64) << p
        spos = 8 * (o[:, None] * d + j[None, :]) + s[:, None]
        out_c.append(val.reshape(nb * 32, d))
        out_s.append(None if mse_only else sb[:, 32 * sw + spos].astype(bool).reshape(nb * 32, d))
        out_n.append(np.asarray(norms)[:, 2 * g])
        out_g.append(np.asarray(norms)[:, 2 * g + 1])
        cw += m * d
        sw += d
    return out_c, out_s, out_n, out_g

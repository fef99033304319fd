"""Packed record formats of the compressed cache (oracle; test infrastructure).

[ZB] paragraph 2: a token's record holds its quantization indices, its sign
bits and its norm. The byte layout below is this library's own choice (the
pages fix none); it is defined in include/turboquant.h and restated here
from that definition, bit by bit.

Token-major records (used for K), one row per token:
  codes : for each group g in order, a stream of m_g * d_g bits in which the
          code of channel j (0-based, within the group) occupies bits
          [m_g j, m_g j + m_g), least significant bit first; the stream is
          zero-padded to whole 32-bit words; stream bit b is bit (b mod 32)
          of word floor(b / 32).
  signs : for each group, d_g bits (bit j = sign bit of channel j), padded
          to whole words, same bit order.
  norms : float32 pairs (n_g, gamma_g) for each group (float16 pairs in the
          fp16-norm layout).

Block records (used for V): rows are grouped in aligned blocks of 32; inside
a block, token slot t = 8 o + s (octet o in 0..3, position s in 0..7).
  codes : for each group g a region of m_g * d_g words; the code of token
          slot t at channel j occupies region bits
          [8 m_g (o d_g + j) + m_g s, ... + m_g), LSB first.
  signs : for each group a region of d_g words; the sign bit of token slot
          t at channel j is region bit 8 (o d_g + j) + s.
  norms : token-major, as above.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def _words(n_bits: int) -> int:
    return (n_bits + 31) // 32


def record_words(dims: Sequence[int], mse_bits: Sequence[int], mse_only: bool = False):
    """(code words per token-major row, sign words per row, norm floats per
    row, code words per 32-token block, sign words per 32-token block).
    MSE-only records have no sign words."""
    cw = sum(_words(m * d) for d, m in zip(dims, mse_bits))
    sw = 0 if mse_only else sum(_words(d) for d in dims)
    bsw = 0 if mse_only else sum(dims)
    return cw, sw, 2 * len(dims), sum(m * d for d, m in zip(dims, mse_bits)), bsw


def record_bytes(dims: Sequence[int], mse_bits: Sequence[int], include_norms: bool = True,
                 mse_only: bool = False, norm_f16: bool = False) -> float:
    """Algorithmic bytes per token: index bits + sign bits (none when
    MSE-only) (+ two float32, or float16, norms per group)."""
    bits = sum((m if mse_only else m + 1) * d for d, m in zip(dims, mse_bits))
    return bits / 8.0 + ((4.0 if norm_f16 else 8.0) * len(dims) if include_norms else 0.0)


def _bits_to_words(bitarray: np.ndarray) -> np.ndarray:
    """[n, nbits] 0/1 array (nbits a multiple of 32) -> [n, nbits/32] uint32."""
    by = np.packbits(bitarray.astype(np.uint8), axis=1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4")


def pack_token_major(idx, bits, norm, gamma, dims, mse_bits, mse_only=False, norm_f16=False):
    """Per-token records from per-group codes/bits/norms (lists over groups).
    Returns (codes [n, Wc] uint32, signs [n, Ws] uint32, norms [n, 2G] float32
    or float16); MSE-only records have Ws = 0."""
    n = idx[0].shape[0]
    code_parts, sign_parts, norm_cols = [], [], []
    for g, (d, m) in enumerate(zip(dims, mse_bits)):
        stream = np.zeros((n, _words(m * d) * 32), dtype=np.uint8)
        for p in range(m):                                   # bit p of code j -> m j + p
            stream[:, m * np.arange(d) + p] = (idx[g] >> p) & 1
        code_parts.append(_bits_to_words(stream))
        if not mse_only:
            sstream = np.zeros((n, _words(d) * 32), dtype=np.uint8)
            sstream[:, :d] = bits[g]
            sign_parts.append(_bits_to_words(sstream))
        norm_cols += [np.asarray(norm[g], np.float32), np.asarray(gamma[g], np.float32)]
    return (np.concatenate(code_parts, axis=1), _concat_signs(sign_parts, code_parts[0].shape[0]),
            np.stack(norm_cols, axis=1).astype(np.float16 if norm_f16 else np.float32))


def _concat_signs(parts, n):
    return np.concatenate(parts, axis=1) if parts else np.zeros((n, 0), np.uint32)


def pack_block32(idx, bits, norm, gamma, dims, mse_bits, mse_only=False, norm_f16=False):
    """Block records for n rows (n a multiple of 32).
    Returns (codes [n/32, sum m_g d_g] uint32, signs [n/32, sum d_g] uint32,
    norms [n, 2G] float32); MSE-only records have no sign words."""
    n = idx[0].shape[0]
    if n % 32:
        raise ValueError("block records need a multiple of 32 rows")
    nb = n // 32
    t = np.arange(32)
    o, s = t // 8, t % 8
    code_parts, sign_parts, norm_cols = [], [], []
    for g, (d, m) in enumerate(zip(dims, mse_bits)):
        region = np.zeros((nb, 32 * m * d), dtype=np.uint8)
        sregion = np.zeros((nb, 32 * d), dtype=np.uint8)
        codes = idx[g].reshape(nb, 32, d)
        sb = bits[g].reshape(nb, 32, d)
        for j in range(d):
            unit = 8 * m * (o * d + j) + m * s               # start bit per token slot
            for p in range(m):
                region[:, unit + p] = (codes[:, :, j] >> p) & 1
            sregion[:, 8 * (o * d + j) + s] = sb[:, :, j]
        code_parts.append(_bits_to_words(region))
        if not mse_only:
            sign_parts.append(_bits_to_words(sregion))
        norm_cols += [np.asarray(norm[g], np.float32), np.asarray(gamma[g], np.float32)]
    return (np.concatenate(code_parts, axis=1), _concat_signs(sign_parts, code_parts[0].shape[0]),
            np.stack(norm_cols, axis=1).astype(np.float16 if norm_f16 else np.float32))

"""Quantize-on-append, written out step by step (oracle; test infrastructure).

[ZB] paragraph 2 and [WD] "Como o TurboQuant funciona": stage one rotates the
vector with a random orthogonal matrix and applies the per-coordinate
Lloyd-Max quantizer; stage two takes the residual of that MSE quantizer and
keeps one bit per coordinate of a Johnson-Lindenstrauss (Gaussian) sketch
of it ([WD] "2. QJL Residual"); the stored record is the indices, the sign
bits and the norm(s).

Readings used here (where the pages leave a step open; each is cited where it is used):
* the rotation is a dense d_g x d_g orthogonal matrix Pi_g given as input;
* the quantizer acts on the unit vector y = Pi_g x_g / ||x_g|| and the norm
  n_g = ||x_g|| is stored (the Beta law is a law of unit vectors);
* two norms are stored per group: n_g and gamma_g = ||r_g||, the residual
  norm that scales the sign sketch in the estimator;
* the sketch S_g is d_g x d_g with iid N(0,1) entries: one sign bit per
  channel, so b bits per channel = (b - 1) Lloyd-Max bits + 1 sign bit;
* sign bit = 1 exactly when the sketch coordinate is >= 0;
* the cell of a coordinate is the number of decision boundaries (midpoints
  of neighbouring centroids) strictly below it, i.e. the nearest centroid,
  with a coordinate exactly on a boundary taking the lower cell; a zero
  vector gets the cell just below 0 (index L/2 - 1), gamma = 0 and all
  sign bits 1;
* fractional widths (3.5, 2.5 bits) are two independent instances on a
  split of the channels: channels are reordered by ``perm`` and cut into
  consecutive groups, each with its own rotation, sketch and codebook;
* an MSE-only instance (the first of the two stages alone: [ZB] paragraph
  2 and [WD] "1. PolarQuant") keeps the same indices and norms but no sign
  bits: m_g bits per channel. Quantization itself is unchanged (the sign
  bits are still computed here, for diagnostics, and are simply not stored);
* fp16 norm storage (a layout option): n_g and gamma_g are computed exactly
  as above and rounded to float16 (nearest even) when stored; the residual
  and the sign bits use the unrounded n_g.
"""
from __future__ import annotations

from dataclasses import dataclass
from itertools import product
from typing import List

import numpy as np

from .codebook import Codebook, lloyd_max


@dataclass
class Quantizer:
    """One quantizer instance: channel order, and per group a rotation,
    a sketch and a codebook."""
    d: int
    perm: np.ndarray              # x_grouped = x[perm]
    dims: List[int]
    rotations: List[np.ndarray]   # float64 d_g x d_g
    sketches: List[np.ndarray]    # float64 d_g x d_g
    codebooks: List[Codebook]
    mse_only: bool = False        # stage one alone: records carry no sign bits
    norm_f16: bool = False        # norms stored as float16

    @staticmethod
    def from_spec(spec, mse_only: bool = False, norm_f16: bool = False) -> "Quantizer":
        """Build from a ``synth.QuantizerSpec`` (random inputs) plus this
        oracle's own Lloyd-Max codebooks."""
        dims = [g.dim for g in spec.groups]
        cbs = [lloyd_max(g.dim, g.mse_bits) for g in spec.groups]
        return Quantizer(d=spec.d, perm=np.asarray(spec.perm, dtype=np.int64), dims=dims,
                         rotations=[np.asarray(r, np.float64) for r in spec.rotations],
                         sketches=[np.asarray(s, np.float64) for s in spec.sketches],
                         codebooks=cbs, mse_only=bool(mse_only), norm_f16=bool(norm_f16))

    @property
    def offsets(self) -> List[int]:
        return [int(v) for v in np.concatenate(([0], np.cumsum(self.dims)[:-1]))]


@dataclass
class QuantizedVectors:
    """Per group g: idx[g] [n, d_g] ints, bits[g] [n, d_g] bools,
    norm[g] and gamma[g] [n] float32 (as stored), plus diagnostics:
    y[g] the unit rotated coordinates (float64), margin[g] the distance of
    each y to its nearest decision boundary, sign_margin[g] = |s| / n_g."""
    idx: List[np.ndarray]
    bits: List[np.ndarray]
    norm: List[np.ndarray]
    gamma: List[np.ndarray]
    y: List[np.ndarray]
    margin: List[np.ndarray]
    sign_margin: List[np.ndarray]


def _cell_index(y: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    # Index of the Lloyd-Max cell: the number of decision boundaries (midpoints
    # between neighbouring centroids) strictly below y. This is the nearest
    # centroid; a y lying exactly on a boundary takes the lower cell.
    return np.sum(y[..., None] > boundaries, axis=-1)


def _residual_and_signs(xg, n, idx, pi, s_mat, c):
    """Stage two for one group: dequantized MSE part, residual, its norm and
    the sign bits of its Gaussian sketch."""
    x_mse = n[:, None] * (c[idx] @ pi)          # n * Pi^T c[idx], row-vector form
    r = xg - x_mse
    gamma = np.linalg.norm(r, axis=1)
    s = r @ s_mat.T                             # S r
    bits = s >= 0.0
    return gamma, s, bits


def quantize(x: np.ndarray, qz: Quantizer) -> QuantizedVectors:
    """Quantize rows of x [n, d] (any float dtype; computed in float64)."""
    x = np.asarray(x, dtype=np.float64)
    xp = x[:, qz.perm]
    out = QuantizedVectors([], [], [], [], [], [], [])
    for off, dg, pi, sm, cb in zip(qz.offsets, qz.dims, qz.rotations, qz.sketches, qz.codebooks):
        xg = xp[:, off:off + dg]
        c = cb.centroids
        L = c.size
        n = np.linalg.norm(xg, axis=1)
        zero = n == 0.0
        safe = np.where(zero, 1.0, n)
        y = (xg @ pi.T) / safe[:, None]          # Pi x / ||x||
        idx = _cell_index(y, cb.boundaries)
        idx[zero] = L // 2 - 1
        gamma, s, bits = _residual_and_signs(xg, n, idx, pi, sm, c)
        margin = np.min(np.abs(y[..., None] - cb.boundaries), axis=-1)
        out.idx.append(idx.astype(np.int64))
        out.bits.append(bits)
        stored = np.float16 if qz.norm_f16 else np.float32
        out.norm.append(n.astype(stored).astype(np.float32))
        out.gamma.append(gamma.astype(stored).astype(np.float32))
        out.y.append(y)
        out.margin.append(margin)
        out.sign_margin.append(np.abs(s) / safe[:, None])
    return out


def legal_variants(x_row: np.ndarray, qz: Quantizer, group: int, qv: QuantizedVectors,
                   row: int, band: float):
    """All records the quantizer may legally produce for one vector and group
    when coordinates closer than ``band`` to a decision boundary may fall on
    either side of it.

    Returns a list of (idx [d_g], bits [d_g], gamma float32, sign_margin
    [d_g]) tuples; the first is the oracle's own choice. The number of
    variants is 2^k with k the number of such coordinates (k is almost
    always 0 or 1)."""
    off, dg = qz.offsets[group], qz.dims[group]
    pi, sm, cb = qz.rotations[group], qz.sketches[group], qz.codebooks[group]
    xg = np.asarray(x_row, dtype=np.float64)[qz.perm][off:off + dg][None, :]
    n = np.array([float(np.linalg.norm(xg))])
    base = qv.idx[group][row].copy()
    y = qv.y[group][row]
    amb = np.nonzero(qv.margin[group][row] < band)[0]
    options = []
    for j in amb:
        k = int(np.argmin(np.abs(y[j] - cb.boundaries)))   # boundary between cells k and k+1
        options.append((j, (k, k + 1)))
    variants = []
    for choice in product(*[o[1] for o in options]) if options else [()]:
        idx = base.copy()
        for (j, _), v in zip(options, choice):
            idx[j] = v
        gamma, s, bits = _residual_and_signs(xg, n, idx[None, :], pi, sm, cb.centroids)
        safe = n[0] if n[0] > 0 else 1.0
        variants.append((idx, bits[0], np.float32(gamma[0]), np.abs(s[0]) / safe))
    # put the oracle's own choice first
    variants.sort(key=lambda v: 0 if np.array_equal(v[0], base) else 1)
    return variants

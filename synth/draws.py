"""Primitive seeded draws (random matrices, Gaussian data, bf16 rounding)."""
from __future__ import annotations

import numpy as np


def rng_for(*entropy: int) -> np.random.Generator:
    """A PCG64 generator keyed by a tuple of non-negative integers."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-distributed d x d orthogonal matrix (float64).

    Drawn as the Q factor of a QR factorisation of an iid N(0,1) matrix,
    with the columns' signs fixed by the signs of R's diagonal so that the
    law is exactly Haar (Mezzadri, "How to generate random matrices from
    the classical compact groups", 2007).
    """
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return q


def gaussian_sketch(rng: np.random.Generator, d: int) -> np.ndarray:
    """d x d matrix of iid N(0,1) entries, drawn in float32 (returned as float32)."""
    return rng.standard_normal((d, d), dtype=np.float32)


def standard_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """iid N(0,1) float32 draws."""
    return rng.standard_normal(shape, dtype=np.float32)


def to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and return
    them as float32 values that are exactly representable in bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    nan = np.isnan(x)
    out = ((u + rounding) >> 16 << 16).astype(np.uint32)
    out = np.where(nan, np.uint32(0x7FC00000), out)
    return out.view(np.float32)


def outlier_channels(rng: np.random.Generator, d: int, k: int) -> np.ndarray:
    """k distinct channel indices in [0, d), sorted."""
    return np.sort(rng.choice(d, size=k, replace=False)).astype(np.int64)


def grouped_channel_permutation(d: int, first: np.ndarray, first_size: int) -> np.ndarray:
    """Channel order for a two-group split.

    The first group holds the channels in ``first`` followed by the lowest
    indexed remaining channels until it has ``first_size`` members (in
    increasing order); the second group holds the rest in increasing order.
    Returned as ``perm`` with the convention x_grouped = x[perm].
    """
    first = [int(c) for c in np.sort(first)]
    rest = [c for c in range(d) if c not in set(first)]
    need = first_size - len(first)
    if need < 0:
        raise ValueError("more designated channels than the first group holds")
    group_a = sorted(first + rest[:need])
    group_b = [c for c in range(d) if c not in set(group_a)]
    return np.array(group_a + group_b, dtype=np.int64)

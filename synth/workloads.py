"""Workload shapes and their seeded draw recipes.

Each workload names a cache shape and a bit width. The draws are keyed by
(seed, stream tag, indices) so every slab can be produced on its own:

* quantizer matrices: tag 1 (K) / 2 (V), then the group index and a
  sub-tag (0: rotation, 1: sketch);
* K/V data: tag 3 (K) / 4 (V), then (batch, kv head, 4096-token block);
* queries: tag 5;
* outlier channel set: tag 6;
* mixture database / queries (nearest-neighbour workload): tags 7, 8, 9.

Rotations are Haar matrices rounded to float32 (both the oracle and the
device consume the same float32 values); sketches are iid N(0,1) float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .draws import (
    rng_for, haar_orthogonal, gaussian_sketch, standard_normal, to_bf16_exact,
    outlier_channels, grouped_channel_permutation,
)

TOKEN_BLOCK = 4096  # granularity of the per-slab seeding of K/V data


@dataclass
class GroupSpec:
    dim: int          # d_g
    mse_bits: int     # m_g (Lloyd-Max bits); total bits per channel = m_g + 1


@dataclass
class QuantizerSpec:
    """Random inputs of one quantizer instance (one per K or V)."""
    d: int
    groups: List[GroupSpec]
    perm: np.ndarray                      # x_grouped = x[perm]
    rotations: List[np.ndarray]           # per group, float64 holding float32 values
    sketches: List[np.ndarray]            # per group, float32

    @property
    def n_groups(self) -> int:
        return len(self.groups)


@dataclass
class Workload:
    name: str
    seed: int
    d: int
    groups: Tuple[Tuple[int, int], ...]   # ((d_g, m_g), ...)
    batch: int
    n_q_heads: int
    n_kv_heads: int
    n_ctx: int                            # tokens attended by the decode step
    n_new: int                            # tokens quantized inside the timed step
    dtype: str                            # "f32" or "bf16"
    scale: float                          # logit scale
    logits_only: bool = False
    n_outliers: int = 0
    outlier_factor: float = 10.0
    first_group_takes_outliers: bool = False
    description: str = ""

    @property
    def capacity(self) -> int:
        return ((self.n_ctx + 31) // 32) * 32

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def _wl(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS = {
    # Tiny single head, 3 bits = 2-bit Lloyd-Max + 1-bit sign sketch; raw inner
    # products (scale 1) of 64 queries against 4096 keys.
    "tiny": _wl(name="tiny", seed=0, d=128, groups=((128, 2),), batch=1, n_q_heads=64,
                n_kv_heads=1, n_ctx=4096, n_new=4096, dtype="f32", scale=1.0,
                logits_only=True,
                description="d=128, 4096 fp32 keys, 64 fp32 queries, 3 bits, logits only"),
    # Llama-3-8B-shaped decode step: GQA 32:8, 4 bits, 4 outlier channels x10.
    "llama8b_decode": _wl(name="llama8b_decode", seed=2, d=128, groups=((128, 3),), batch=1,
                          n_q_heads=32, n_kv_heads=8, n_ctx=32768, n_new=1, dtype="bf16",
                          scale=1.0 / np.sqrt(128.0), n_outliers=4,
                          description="B=1, 32 q / 8 kv heads, d=128, N=32768, 4 bits, "
                                      "append 1 token then decode"),
    # 70B-shaped long context: GQA 64:8, 3 bits, an 8192-token prefill chunk.
    "llama70b_long": _wl(name="llama70b_long", seed=3, d=128, groups=((128, 2),), batch=4,
                         n_q_heads=64, n_kv_heads=8, n_ctx=131072, n_new=8192, dtype="bf16",
                         scale=1.0 / np.sqrt(128.0),
                         description="B=4, 64 q / 8 kv heads, d=128, N=131072, 3 bits, "
                                     "8192-token chunk quantized then decode"),
    # Mixed fractional widths: 64 || 64 channel split with 8 outlier channels.
    "mixed_3p5": _wl(name="mixed_3p5", seed=4, d=128, groups=((64, 3), (64, 2)), batch=16,
                     n_q_heads=32, n_kv_heads=8, n_ctx=32768, n_new=1, dtype="bf16",
                     scale=1.0 / np.sqrt(128.0), n_outliers=8,
                     first_group_takes_outliers=True,
                     description="B=16, 32 q / 8 kv heads, N=32768, 3.5 bits/channel "
                                 "(64 ch @ 4 bits || 64 ch @ 3 bits)"),
    "mixed_2p5": _wl(name="mixed_2p5", seed=4, d=128, groups=((64, 2), (64, 1)), batch=16,
                     n_q_heads=32, n_kv_heads=8, n_ctx=32768, n_new=1, dtype="bf16",
                     scale=1.0 / np.sqrt(128.0), n_outliers=8,
                     first_group_takes_outliers=True,
                     description="B=16, 32 q / 8 kv heads, N=32768, 2.5 bits/channel "
                                 "(64 ch @ 3 bits || 64 ch @ 2 bits)"),
    # Nearest-neighbour database: d=200 unit vectors from a Gaussian mixture, 4 bits.
    "nn_search": _wl(name="nn_search", seed=5, d=200, groups=((200, 3),), batch=1,
                     n_q_heads=1, n_kv_heads=1, n_ctx=1_000_000, n_new=1_000_000,
                     dtype="f32", scale=1.0, logits_only=True,
                     description="1e6 database vectors + 1e4 queries, d=200, "
                                 "1000-component mixture, L2-normalised, 4 bits"),
}


def workload(name: str, **overrides) -> Workload:
    """A workload by name; keyword overrides give scaled-down variants."""
    base = WORKLOADS[name]
    if not overrides:
        return base
    kw = dict(base.__dict__)
    kw.update(overrides)
    return Workload(**kw)


def _outliers(wl: Workload) -> np.ndarray:
    if wl.n_outliers == 0:
        return np.zeros(0, dtype=np.int64)
    return outlier_channels(rng_for(wl.seed, 6), wl.d, wl.n_outliers)


def draw_quantizer(wl: Workload, kind: str) -> QuantizerSpec:
    """Rotation(s), sketch(es) and channel order for the K or V quantizer."""
    tag = {"K": 1, "V": 2}[kind]
    groups = [GroupSpec(dim=g, mse_bits=m) for g, m in wl.groups]
    if len(groups) == 1:
        perm = np.arange(wl.d, dtype=np.int64)
    else:
        first = _outliers(wl) if wl.first_group_takes_outliers else np.zeros(0, np.int64)
        perm = grouped_channel_permutation(wl.d, first, groups[0].dim)
    rots, sks = [], []
    for gi, g in enumerate(groups):
        pi = haar_orthogonal(rng_for(wl.seed, tag, gi, 0), g.dim)
        rots.append(pi.astype(np.float32).astype(np.float64))
        sks.append(gaussian_sketch(rng_for(wl.seed, tag, gi, 1), g.dim))
    return QuantizerSpec(d=wl.d, groups=groups, perm=perm, rotations=rots, sketches=sks)


def draw_kv_slab(wl: Workload, kind: str, b: int, h: int, t0: int, t1: int) -> np.ndarray:
    """Tokens [t0, t1) of the K or V stream of (batch b, kv head h), float32
    values (bf16-exact when the workload is bf16). Outlier channels are
    multiplied by the workload's outlier factor."""
    tag = {"K": 3, "V": 4}[kind]
    out = np.empty((t1 - t0, wl.d), dtype=np.float32)
    blk0, blk1 = t0 // TOKEN_BLOCK, (t1 - 1) // TOKEN_BLOCK
    pos = 0
    for blk in range(blk0, blk1 + 1):
        a = standard_normal(rng_for(wl.seed, tag, b, h, blk), (TOKEN_BLOCK, wl.d))
        lo = max(t0, blk * TOKEN_BLOCK) - blk * TOKEN_BLOCK
        hi = min(t1, (blk + 1) * TOKEN_BLOCK) - blk * TOKEN_BLOCK
        out[pos:pos + hi - lo] = a[lo:hi]
        pos += hi - lo
    o = _outliers(wl)
    if o.size:
        out[:, o] *= np.float32(wl.outlier_factor)
    if wl.dtype == "bf16":
        out = to_bf16_exact(out)
    return out


def draw_queries(wl: Workload) -> np.ndarray:
    """Queries [batch, n_q_heads, d], float32 (bf16-exact when bf16)."""
    q = standard_normal(rng_for(wl.seed, 5), (wl.batch, wl.n_q_heads, wl.d))
    if wl.dtype == "bf16":
        q = to_bf16_exact(q)
    return q


def draw_mixture_vectors(wl: Workload, n: int, which: str, start: int = 0,
                         n_components: int = 1000, spread: float = 0.5) -> np.ndarray:
    """Unit vectors from a Gaussian mixture: x = mu_c + spread * eps, then
    L2-normalised. ``which`` is "db" or "query"; rows [start, start + n).
    The mixture means are shared by both sets."""
    mu = standard_normal(rng_for(wl.seed, 7), (n_components, wl.d))
    tag = {"db": 8, "query": 9}[which]
    out = np.empty((n, wl.d), dtype=np.float32)
    blk0, blk1 = start // 65536, (start + n - 1) // 65536
    pos = 0
    for blk in range(blk0, blk1 + 1):
        r = rng_for(wl.seed, tag, blk)
        comp = r.integers(0, n_components, size=65536)
        eps = standard_normal(r, (65536, wl.d))
        x = mu[comp] + np.float32(spread) * eps
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        lo = max(start, blk * 65536) - blk * 65536
        hi = min(start + n, (blk + 1) * 65536) - blk * 65536
        out[pos:pos + hi - lo] = x[lo:hi]
        pos += hi - lo
    return out

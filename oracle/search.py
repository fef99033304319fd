"""Nearest-neighbour search with the compressed codes (oracle; test
infrastructure).

[WD] "Os numeros que importam": the method also serves vector search (a
word-vector benchmark, with recall above methods built on large
codebooks). A query is compared with every database vector through the
same inner-product estimator that gives the attention logits, and the best
matches are kept.

Readings used here (where the pages leave a step open; each is cited where it is used):
* score(q, i) = <q, x~_i>, with x~_i the dequantized database vector
  (``estimate.dequantize``; no scale factor);
* the k best of a query are the k largest scores in decreasing order, equal
  scores going to the lower database index;
* the exact neighbours are the same selection over the true inner products
  <q, x_i>, and recall@k is the fraction of a query's exact k neighbours
  that the search returns, averaged over queries.
"""
from __future__ import annotations

import numpy as np

from .estimate import dequantize, estimate_logits
from .quantize import Quantizer


def top_k(scores: np.ndarray, k: int):
    """Rows of ``scores`` [n_q, n] -> (indices [n_q, k], scores [n_q, k]):
    the k largest entries of each row in decreasing order, ties to the lower
    column index."""
    scores = np.asarray(scores, dtype=np.float64)
    n_q, n = scores.shape
    k_eff = min(k, n)
    idx = np.empty((n_q, k_eff), dtype=np.int64)
    cols = np.arange(n)
    for r in range(n_q):
        # primary key: -score (ascending), secondary: column index
        order = np.lexsort((cols, -scores[r]))
        idx[r] = order[:k_eff]
    return idx, np.take_along_axis(scores, idx, axis=1)


def estimated_scores(q: np.ndarray, idx, bits, norm, gamma, qz: Quantizer, chunk: int = 65536) -> np.ndarray:
    """<q_j, x~_i> for queries [n_q, d] and the database given by its codes,
    sign bits and stored norms (per-group lists, as in QuantizedVectors);
    the database is dequantized ``chunk`` rows at a time."""
    q = np.asarray(q, dtype=np.float64)
    n_db = idx[0].shape[0]
    out = np.empty((q.shape[0], n_db), dtype=np.float64)
    for s in range(0, n_db, chunk):
        e = min(n_db, s + chunk)
        xt = dequantize([a[s:e] for a in idx], [a[s:e] for a in bits], [a[s:e] for a in norm],
                        [a[s:e] for a in gamma], qz)
        out[:, s:e] = estimate_logits(q, xt, 1.0)
    return out


def search(q: np.ndarray, qv, qz: Quantizer, k: int):
    """(indices, scores) of the k best database vectors per query under the
    estimator; ``qv`` is the database's QuantizedVectors."""
    return top_k(estimated_scores(q, qv.idx, qv.bits, qv.norm, qv.gamma, qz), k)


def exact_search(q: np.ndarray, x: np.ndarray, k: int):
    """(indices, inner products) of the k best database vectors per query
    under the true inner product."""
    return top_k(np.asarray(q, np.float64) @ np.asarray(x, np.float64).T, k)


def recall_at_k(found: np.ndarray, exact: np.ndarray) -> float:
    """Mean over queries of |found_j & exact_j| / k."""
    found = np.asarray(found)
    exact = np.asarray(exact)
    k = exact.shape[1]
    hits = [len(set(f.tolist()) & set(e.tolist())) for f, e in zip(found, exact)]
    return float(np.mean(hits)) / k

"""Pins of the oracle's nearest-neighbour search.

top_k is checked against an exhaustive rank count written with loops on
inputs full of ties; exact_search against planted neighbours and
loop-computed inner products; the estimated scores against explicit
dequantization and against the true inner products of planted neighbours
(a vector is its own best match under the estimator); recall@k on cases
with a closed-form value.
"""
import numpy as np
import pytest

import oracle
import synth


def _rank_select(scores, k):
    # rank of entry j = number of entries that beat it (larger score, or the
    # same score at a lower index); the k best are the ranks 0 .. k - 1
    n = len(scores)
    rank = []
    for j in range(n):
        r = 0
        for i in range(n):
            if scores[i] > scores[j] or (scores[i] == scores[j] and i < j):
                r += 1
        rank.append(r)
    out = [None] * min(k, n)
    for j, r in enumerate(rank):
        if r < len(out):
            out[r] = j
    return out


def test_top_k_against_rank_count_with_ties():
    rng = np.random.default_rng(4)
    s = rng.integers(0, 4, size=(6, 40)).astype(np.float64)  # many ties
    for k in (1, 3, 10, 40):
        idx, val = oracle.top_k(s, k)
        for r in range(s.shape[0]):
            assert idx[r].tolist() == _rank_select(s[r].tolist(), k)
            assert np.array_equal(val[r], s[r][idx[r]])


def test_top_k_shorter_than_k():
    idx, val = oracle.top_k(np.array([[0.5, 2.0, 2.0]]), 10)
    assert idx.tolist() == [[1, 2, 0]] and val.tolist() == [[2.0, 2.0, 0.5]]


def test_exact_search_planted_neighbours():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 24))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    planted = np.array([7, 123, 299])
    q = x[planted] + 1e-3 * rng.standard_normal((3, 24))
    idx, val = oracle.exact_search(q, x, 5)
    assert idx[:, 0].tolist() == planted.tolist()
    for r in range(3):
        for c in range(5):
            ip = sum(q[r, t] * x[idx[r, c], t] for t in range(24))
            assert abs(val[r, c] - ip) < 1e-12


def _quantizer(d, m, seed):
    spec = synth.QuantizerSpec(
        d=d, groups=[synth.GroupSpec(dim=d, mse_bits=m)], perm=np.arange(d),
        rotations=[synth.haar_orthogonal(synth.rng_for(seed, 0, 0), d).astype(np.float32).astype(np.float64)],
        sketches=[synth.gaussian_sketch(synth.rng_for(seed, 0, 1), d)])
    return oracle.Quantizer.from_spec(spec)


def test_estimated_scores_equal_explicit_dequantization_in_any_chunking():
    qz = _quantizer(40, 3, 8)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((90, 40))
    q = rng.standard_normal((4, 40))
    qv = oracle.quantize(x, qz)
    xt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)
    ref = np.array([[float(np.dot(q[r], xt[i])) for i in range(90)] for r in range(4)])
    for chunk in (7, 90, 1000):
        got = oracle.estimated_scores(q, qv.idx, qv.bits, qv.norm, qv.gamma, qz, chunk=chunk)
        assert np.max(np.abs(got - ref)) < 1e-12


def test_every_vector_is_its_own_best_match():
    # unit vectors in d = 64 at 4 bits: the estimated self inner product is
    # close to 1 while other vectors score about N(0, 1/64)
    qz = _quantizer(64, 3, 9)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((400, 64))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    qv = oracle.quantize(x, qz)
    idx, val = oracle.search(x[:50], qv, qz, 3)
    assert idx[:, 0].tolist() == list(range(50))
    assert np.all(np.abs(val[:, 0] - 1.0) < 0.15)


def test_estimated_scores_track_true_inner_products():
    # unbiased estimator: over many database vectors the error has mean ~0
    qz = _quantizer(64, 3, 10)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3000, 64))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    q = x[:1] * 0.9 + 0.1 * rng.standard_normal((1, 64))
    qv = oracle.quantize(x, qz)
    est = oracle.estimated_scores(q, qv.idx, qv.bits, qv.norm, qv.gamma, qz)[0]
    err = est - (x @ q[0])
    assert abs(err.mean()) < 4 * err.std() / np.sqrt(err.size)
    assert err.std() < 0.05


@pytest.mark.parametrize("found,exact,expect", [
    ([[1, 2, 3]], [[3, 2, 1]], 1.0),
    ([[4, 5, 6]], [[1, 2, 3]], 0.0),
    ([[1, 2, 9, 8]], [[1, 2, 3, 4]], 0.5),
    ([[1, 2], [7, 8]], [[1, 3], [7, 8]], 0.75),
])
def test_recall_closed_forms(found, exact, expect):
    assert oracle.recall_at_k(np.array(found), np.array(exact)) == expect

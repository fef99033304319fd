"""GPU parity of tq_search (nearest-neighbour search with the compressed
codes) against the CPU oracle, through the C ABI.

The database records are the oracle's own quantization of the synthetic
vectors, packed by the oracle's packer and uploaded, so the device and the
oracle score the identical records. Equal-score order aside, the k best of
a query are unique; floating point can swap two database vectors whose
oracle scores are closer than the score tolerance. So the check is:
  * returned scores match the oracle's scores of the returned rows within
    TOL = 2e-3 of the query's largest |score| (the logit tolerance),
  * the returned rows are distinct and in decreasing score order,
  * every returned row's oracle score is at least the oracle's k-th best
    minus 2 TOL, and every oracle top-k row whose score beats the oracle's
    (k+1)-th best by more than 2 TOL is returned.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def tq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_vector_rotation_amd as m
    m.lib()
    return m


def _db(tq, spec, x, n_rows=None, chunk=100_000, norm_f16=False):
    """Oracle-quantized database uploaded as a token-major cache; returns the
    device cache and the oracle's (idx, bits, norm, gamma), quantized and
    packed in chunks."""
    oq, dq = gc.quantizers(spec, norm_f16=norm_f16)
    n = x.shape[0]
    n_rows = n_rows or n
    dims = [g.dim for g in spec.groups]
    bits = [g.mse_bits for g in spec.groups]
    cw, sw, nf, _, _ = oracle.record_words(dims, bits)
    codes = np.zeros((n_rows, cw), np.uint32)
    signs = np.zeros((n_rows, sw), np.uint32)
    norms = np.zeros((n_rows, nf), np.float16 if norm_f16 else np.float32)
    idx, bts, nrm, gam = [], [], [], []
    for s in range(0, n, chunk):
        qv = oracle.quantize(x[s:s + chunk].astype(np.float64), oq)
        c, sg, nm = oracle.pack_token_major(qv.idx, qv.bits, qv.norm, qv.gamma, dims, bits, False, norm_f16)
        codes[s:s + chunk], signs[s:s + chunk], norms[s:s + chunk] = c, sg, nm
        idx.append(qv.idx[0].astype(np.int8))
        bts.append(qv.bits[0])
        nrm.append(qv.norm[0])
        gam.append(qv.gamma[0])
    cache = gc.to_device_cache(dq, tq.TQ_TOKEN_MAJOR, n_rows, (codes.ravel(), signs.ravel(), norms.ravel()))
    rec = ([np.concatenate(idx)], [np.concatenate(bts)], [np.concatenate(nrm)], [np.concatenate(gam)])
    return oq, dq, cache, rec


def _search(tq, dq, cache, n_db, q, k, bf16=False):
    import torch
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()
    if bf16:
        qt = qt.to(torch.bfloat16)
    oi, osc = tq.tq_search(dq, cache, n_db, qt, k)
    torch.cuda.synchronize()
    return oi.cpu().numpy(), osc.cpu().numpy().astype(np.float64)


def _check(got_idx, got_score, ref_scores, k):
    """ref_scores [n_q, n_db] oracle estimated scores."""
    n_q, n_db = ref_scores.shape
    kk = min(k, n_db)
    for r in range(n_q):
        s = ref_scores[r]
        tol = TOL * np.max(np.abs(s))
        gi = got_idx[r]
        assert np.all(gi[kk:] == -1) and np.all(np.isneginf(got_score[r][kk:]))
        gi, gs = gi[:kk], got_score[r][:kk]
        assert np.all(gi >= 0) and len(set(gi.tolist())) == kk, (r, gi)
        assert np.all(np.abs(gs - s[gi]) <= tol), (r, np.max(np.abs(gs - s[gi])), tol)
        assert np.all(np.diff(gs) <= 0)
        order = np.lexsort((np.arange(n_db), -s))
        kth = s[order[kk - 1]]
        assert np.all(s[gi] >= kth - 2 * tol), r
        nxt = s[order[kk]] if n_db > kk else -np.inf
        must = order[:kk][s[order[:kk]] > nxt + 2 * tol]
        assert set(must.tolist()) <= set(gi.tolist()), r


CASES = [
    # d, m, n_db, n_q, k, bf16 queries
    (200, 3, 3000, 70, 10, False),
    (200, 3, 1000, 1, 10, True),
    (200, 3, 37, 5, 10, False),     # 3 tiles, ragged
    (200, 3, 5, 3, 10, False),      # fewer rows than k
    (200, 2, 2500, 40, 7, False),
    (200, 1, 2000, 33, 10, False),
    (128, 3, 4000, 64, 10, False),
    (128, 2, 999, 20, 1, True),
]


@pytest.mark.parametrize("d,m,n_db,n_q,k,bf16", CASES)
def test_search_matches_oracle(tq, d, m, n_db, n_q, k, bf16):
    wl = synth.workload("nn_search", d=d, groups=((d, m),))
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_mixture_vectors(wl, n_db, "db")
    q = synth.draw_mixture_vectors(wl, n_q, "query")
    if bf16:
        q = synth.to_bf16_exact(q)
    oq, dq, cache, rec = _db(tq, spec, x)
    gi, gs = _search(tq, dq, cache, n_db, q, k, bf16)
    ref = oracle.estimated_scores(q, *rec, oq)
    _check(gi, gs, ref, k)


def test_duplicates_go_to_the_lower_index(tq):
    # the database holds each of 40 vectors five times; the query is one of
    # them: its five copies score identically and come back in index order
    wl = synth.workload("nn_search")
    spec = synth.draw_quantizer(wl, "K")
    base = synth.draw_mixture_vectors(wl, 40, "db")
    x = np.concatenate([base] * 5)
    oq, dq, cache, rec = _db(tq, spec, x)
    gi, gs = _search(tq, dq, cache, 200, base[[3, 17]], 5)
    assert gi[0].tolist() == [3, 43, 83, 123, 163]
    assert gi[1].tolist() == [17, 57, 97, 137, 177]
    assert np.all(gs[:, 0] == gs[:, 4])


def test_full_size_sampled_queries(tq):
    # the nearest-neighbour workload at full size: 1,000,000 database vectors
    # (d = 200, 4 bits), 10,000 queries in one call; 12 sampled queries are
    # checked against the oracle over the whole database, and their recall@10
    # against exact brute force is reported
    wl = synth.workload("nn_search")
    spec = synth.draw_quantizer(wl, "K")
    n_db, n_q = 1_000_000, 10_000
    x = synth.draw_mixture_vectors(wl, n_db, "db")
    q = synth.draw_mixture_vectors(wl, n_q, "query")
    oq, dq, cache, rec = _db(tq, spec, x)
    gi, gs = _search(tq, dq, cache, n_db, q, 10)
    sample = np.linspace(0, n_q - 1, 12).astype(int)
    ref = oracle.estimated_scores(q[sample], *rec, oq)
    _check(gi[sample], gs[sample], ref, 10)
    ex, _ = oracle.exact_search(q[sample], x, 10)
    # the device's recall equals the oracle estimator's own recall on the same
    # queries (the top-k check above leaves only ties free: allow two swaps)
    oi = np.argsort(-ref, axis=1, kind="stable")[:, :10]
    r_dev, r_orc = oracle.recall_at_k(gi[sample], ex), oracle.recall_at_k(oi, ex)
    print("recall@10 on the sampled queries: device", r_dev, "oracle estimator", r_orc)
    assert abs(r_dev - r_orc) <= 2 / (len(sample) * 10)


test_full_size_sampled_queries = pytest.mark.timeout(900)(test_full_size_sampled_queries)


@pytest.mark.parametrize("d,m", [(200, 3), (128, 2)])
def test_search_fp16_norms(tq, d, m):
    # a database whose records store the norms as float16
    wl = synth.workload("nn_search", d=d, groups=((d, m),))
    spec = synth.draw_quantizer(wl, "K")
    x = synth.draw_mixture_vectors(wl, 2500, "db")
    q = synth.draw_mixture_vectors(wl, 30, "query")
    oq, dq, cache, rec = _db(tq, spec, x, norm_f16=True)
    gi, gs = _search(tq, dq, cache, 2500, q, 10)
    _check(gi, gs, oracle.estimated_scores(q, *rec, oq), 10)

"""Pins of the oracle's quantizer and estimator.

Pinned by invariants of orthogonal matrices, the law of a coordinate of a
uniform unit vector (Kolmogorov-Smirnov), brute force at tiny sizes,
vectors built with prescribed rotated coordinates, the Gaussian sign
identity E[<s,q> sign<s,r>] = sqrt(2/pi) <q, r/|r|> (unbiasedness and
closed-form variance over many sketch draws), and algebraic identities of
attention (explicit softmax vs a split online softmax, GQA vs repeated heads).
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
import synth


def _quantizer(d=32, groups=((32, 2),), seed=7, perm=None, exact=False):
    rots, sks, gspecs = [], [], []
    for gi, (dg, m) in enumerate(groups):
        pi = synth.haar_orthogonal(synth.rng_for(seed, gi, 0), dg)
        if not exact:
            pi = pi.astype(np.float32).astype(np.float64)
        rots.append(pi)
        sks.append(synth.gaussian_sketch(synth.rng_for(seed, gi, 1), dg))
        gspecs.append(synth.GroupSpec(dim=dg, mse_bits=m))
    if perm is None:
        perm = np.arange(d)
    spec = synth.QuantizerSpec(d=d, groups=gspecs, perm=np.asarray(perm), rotations=rots, sketches=sks)
    return oracle.Quantizer.from_spec(spec)


def test_rotation_preserves_norm_fp32_haar():
    wl = synth.workload("tiny")
    qz = oracle.Quantizer.from_spec(synth.draw_quantizer(wl, "K"))
    pi = qz.rotations[0]
    assert np.max(np.abs(pi.T @ pi - np.eye(128))) < 1e-6
    x = synth.draw_kv_slab(wl, "K", 0, 0, 0, 512).astype(np.float64)
    qv = oracle.quantize(x, qz)
    # stored norm is the input norm; the unit rotated vector has norm 1 to fp32-matrix precision
    ref = np.array([math.sqrt(math.fsum(v * v for v in row)) for row in x])
    assert np.max(np.abs(qv.norm[0] / ref - 1)) < 1e-7
    assert np.max(np.abs(np.linalg.norm(qv.y[0], axis=1) - 1)) < 1e-6


@pytest.mark.parametrize("case", ["spike", "gaussian"])
def test_rotated_coordinates_follow_beta_law(case):
    d = 64
    cb_dummy = ((d, 2),)
    if case == "spike":
        # a fixed adversarial vector (all mass on 4 channels, x10) under 2000 Haar draws
        x = np.zeros(d)
        x[[3, 17, 40, 63]] = [10.0, -10.0, 10.0, 10.0]
        ys = []
        for s in range(2000):
            qz = _quantizer(d, cb_dummy, seed=1000 + s, exact=True)
            ys.append(oracle.quantize(x[None, :], qz).y[0][0, [0, 21, 50]])
        sample = np.concatenate(ys)
    else:
        qz = _quantizer(d, cb_dummy, seed=5, exact=True)
        x = np.random.default_rng(3).standard_normal((3000, d))
        sample = oracle.quantize(x, qz).y[0][:, [1, 33, 60]].ravel()
    p = stats.kstest(sample, lambda v: oracle.coordinate_cdf(v, d)).pvalue
    assert p > 1e-3
    n = sample.size
    m2, m4 = np.mean(sample ** 2), np.mean(sample ** 4)
    sd2 = math.sqrt((3 / (d * (d + 2)) - 1 / d ** 2) / n)
    assert abs(m2 - 1 / d) < 5 * sd2
    # the law is a Beta law of (y+1)/2 with both shapes (d-1)/2
    p2 = stats.kstest((sample + 1) / 2, stats.beta((d - 1) / 2, (d - 1) / 2).cdf).pvalue
    assert p2 > 1e-3


def test_nearest_centroid_brute_force_equals_boundary_count():
    d = 8
    for m in (1, 2, 3, 4):
        qz = _quantizer(d, ((d, m),), seed=11)
        x = np.random.default_rng(m).standard_normal((4000, d))
        qv = oracle.quantize(x, qz)
        c = qz.codebooks[0].centroids
        y = qv.y[0]
        brute = np.array([[min(range(c.size), key=lambda k: (abs(v - c[k]), k)) for v in row]
                          for row in y[:300]])
        assert np.array_equal(brute, qv.idx[0][:300])
        count = np.searchsorted(qz.codebooks[0].boundaries, y, side="left")
        assert np.array_equal(count, qv.idx[0])


def test_prescribed_rotated_coordinates():
    # x = n Pi^T u for a unit vector u: the codes are the cells of u's entries
    # (no matrix product involved), gamma = n ||u - c[idx]||, and the MSE part of
    # <q, x~> equals n <Pi q, c[idx]>. Pins the Pi versus Pi^T convention.
    d = 16
    qz = _quantizer(d, ((d, 3),), seed=21, exact=True)
    pi = qz.rotations[0]
    c, t = qz.codebooks[0].centroids, qz.codebooks[0].boundaries
    rng = np.random.default_rng(8)
    for _ in range(20):
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        n = 3.7
        x = n * (pi.T @ u)
        qv = oracle.quantize(x[None, :], qz)
        cells = np.array([sum(1 for tk in t if uj > tk) for uj in u])
        assert np.array_equal(qv.idx[0][0], cells)
        assert abs(qv.gamma[0][0] - n * np.linalg.norm(u - c[cells])) < 1e-5
        q = rng.standard_normal(d)
        mse_only = oracle.dequantize(qv.idx, [np.ones((1, d), bool)], qv.norm, [np.zeros(1)], qz)
        assert abs(q @ mse_only[0] - n * (pi @ q) @ c[cells]) < 1e-5


def test_zero_vector():
    d = 16
    for m in (1, 2, 3):
        qz = _quantizer(d, ((d, m),), seed=2)
        qv = oracle.quantize(np.zeros((1, d)), qz)
        assert np.all(qv.idx[0] == 2 ** m // 2 - 1)
        assert qv.gamma[0][0] == 0 and qv.norm[0][0] == 0
        assert np.all(qv.bits[0])
        back = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)
        assert np.all(back == 0)


def test_boundary_goes_to_lower_cell():
    # A rotated coordinate lying exactly on a decision boundary takes the lower
    # cell: build x with Pi = I so that y_0 equals t_k bit for bit.
    d = 4
    for m in (2, 3):
        cb = oracle.lloyd_max(d, m)
        qz = oracle.Quantizer(d=d, perm=np.arange(d), dims=[d], rotations=[np.eye(d)],
                              sketches=[np.eye(d)], codebooks=[cb])
        for k, t in enumerate(cb.boundaries):
            rest = math.sqrt(1 - t * t)
            x = np.array([t, rest, 0.0, 0.0])
            qv = oracle.quantize(x[None, :], qz)
            if qv.y[0][0, 0] == t:                  # exact on the boundary
                assert qv.idx[0][0, 0] == k
            nudged = np.nextafter(t, 2.0) * np.array([1.0, 0, 0, 0]) + np.array([0, rest, 0, 0])
            qv2 = oracle.quantize(nudged[None, :], qz)
            if qv2.y[0][0, 0] > t:
                assert qv2.idx[0][0, 0] == k + 1


def _qjl_draws(x, q, d, m, n_draws, seed0):
    """Estimator <q, x~> over independent sketch draws (rotation fixed)."""
    pi = synth.haar_orthogonal(synth.rng_for(99, 0, 0), d)
    cbs = [oracle.lloyd_max(d, m)]
    est = np.empty(n_draws)
    gam = None
    for s in range(n_draws):
        sk = np.random.default_rng(seed0 + s).standard_normal((d, d))
        qz = oracle.Quantizer(d=d, perm=np.arange(d), dims=[d], rotations=[pi], sketches=[sk],
                              codebooks=cbs)
        qv = oracle.quantize(x[None, :], qz)
        xt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)[0]
        est[s] = q @ xt
        r = x - qv.norm[0][0] * (cbs[0].centroids[qv.idx[0][0]] @ pi)
        gam = r
    return est, gam


def test_qjl_estimator_unbiased_with_closed_form_variance():
    d, m = 16, 2
    rng = np.random.default_rng(4)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    est, r = _qjl_draws(x, q, d, m, 20000, 10_000)
    # stored gamma is float32; the residual itself does not depend on the sketch
    var = (math.pi / (2 * d)) * (r @ r) * (q @ q) - (q @ r) ** 2 / d
    z = (est.mean() - q @ x) / math.sqrt(var / est.size)
    assert abs(z) < 5
    assert abs(est.var(ddof=1) / var - 1) < 0.05


def test_qjl_wrong_constant_would_be_caught():
    # The same statistic with alpha = sqrt(2/pi)/d (a plausible slip) is biased
    # by more than 5 standard errors: the unbiasedness test has the power to see it.
    d, m = 16, 2
    rng = np.random.default_rng(4)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    est, r = _qjl_draws(x, q, d, m, 20000, 10_000)
    mse_part = est.mean() - q @ r            # estimator mean of the MSE part + QJL part
    qjl_mean = est.mean() - (q @ x - q @ r)
    wrong = (q @ x - q @ r) + qjl_mean * (2 / math.pi)
    var = (math.pi / (2 * d)) * (r @ r) * (q @ q) - (q @ r) ** 2 / d
    # the seeded draw has a residual inner product far from zero (the slip's
    # bias is (2/pi - 1) <q, r>), so the comparison below has a signal to see
    assert abs(q @ r) > 0.1
    assert abs(wrong - q @ x) / math.sqrt(var / est.size) > 5


def test_grouped_vector_unbiased_through_permutation():
    # Two groups of different widths behind a channel permutation: averaged over
    # sketch draws the dequantized vector is the input, channel by channel.
    d = 24
    perm = np.random.default_rng(0).permutation(d)
    x = np.random.default_rng(1).standard_normal(d) * np.linspace(0.5, 3, d)
    acc, acc2, n = np.zeros(d), np.zeros(d), 4000
    base = _quantizer(d, ((16, 2), (8, 1)), seed=3, perm=perm, exact=True)
    for s in range(n):
        r = np.random.default_rng(50_000 + s)
        qz = oracle.Quantizer(d=d, perm=base.perm, dims=base.dims, rotations=base.rotations,
                              sketches=[r.standard_normal((16, 16)), r.standard_normal((8, 8))],
                              codebooks=base.codebooks)
        qv = oracle.quantize(x[None, :], qz)
        xt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)[0]
        acc += xt
        acc2 += xt * xt
    mean = acc / n
    se = np.sqrt((acc2 / n - mean ** 2) / n)
    assert np.all(np.abs(mean - x) < 5 * se)


def test_factored_estimator_identity():
    # Logit = sum_g n_g <Pi_g q_g, c[idx]> + alpha_g gamma_g <S_g q_g, z>
    # (the form a kernel evaluates) equals <q, x~> from explicit dequantization.
    d = 8
    perm = np.array([3, 0, 6, 1, 7, 2, 5, 4])
    qz = _quantizer(d, ((4, 2), (4, 3)), seed=17, perm=perm)
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((16, d))
    qs = rng.standard_normal((4, d))
    qv = oracle.quantize(keys, qz)
    kt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)
    explicit = oracle.estimate_logits(qs, kt, 0.5)
    fact = np.zeros_like(explicit)
    qp = qs[:, perm]
    for g, (off, dg) in enumerate(zip(qz.offsets, qz.dims)):
        qg = qp[:, off:off + dg]
        qrot = qg @ qz.rotations[g].T
        qsk = qg @ qz.sketches[g].T
        c = qz.codebooks[g].centroids[qv.idx[g]]
        z = np.where(qv.bits[g], 1.0, -1.0)
        alpha = math.sqrt(math.pi / 2) / dg
        fact += qrot @ (c * qv.norm[g][:, None].astype(np.float64)).T
        fact += alpha * (qsk @ (z * qv.gamma[g][:, None].astype(np.float64)).T)
    assert np.max(np.abs(0.5 * fact - explicit)) < 1e-12


def test_grouped_equals_separate_instances():
    d = 16
    perm = np.random.default_rng(9).permutation(d)
    qz = _quantizer(d, ((8, 2), (8, 3)), seed=31, perm=perm)
    x = np.random.default_rng(3).standard_normal((50, d))
    qv = oracle.quantize(x, qz)
    for g in range(2):
        single = oracle.Quantizer(d=8, perm=np.arange(8), dims=[8], rotations=[qz.rotations[g]],
                                  sketches=[qz.sketches[g]], codebooks=[qz.codebooks[g]])
        sub = x[:, perm][:, 8 * g:8 * g + 8]
        sv = oracle.quantize(sub, single)
        assert np.array_equal(sv.idx[0], qv.idx[g]) and np.array_equal(sv.bits[0], qv.bits[g])
        assert np.array_equal(sv.norm[0], qv.norm[g]) and np.array_equal(sv.gamma[0], qv.gamma[g])


def _online_split(logits, v, n_split):
    """Flash-decoding recurrence: per split a running max, sum and weighted
    accumulator; then a log-sum-exp merge of the splits."""
    parts = []
    for chunk in np.array_split(np.arange(logits.size), n_split):
        m, l, acc = -np.inf, 0.0, np.zeros(v.shape[1])
        for i in chunk:
            m_new = max(m, logits[i])
            corr = math.exp(m - m_new) if m != -np.inf else 0.0
            p = math.exp(logits[i] - m_new)
            l, acc, m = l * corr + p, acc * corr + p * v[i], m_new
        parts.append((m, l, acc))
    mm = max(p[0] for p in parts)
    L = sum(p[1] * math.exp(p[0] - mm) for p in parts)
    A = sum(p[2] * math.exp(p[0] - mm) for p in parts)
    return A / L


def test_attention_decode_special_cases():
    rng = np.random.default_rng(5)
    hkv, g, n, d = 2, 3, 40, 8
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    q = rng.standard_normal((hkv * g, d))
    logits, out = oracle.attention_decode(q, k, v, 0.3)
    for h in range(hkv * g):
        assert np.allclose(_online_split(logits[h], v[h // g], 5), out[h], atol=1e-12)
    # GQA equals MHA with every KV head repeated G times
    _, out_mha = oracle.attention_decode(q, np.repeat(k, g, axis=0), np.repeat(v, g, axis=0), 0.3)
    assert np.allclose(out, out_mha, atol=1e-14)
    # one token: the output is that token's value
    _, o1 = oracle.attention_decode(q, k[:, :1], v[:, :1], 0.3)
    assert np.allclose(o1, np.repeat(v[:, 0], g, axis=0), atol=1e-14)
    # zero query: uniform weights, output is the mean value
    _, o0 = oracle.attention_decode(np.zeros_like(q), k, v, 0.3)
    assert np.allclose(o0, np.repeat(v.mean(axis=1), g, axis=0), atol=1e-14)
    # softmax invariance to a constant shift and sum to one
    s = oracle.softmax(logits)
    assert np.allclose(s.sum(axis=1), 1) and np.allclose(oracle.softmax(logits + 100), s)


def test_attention_prefill_causal_chunk():
    # a chunk of T query tokens: T = 1 is the decode step; a token's output
    # ignores every later token (change them and it stays); the last token
    # sees the whole context; the first sees the prefix and itself; brute
    # force on a tiny case with explicit exponentials
    rng = np.random.default_rng(6)
    hkv, g, n, d, T = 2, 2, 12, 4, 5
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    q = rng.standard_normal((T, hkv * g, d))
    lg1, o1 = oracle.attention_prefill(q[-1:], k, v, 0.7)
    lgd, od = oracle.attention_decode(q[-1], k, v, 0.7)
    assert np.allclose(o1[0], od, atol=1e-14) and np.allclose(lg1[:, 0], lgd, atol=1e-14)
    lg, out = oracle.attention_prefill(q, k, v, 0.7)
    for i in range(T):
        lim = n - T + i + 1
        assert np.all(np.isneginf(lg[:, i, lim:])) and np.all(np.isfinite(lg[:, i, :lim]))
        k2, v2 = k.copy(), v.copy()
        k2[:, lim:] = rng.standard_normal(k2[:, lim:].shape)
        v2[:, lim:] = 1e3
        _, out2 = oracle.attention_prefill(q, k2, v2, 0.7)
        assert np.allclose(out2[i], out[i], atol=1e-12)
    for i in range(T):
        for h in range(hkv * g):
            lim = n - T + i + 1
            w = [math.exp(0.7 * sum(q[i, h, e] * k[h // g, t, e] for e in range(d))) for t in range(lim)]
            ref = [sum(w[t] * v[h // g, t, e] for t in range(lim)) / sum(w) for e in range(d)]
            assert np.allclose(out[i, h], ref, atol=1e-12)


def test_attention_prefill_tokens_without_keys():
    # a chunk longer than the sequence: the first T - n tokens see no key,
    # keep -inf logits and get the empty sum (zero); the others equal the
    # decode step over their own visible prefix
    rng = np.random.default_rng(8)
    hkv, g, n, d, T = 1, 3, 3, 4, 5
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    q = rng.standard_normal((T, hkv * g, d))
    lg, out = oracle.attention_prefill(q, k, v, 0.5)
    for i in range(T):
        lim = n - T + i + 1
        if lim <= 0:
            assert np.all(out[i] == 0.0) and np.all(np.isneginf(lg[:, i]))
        else:
            lgd, od = oracle.attention_decode(q[i], k[:, :lim], v[:, :lim], 0.5)
            assert np.allclose(out[i], od, atol=1e-14) and np.allclose(lg[:, i, :lim], lgd, atol=1e-14)
            assert np.all(np.isneginf(lg[:, i, lim:]))


def test_legal_variants_cover_near_boundary_choices():
    d = 16
    qz = _quantizer(d, ((d, 2),), seed=41)
    x = np.random.default_rng(0).standard_normal((200, d))
    qv = oracle.quantize(x, qz)
    row = int(np.argmin(qv.margin[0].min(axis=1)))
    band = float(qv.margin[0][row].min()) * 1.0001
    vars_ = oracle.legal_variants(x[row], qz, 0, qv, row, band)
    assert len(vars_) == 2
    assert np.array_equal(vars_[0][0], qv.idx[0][row]) and np.array_equal(vars_[0][1], qv.bits[0][row])
    diff = np.nonzero(vars_[0][0] != vars_[1][0])[0]
    assert diff.size == 1 and abs(int(vars_[0][0][diff[0]]) - int(vars_[1][0][diff[0]])) == 1

"""Pins of the oracle's MSE-only variant (stage one alone, no sign bits).

* the reconstruction lies on the rotated codebook grid and its distance to
  the input is the stored residual norm gamma;
* over uniformly distributed directions the mean of <x~, x> / |x|^2 is
  1 - D, with D the codebook's mean squared error per unit vector: at one
  bit D has the closed form 1 - d c^2 with c = E|y_1| under the coordinate
  law; at three bits D is integrated numerically from the coordinate
  density written out here (independent of the oracle's codebook module);
  the mean of |x~|^2 / |x|^2 is the same 1 - D (centroid condition), while
  the two-stage estimate of the same vectors is unbiased;
* the record sizes and packed words without sign words.
"""
import math

import numpy as np
import pytest
from scipy import integrate

import oracle
import synth
from tests import recfmt


def _quantizer(d, m, seed, mse_only=True):
    pi = synth.haar_orthogonal(synth.rng_for(seed, 0, 0), d)
    sk = synth.gaussian_sketch(synth.rng_for(seed, 0, 1), d)
    spec = synth.QuantizerSpec(d=d, groups=[synth.GroupSpec(dim=d, mse_bits=m)], perm=np.arange(d),
                               rotations=[pi], sketches=[sk])
    return oracle.Quantizer.from_spec(spec, mse_only=mse_only)


def _unit(n, d, seed):
    x = np.random.default_rng(seed).standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _density(t, d):
    # density of one coordinate of a uniform unit vector in R^d
    lg = math.lgamma(d / 2) - math.lgamma((d - 1) / 2) - 0.5 * math.log(math.pi)
    return math.exp(lg) * (1 - t * t) ** ((d - 3) / 2)


def test_reconstruction_on_grid_and_residual_norm():
    d, m = 24, 2
    qz = _quantizer(d, m, 3)
    x = np.random.default_rng(1).standard_normal((50, d)) * 3.0
    qv = oracle.quantize(x, qz)
    xt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)
    n = qv.norm[0].astype(np.float64)
    c = qz.codebooks[0].centroids
    # rotating the reconstruction back gives n c[idx] exactly (up to rounding)
    assert np.max(np.abs(xt @ qz.rotations[0].T - n[:, None] * c[qv.idx[0]])) < 1e-12 * 10
    # the stored gamma is |x - x~| (float32)
    err = np.linalg.norm(x - xt, axis=1)
    assert np.all(np.abs(err - qv.gamma[0]) <= 1e-6 * n)


def test_one_bit_bias_closed_form():
    d = 16
    qz = _quantizer(d, 1, 5)
    # one-bit centroids are +-c, c = E|y_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert np.allclose(np.abs(qz.codebooks[0].centroids), c, rtol=1e-9)
    x = _unit(20000, d, 2)
    qv = oracle.quantize(x, qz)
    xt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)
    ip = np.sum(xt * x, axis=1)
    expect = d * c * c                       # = 1 - D at one bit
    z = (ip.mean() - expect) / (ip.std(ddof=1) / math.sqrt(ip.size))
    assert abs(z) < 5, (ip.mean(), expect)
    # and it is well below 1: the MSE-only estimate shrinks inner products
    assert expect < 0.7


def test_three_bit_bias_and_centroid_condition():
    d, m = 16, 3
    qz = _quantizer(d, m, 6)
    cb = qz.codebooks[0]
    edges = np.concatenate(([-1.0], cb.boundaries, [1.0]))
    D = 0.0
    for k, ck in enumerate(cb.centroids):
        D += integrate.quad(lambda t: (t - ck) ** 2 * _density(t, d), edges[k], edges[k + 1],
                            epsabs=1e-13, epsrel=1e-11)[0]
    D *= d
    assert 0.01 < D < 0.08
    x = _unit(20000, d, 3)
    qv = oracle.quantize(x, qz)
    xt = oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)
    for stat in (np.sum(xt * x, axis=1), np.sum(xt * xt, axis=1)):
        z = (stat.mean() - (1 - D)) / (stat.std(ddof=1) / math.sqrt(stat.size))
        assert abs(z) < 5, (stat.mean(), 1 - D)


def test_two_stage_estimate_of_the_same_vectors_is_unbiased():
    # contrast: with fresh sketches the two-stage estimate of <x, x> has mean 1
    d, m = 16, 1
    x = _unit(1, d, 4)[0]
    pi = synth.haar_orthogonal(synth.rng_for(8, 0, 0), d)
    cbs = [oracle.lloyd_max(d, m)]
    full, mse = [], []
    for s in range(4000):
        sk = np.random.default_rng(50_000 + s).standard_normal((d, d))
        for flag, acc in ((False, full), (True, mse)):
            qz = oracle.Quantizer(d=d, perm=np.arange(d), dims=[d], rotations=[pi], sketches=[sk],
                                  codebooks=cbs, mse_only=flag)
            qv = oracle.quantize(x[None, :], qz)
            acc.append(float(oracle.dequantize(qv.idx, qv.bits, qv.norm, qv.gamma, qz)[0] @ x))
    full, mse = np.array(full), np.array(mse)
    assert abs(full.mean() - 1.0) < 5 * full.std(ddof=1) / math.sqrt(full.size)
    # the MSE-only estimate does not depend on the sketch, and is biased low here
    assert np.ptp(mse) == 0.0 and mse[0] < 0.95


def test_record_sizes_without_sign_words():
    assert oracle.record_words([128], [3], mse_only=True) == (12, 0, 2, 384, 0)
    assert oracle.record_words([64, 64], [3, 2], mse_only=True) == (10, 0, 4, 320, 0)
    assert oracle.record_bytes([128], [3], mse_only=True) == 56         # 48 code bytes + 2 fp32 norms
    assert oracle.record_bytes([128], [4], include_norms=False, mse_only=True) == 64


@pytest.mark.parametrize("dims,bits", [([128], [3]), ([64, 64], [3, 2]), ([40], [4])])
def test_packed_records_match_the_full_layout_codes(dims, bits):
    rng = np.random.default_rng(9)
    n = 64
    idx = [rng.integers(0, 1 << m, (n, d)) for d, m in zip(dims, bits)]
    sb = [rng.integers(0, 2, (n, d)).astype(bool) for d in dims]
    nrm = [rng.random(n).astype(np.float32) for _ in dims]
    gam = [rng.random(n).astype(np.float32) for _ in dims]
    for pack, unpack in ((oracle.pack_token_major, recfmt.unpack_token_major),
                         (oracle.pack_block32, recfmt.unpack_block32)):
        c1, s1, n1 = pack(idx, sb, nrm, gam, dims, bits)
        c0, s0, n0 = pack(idx, sb, nrm, gam, dims, bits, True)
        assert s0.shape[1] == 0 and np.array_equal(c0, c1) and np.array_equal(n0, n1)
        got = unpack(c0, s0, n0, dims, bits, mse_only=True)
        for g in range(len(dims)):
            assert np.array_equal(got[0][g], idx[g]) and got[1][g] is None
            assert np.array_equal(got[2][g], nrm[g]) and np.array_equal(got[3][g], gam[g])

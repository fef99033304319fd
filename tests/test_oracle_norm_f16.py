"""Pins of the oracle's fp16 norm storage (a layout option).

The stored n_g and gamma_g are the float16 numbers nearest to the exact
norms (checked against the binary16 neighbours of each stored value, not
by re-running the rounding), codes and sign bits are those of the float32
layout, the dequantized vectors move by at most the rounding bound, and the
record sizes shrink by 4 bytes per group.
"""
import numpy as np
import pytest

import oracle
import synth


def _spec(d, m, seed):
    pi = synth.haar_orthogonal(synth.rng_for(seed, 0, 0), d)
    sk = synth.gaussian_sketch(synth.rng_for(seed, 0, 1), d)
    return synth.QuantizerSpec(d=d, groups=[synth.GroupSpec(dim=d, mse_bits=m)], perm=np.arange(d),
                               rotations=[pi], sketches=[sk])


def test_stored_norms_are_nearest_binary16():
    spec = _spec(32, 2, 3)
    q16 = oracle.Quantizer.from_spec(spec, norm_f16=True)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 32)) * np.exp(rng.uniform(-4, 4, (300, 1)))
    qv = oracle.quantize(x, q16)
    exact = np.linalg.norm(x, axis=1)
    s = qv.norm[0].astype(np.float64)
    h = qv.norm[0].astype(np.float16)
    assert np.array_equal(h.astype(np.float64), s)             # representable in binary16
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(0)).astype(np.float64)
    assert np.all(np.abs(s - exact) <= np.abs(up - exact))
    assert np.all(np.abs(s - exact) <= np.abs(dn - exact))
    assert np.all(np.abs(s - exact) <= 2.0 ** -11 * exact)    # half a unit in the last place


def test_codes_and_bits_unchanged_and_dequantization_bound():
    spec = _spec(48, 3, 4)
    q32 = oracle.Quantizer.from_spec(spec)
    q16 = oracle.Quantizer.from_spec(spec, norm_f16=True)
    x = np.random.default_rng(3).standard_normal((200, 48)) * 5.0
    a, b = oracle.quantize(x, q32), oracle.quantize(x, q16)
    assert np.array_equal(a.idx[0], b.idx[0]) and np.array_equal(a.bits[0], b.bits[0])
    xa = oracle.dequantize(a.idx, a.bits, a.norm, a.gamma, q32)
    xb = oracle.dequantize(b.idx, b.bits, b.norm, b.gamma, q16)
    # each of the two parts scales by its own norm's rounding (<= 2^-11 relative)
    c = q32.codebooks[0].centroids[a.idx[0]]
    mse_len = np.linalg.norm(c, axis=1) * a.norm[0]
    qjl_len = np.sqrt(np.pi / 2) / 48 * a.gamma[0] * np.linalg.norm(
        np.where(a.bits[0], 1.0, -1.0) @ q32.sketches[0], axis=1)
    bound = 2.0 ** -11 * (mse_len + qjl_len) * (1 + 1e-6) + 1e-6 * mse_len
    assert np.all(np.linalg.norm(xa - xb, axis=1) <= bound)


def test_record_bytes_and_packing():
    assert oracle.record_bytes([128], [3], norm_f16=True) == 68
    assert oracle.record_bytes([64, 64], [3, 2], norm_f16=True) == 64
    assert oracle.record_bytes([128], [3], mse_only=True, norm_f16=True) == 52
    rng = np.random.default_rng(5)
    n = 32
    idx = [rng.integers(0, 8, (n, 128))]
    bits = [rng.integers(0, 2, (n, 128)).astype(bool)]
    nrm = [rng.random(n).astype(np.float16).astype(np.float32)]
    gam = [rng.random(n).astype(np.float16).astype(np.float32)]
    for pack in (oracle.pack_token_major, oracle.pack_block32):
        c32, s32, n32 = pack(idx, bits, nrm, gam, [128], [3])
        c16, s16, n16 = pack(idx, bits, nrm, gam, [128], [3], False, True)
        assert n16.dtype == np.float16 and np.array_equal(n16.astype(np.float32), n32)
        assert np.array_equal(c16, c32) and np.array_equal(s16, s32)

"""Shared helpers of the GPU parity tests: seeded inputs -> (oracle, device)
quantizers, oracle-built caches uploaded to the device, and the record
comparison rule.

Comparison rule for quantized records (codes and sign bits bit-exact except
near decision boundaries): a rotated unit coordinate closer than BAND to a
decision boundary may take either neighbouring cell, and a sketch
coordinate with |s| / n_g < BAND may take either sign; the number of such
disagreements must stay below FRACTION of all coordinates. A vector whose
codes differ from the oracle's must equal one of the oracle's legal variants
(codes, signs and residual norm recomputed for that choice). Norms: n_g to
1e-6 relative, gamma_g to 2e-6 n_g.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth
from tests import recfmt

BAND = 1e-6
FRACTION = 1e-5


def quantizers(spec, mse_only=False, norm_f16=False):
    """(oracle.Quantizer, device Quantizer) for one synth.QuantizerSpec."""
    import kv_cache_vector_rotation_amd as tq
    oq = oracle.Quantizer.from_spec(spec, mse_only=mse_only, norm_f16=norm_f16)
    dq = tq.Quantizer.from_parts(spec.rotations, spec.sketches, [g.mse_bits for g in spec.groups],
                                 perm=spec.perm, mse_only=mse_only, norm_f16=norm_f16)
    return oq, dq


def compare_records(x, oq, qv, got, check_fraction=True):
    """got = (codes, signs, n, gamma) lists per group (from recfmt), rows aligned
    with x / qv. Returns a dict of counts; raises AssertionError on a
    violation. MSE-only records (sign bits None) are checked on codes and
    norms alone. fp16 norms (oq.norm_f16) may differ from the oracle's by one
    float16 unit: the device rounds its float32 value, the oracle its float64
    value."""
    gc, gs, gn, gg = got
    mse_only = gs[0] is None
    h_rel = 2.0 ** -10 if oq.norm_f16 else 0.0
    n_vec = x.shape[0]
    total = n_vec * oq.d
    flips_code = flips_sign = 0
    for g in range(len(oq.dims)):
        idx, bits = qv.idx[g], qv.bits[g]
        norm_ref = qv.norm[g].astype(np.float64)
        nrel = np.abs(gn[g].astype(np.float64) - norm_ref) / np.maximum(norm_ref, 1e-30)
        assert np.all((nrel <= 1e-6 + h_rel) | (norm_ref == 0)), f"norm mismatch, worst {nrel.max()}"
        code_diff = gc[g] != idx
        bad_rows = np.nonzero(code_diff.any(axis=1))[0]
        # every differing code must sit within the band of a boundary
        assert np.all(qv.margin[g][code_diff] < BAND), "code differs away from a boundary"
        flips_code += int(code_diff.sum())
        ok_rows = np.setdiff1d(np.arange(n_vec), bad_rows)
        if not mse_only:
            sdiff = gs[g][ok_rows] != bits[ok_rows]
            assert np.all(qv.sign_margin[g][ok_rows][sdiff] < BAND), "sign differs away from zero"
            flips_sign += int(sdiff.sum())
        gam_ref = qv.gamma[g][ok_rows].astype(np.float64)
        assert np.all(np.abs(gg[g][ok_rows].astype(np.float64) - gam_ref)
                      <= 2e-6 * np.maximum(norm_ref[ok_rows], 1e-30) + h_rel * gam_ref), "residual norm mismatch"
        for r in bad_rows:
            variants = oracle.legal_variants(x[r], oq, g, qv, int(r), BAND)
            match = False
            for vidx, vbits, vgam, vmargin in variants:
                if not np.array_equal(vidx, gc[g][r]):
                    continue
                sd = np.zeros_like(vbits) if mse_only else vbits != gs[g][r]
                if np.all(vmargin[sd] < BAND) and abs(float(gg[g][r]) - float(vgam)) <= \
                        2e-6 * max(norm_ref[r], 1e-30) + h_rel * float(vgam):
                    match = True
                    flips_sign += int(sd.sum())
                    break
            assert match, f"row {r} group {g}: record matches no legal variant"
    if check_fraction:
        assert flips_code + flips_sign < FRACTION * total, (flips_code, flips_sign, total)
    return {"code_flips": flips_code, "sign_flips": flips_sign, "coords": total}


def oracle_cache_arrays(qv, dims, bits, fmt, n_rows, rows, mse_only=False, norm_f16=False):
    """Pack oracle records and place them at the given rows of an n_rows cache.
    Returns numpy (codes, signs, norms) flat arrays matching the device layout."""
    import kv_cache_vector_rotation_amd as tq
    info = oracle.record_words(dims, bits, mse_only)
    cw, sw, nf, bcw, bsw = info
    norms = np.zeros((n_rows, nf), np.float16 if norm_f16 else np.float32)
    if fmt == tq.TQ_TOKEN_MAJOR:
        c, s, nm = oracle.pack_token_major(qv.idx, qv.bits, qv.norm, qv.gamma, dims, bits, mse_only, norm_f16)
        codes = np.zeros((n_rows, cw), np.uint32)
        signs = np.zeros((n_rows, sw), np.uint32)
        codes[rows], signs[rows], norms[rows] = c, s, nm
        return codes.ravel(), signs.ravel(), norms.ravel()
    # block records: rows must cover whole blocks in order
    rows = np.asarray(rows)
    assert rows.size % 32 == 0 and np.all(rows.reshape(-1, 32)[:, 0] % 32 == 0)
    assert np.all(np.diff(rows.reshape(-1, 32), axis=1) == 1)
    c, s, nm = oracle.pack_block32(qv.idx, qv.bits, qv.norm, qv.gamma, dims, bits, mse_only, norm_f16)
    codes = np.zeros((n_rows // 32, bcw), np.uint32)
    signs = np.zeros((n_rows // 32, bsw), np.uint32)
    blocks = rows.reshape(-1, 32)[:, 0] // 32
    codes[blocks], signs[blocks] = c, s
    norms[rows] = nm
    return codes.ravel(), signs.ravel(), norms.ravel()


def to_device_cache(dq, fmt, n_rows, arrays):
    import torch
    import kv_cache_vector_rotation_amd as tq
    c, s, n = arrays
    cache = tq.Cache.empty(dq, n_rows, fmt)
    cache.codes.copy_(torch.from_numpy(c.view(np.int32)))
    cache.signs.copy_(torch.from_numpy(s.view(np.int32)))
    cache.norms.copy_(torch.from_numpy(n))
    return cache


def read_cache(cache, dq):
    """Device cache -> recfmt tuple (codes, signs, n, gamma per group)."""
    import kv_cache_vector_rotation_amd as tq
    info = tq.tq_record_layout(dq.layout)
    codes = cache.codes.cpu().numpy().view(np.uint32)
    signs = cache.signs.cpu().numpy().view(np.uint32)
    norms = cache.norms.cpu().numpy().reshape(cache.n_rows, info.norm_floats)
    mse = bool(dq.layout.mse_only)
    if cache.fmt == tq.TQ_TOKEN_MAJOR:
        return recfmt.unpack_token_major(codes.reshape(cache.n_rows, -1), signs.reshape(cache.n_rows, -1),
                                         norms, dq.dims, dq.mse_bits, mse)
    nb = cache.n_rows // 32
    return recfmt.unpack_block32(codes.reshape(nb, -1), signs.reshape(nb, -1), norms, dq.dims, dq.mse_bits, mse)


def select_rows(got, rows):
    return tuple([None if a is None else a[rows] for a in part] for part in got)


def normwise_close(got, ref, tol=2e-3):
    """Per row: max |got - ref| <= tol * max |ref| (rows = last axis reduced)."""
    err = np.max(np.abs(got - ref), axis=-1)
    scale = np.max(np.abs(ref), axis=-1)
    worst = float(np.max(err / np.maximum(scale, 1e-30)))
    return worst <= tol, worst

"""Inner-product estimation and attention over the compressed cache
(oracle; test infrastructure).

[WD] intro and table in "Os numeros que importam": the compressed cache is
used to compute attention logits; [WD] "2. QJL Residual": the 1-bit sketch
of the residual removes the bias of the inner product. The decode step then
takes softmax(logits) times the dequantized values.

Readings used here (where the pages leave a step open; each is cited where it is used):
* dequantized vector, per group:
      x~_g = n_g Pi_g^T c[idx] + alpha_g gamma_g S_g^T z,
  with z = 2 bit - 1 and alpha_g = sqrt(pi/2) / d_g. For S_g with iid
  N(0,1) rows this is unbiased for x_g: E[S^T sign(S r)] = d_g sqrt(2/pi)
  r / ||r|| (Gaussian sign identity). Channels are then put back in their
  original order (the inverse of ``perm``);
* queries are not quantized: logit = scale * <q, x~>;
* decode attends over every cached token (no mask); query head h reads KV
  head floor(h / G) with G = n_q_heads / n_kv_heads;
* V uses the same dequantization as K with its own quantizer;
* an MSE-only quantizer (stage one alone) dequantizes to n_g Pi_g^T c[idx]:
  no sign term. That estimate is biased: over random rotations its mean is
  (1 - D) x, with D the codebook's mean squared error on unit vectors.
The norms used are the stored float32 values.
"""
from __future__ import annotations

import numpy as np

from .quantize import Quantizer


def dequantize(idx, bits, norm, gamma, qz: Quantizer) -> np.ndarray:
    """Rebuild vectors [n, d] (float64) from per-group codes, sign bits and
    stored norms (lists over groups, as in ``QuantizedVectors``)."""
    n_vec = idx[0].shape[0]
    xp = np.zeros((n_vec, qz.d), dtype=np.float64)
    for g, (off, dg) in enumerate(zip(qz.offsets, qz.dims)):
        c = qz.codebooks[g].centroids
        pi, sm = qz.rotations[g], qz.sketches[g]
        alpha = np.sqrt(np.pi / 2.0) / dg
        z = np.where(bits[g], 1.0, -1.0)
        n = np.asarray(norm[g], dtype=np.float64)[:, None]
        gm = np.asarray(gamma[g], dtype=np.float64)[:, None]
        mse_part = n * (c[idx[g]] @ pi)               # n Pi^T c[idx]
        if qz.mse_only:
            xp[:, off:off + dg] = mse_part
            continue
        qjl_part = alpha * gm * (z @ sm)              # alpha gamma S^T z
        xp[:, off:off + dg] = mse_part + qjl_part
    out = np.empty_like(xp)
    out[:, qz.perm] = xp
    return out


def estimate_logits(q: np.ndarray, k_tilde: np.ndarray, scale: float) -> np.ndarray:
    """scale * <q_h, k~_i> for queries [H, d] and dequantized keys [N, d]."""
    return scale * (np.asarray(q, np.float64) @ k_tilde.T)


def softmax(logits: np.ndarray) -> np.ndarray:
    """Row-wise softmax with the row maximum subtracted first."""
    z = logits - np.max(logits, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_decode(q: np.ndarray, k_tilde: np.ndarray, v_tilde: np.ndarray | None,
                     scale: float):
    """One decode step for one batch element.

    q [H_q, d]; k_tilde / v_tilde [H_kv, N, d] (dequantized caches).
    Returns (logits [H_q, N], out [H_q, d] or None when v_tilde is None)."""
    hq = q.shape[0]
    hkv = k_tilde.shape[0]
    group = hq // hkv
    logits = np.empty((hq, k_tilde.shape[1]), dtype=np.float64)
    out = None if v_tilde is None else np.empty((hq, q.shape[1]), dtype=np.float64)
    for h in range(hq):
        kv = h // group
        logits[h] = estimate_logits(q[h][None, :], k_tilde[kv], scale)[0]
        if v_tilde is not None:
            p = softmax(logits[h])
            out[h] = p @ v_tilde[kv]
    return logits, out


def attention_prefill(q: np.ndarray, k_tilde: np.ndarray, v_tilde: np.ndarray | None, scale: float):
    """A chunk of T query tokens for one batch element, attended causally.

    q [T, H_q, d]; k_tilde / v_tilde [H_kv, N, d] (dequantized caches that
    already hold the chunk's own T tokens as their last rows). Query token i
    sits at position N - T + i and sees tokens 0 .. N - T + i (reading: a
    prefill chunk attends to the cached prefix and causally within itself).
    A token with no visible key (N - T + i < 0: a sequence shorter than the
    chunk) keeps -inf logits and gets a zero output, the empty sum (reading:
    the pages say nothing of this case).
    Returns (logits [H_q, T, N] with -inf past each token's limit,
    out [T, H_q, d] or None)."""
    T, hq, d = q.shape
    hkv, n = k_tilde.shape[0], k_tilde.shape[1]
    group = hq // hkv
    logits = np.full((hq, T, n), -np.inf)
    out = None if v_tilde is None else np.empty((T, hq, d), dtype=np.float64)
    for i in range(T):
        lim = n - T + i + 1
        if lim <= 0:
            if out is not None:
                out[i] = 0.0
            continue
        for h in range(hq):
            kv = h // group
            row = estimate_logits(q[i, h][None, :], k_tilde[kv, :lim], scale)[0]
            logits[h, i, :lim] = row
            if v_tilde is not None:
                out[i, h] = softmax(row[None, :])[0] @ v_tilde[kv, :lim]
    return logits, out

"""The steps around the delta rule in a linear-attention layer, in float64. TEST INFRASTRUCTURE ONLY.

Definitions followed (model page ``model.py``; the layer order is that of ``_linear_layer`` and
``_fork_linear_layer``):

* ``dn_gates`` (function ``_dn_gates``): beta = sigmoid(b) * valid and
  g = -exp(A_log) * softplus(a + dt_bias) * valid, per (row, token, value head), with A_log and
  dt_bias per value head. Padded positions get beta = g = 0 exactly.
* ``conv_silu`` (function ``_conv_silu`` plus the tail gather of ``_linear_layer``): the
  depthwise causal convolution over ext = [tail ; mixed] along time,
      pre[t, c] = sum_{j=0}^{K-1} ext[t + j, c] w[c, j],   out = silu(pre),
  split along channels into q (Hk*D), k (Hk*D) and v (Hv*D); the new tail is
  ext[len_b + j] for j = 0 .. K-2, the last K-1 inputs up to the row's length.
* ``gated_rmsnorm`` (function ``_gated_rms``): y = w * x / sqrt(mean(x^2) + eps) * silu(z)
  over the last axis (one value head's D = 128 outputs).

Every intermediate is float64; the page's casts between float32 and the activation dtype are
rounding choices, not part of the definition (its float32 upcasts before the norm and the
softplus exist only to keep bf16 accurate). Inputs arrive at the values the GPU receives.
"""
from __future__ import annotations

import numpy as np


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def valid_mask(B: int, L: int, lengths) -> np.ndarray:
    """[B, L] float64: 1 where t < lengths[b] (all ones if lengths is None)."""
    if lengths is None:
        return np.ones((B, L))
    return (np.arange(L)[None, :] < np.asarray(lengths, dtype=np.int64)[:, None]).astype(np.float64)


def dn_gates(b, a, A_log, dt_bias, lengths=None):
    """beta, g [B, L, Hv] from the raw projections b, a [B, L, Hv] and the per-head A_log,
    dt_bias [Hv] (``model.py``, function ``_dn_gates``)."""
    b = np.asarray(b, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    v = valid_mask(b.shape[0], b.shape[1], lengths)[..., None]
    beta = sigmoid(b) * v
    g = -np.exp(A_log) * softplus(a + dt_bias) * v
    return beta, g


def conv_silu(mixed, tail, w, Hk: int, Hv: int, D: int = 128, lengths=None):
    """Causal depthwise conv + SiLU with tail continuation and the q/k/v split.

    mixed [B, L, Cm] with Cm = (2 Hk + Hv) D; tail [B, K-1, Cm] (None = zeros); w [Cm, K].
    Returns q [B, L, Hk, D], k [B, L, Hk, D], v [B, L, Hv, D] and new_tail [B, K-1, Cm]
    (``model.py``, functions ``_conv_silu`` and ``_linear_layer``).
    """
    mixed = np.asarray(mixed, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, L, Cm = mixed.shape
    K = w.shape[1]
    assert Cm == (2 * Hk + Hv) * D and w.shape[0] == Cm
    tail = np.zeros((B, K - 1, Cm)) if tail is None else np.asarray(tail, dtype=np.float64)
    ext = np.concatenate([tail, mixed], axis=1)                 # [B, K-1+L, Cm]
    pre = np.zeros((B, L, Cm))
    for j in range(K):
        pre += ext[:, j:j + L, :] * w[:, j]
    out = silu(pre)
    lens = np.full(B, L) if lengths is None else np.asarray(lengths, dtype=np.int64)
    new_tail = np.stack([ext[bi, lens[bi]:lens[bi] + K - 1] for bi in range(B)])
    kd = Hk * D
    q = out[..., :kd].reshape(B, L, Hk, D)
    k = out[..., kd:2 * kd].reshape(B, L, Hk, D)
    v = out[..., 2 * kd:].reshape(B, L, Hv, D)
    return q, k, v, new_tail


def gated_rmsnorm(x, z, w, eps: float):
    """w * x / sqrt(mean(x^2, last axis) + eps) * silu(z) (``model.py``, function ``_gated_rms``)."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    r = 1.0 / np.sqrt((x * x).mean(-1, keepdims=True) + eps)
    return w * (x * r) * silu(z)

"""The gated delta rule as a float64 token-by-token recurrence. TEST INFRASTRUCTURE ONLY.

Definition followed (kernel-test page ``r15_kernel_test.py``, function ``truth_f64``; the same
order in the model page ``model.py``, function ``delta_rule_reference``):

1. upcast every input to float64 (bf16 inputs are taken at their bf16 values);
2. q_hat = q / sqrt(sum q^2 + 1e-6) * D^-1/2 and k_hat = k / sqrt(sum k^2 + 1e-6)
   (``model.py``, function ``_l2norm``: eps is added to the sum of squares inside the rsqrt);
3. right-pad guard: beta' = beta * valid and g' = g * valid, valid_t = [t < length]
   (``model.py``, function ``_dn_gates``, which multiplies both gates by the valid mask);
4. per (row b, value head h), with key head kh = floor(h / (Hv / Hk)) (``model.py``,
   function ``_linear_layer``, which repeats each key head r times along the head axis, and
   the kernel-test page's head pairs 0::2 == 1::2), starting from S = s0[s0_row[b], h] or 0:
   for t = 0 .. L-1:
       S <- S * exp(g'_t)
       kv <- S^T k_hat_t
       delta <- beta'_t (v_t - kv)
       S <- S + k_hat_t delta^T
       o_t <- S^T q_hat_t
5. return o (float64 [B, L, Hv, Dv]) and the last S (float64 [B, Hv, Dk, Dv]).

The state is [Dk, Dv] (key index first), as the model page's ``State`` docstring gives
(recurrent [B, H, K, V]). The output at a pad position is what the recurrence gives there
(the frozen state read with that position's q_hat); no zeroing is applied.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2norm(x: np.ndarray, eps: float = EPS) -> np.ndarray:
    """x / sqrt(sum(x^2, last axis) + eps), in float64 (``model.py``, function ``_l2norm``)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def guard(g: np.ndarray, beta: np.ndarray, lengths) -> tuple[np.ndarray, np.ndarray]:
    """beta' = beta * valid, g' = g * valid with valid[b, t] = t < lengths[b].

    ``model.py``, function ``_dn_gates``: pads become exact no-ops (no write, no decay).
    lengths None means every position is valid.
    """
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    if lengths is None:
        return g, beta
    L = g.shape[1]
    valid = (np.arange(L)[None, :] < np.asarray(lengths, dtype=np.int64)[:, None]).astype(np.float64)
    return g * valid[..., None], beta * valid[..., None]


def gated_delta_rule(q, k, v, g, beta, lengths=None, s0=None, s0_row=None, rows=None, heads=None):
    """Token-by-token float64 gated delta rule.

    q, k: [B, L, Hk, Dk]; v: [B, L, Hv, Dv]; g, beta: [B, L, Hv]; lengths: [B] or None;
    s0: [n_s0, Hv, Dk, Dv] or None (zeros); s0_row: [B] indices into s0 or None (row b uses
    s0[b]). rows / heads: optional index lists selecting which batch rows and value heads to
    compute (each (row, head) pair is independent, so a subset is exact); the outputs then
    have len(rows) and len(heads) entries on those axes.

    Returns (o [B', L, H', Dv], S [B', H', Dk, Dv]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if Hv % Hk:
        raise ValueError("Hv must be a multiple of Hk")
    r = Hv // Hk
    rows = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hv) if heads is None else np.asarray(heads, dtype=np.int64)
    kh = heads // r

    gq, bq = guard(g, beta, lengths)
    gq, bq = gq[rows][:, :, heads], bq[rows][:, :, heads]            # [B', L, H']
    qh = l2norm(q[rows][:, :, kh]) * Dk ** -0.5                       # [B', L, H', Dk]
    kn = l2norm(k[rows][:, :, kh])
    vv = v[rows][:, :, heads]                                          # [B', L, H', Dv]

    nb, nh = len(rows), len(heads)
    if s0 is None:
        S = np.zeros((nb, nh, Dk, Dv))
    else:
        s0 = np.asarray(s0, dtype=np.float64)
        src = rows if s0_row is None else np.asarray(s0_row, dtype=np.int64)[rows]
        S = s0[src][:, heads].copy()
    o = np.empty((nb, L, nh, Dv))
    for t in range(L):
        S *= np.exp(gq[:, t])[..., None, None]
        kt = kn[:, t]                                                  # [B', H', Dk]
        kv = np.matmul(kt[..., None, :], S)[..., 0, :]                 # S^T k
        delta = (vv[:, t] - kv) * bq[:, t, :, None]
        S += kt[..., :, None] * delta[..., None, :]
        o[:, t] = np.matmul(qh[:, t][..., None, :], S)[..., 0, :]      # S^T q
    return o, S

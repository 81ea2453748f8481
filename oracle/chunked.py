"""The gated delta rule evaluated C tokens at a time, in float64. TEST INFRASTRUCTURE ONLY.

This is a second, independent formulation of the recurrence in ``recurrence.py``, used to pin
the chunk algebra on tiny shapes. It is derived from the recurrence of the kernel-test page
(``r15_kernel_test.py``, function ``truth_f64``) by unrolling it over one chunk; the pages
name the chunked kernel forms (``R64``, cumulative or direct decay) but never spell out their
algebra. With gamma_t = sum_{i <= t} g'_i inside the chunk (t = 0 .. C-1), and S0 the state
entering the chunk:

    A[t, i]  = beta'_t exp(gamma_t - gamma_i) (k_hat_t . k_hat_i)   for i < t, else 0
    T        = (I + A)^-1                                            (explicit inverse here)
    W        = T diag(beta' exp(gamma)) K_hat
    U        = T diag(beta') V
    Delta    = U - W S0                                              (row t = delta_t^T)
    O        = diag(exp(gamma)) Q_hat S0 + (Q_hat K_hat^T * E) Delta, E[t, i] = exp(gamma_t - gamma_i) for i <= t
    S_C      = exp(gamma_{C-1}) S0 + K_hat^T diag(exp(gamma_{C-1} - gamma)) Delta

A partial last chunk simply has fewer rows. With C = 1 this is the recurrence itself.
Exponents are only ever taken of non-positive differences on the kept (lower) triangle; the
masked entries are set before the exponential, so nothing overflows.
"""
from __future__ import annotations

import numpy as np

from .recurrence import guard, l2norm


def gated_delta_rule_chunked(q, k, v, g, beta, C: int, lengths=None, s0=None, s0_row=None):
    """Same contract as ``recurrence.gated_delta_rule`` (all rows and heads), chunk size C."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    r = Hv // Hk
    gq, bq = guard(g, beta, lengths)
    qh = l2norm(q) * Dk ** -0.5
    kn = l2norm(k)
    o = np.empty((B, L, Hv, Dv))
    S_out = np.empty((B, Hv, Dk, Dv))
    for b in range(B):
        for h in range(Hv):
            kh = h // r
            if s0 is None:
                S = np.zeros((Dk, Dv))
            else:
                src = b if s0_row is None else int(np.asarray(s0_row)[b])
                S = np.asarray(s0, dtype=np.float64)[src, h].copy()
            for c0 in range(0, L, C):
                c1 = min(c0 + C, L)
                Qc, Kc, Vc = qh[b, c0:c1, kh], kn[b, c0:c1, kh], v[b, c0:c1, h]
                bc = bq[b, c0:c1, h]
                gam = np.cumsum(gq[b, c0:c1, h])
                n = c1 - c0
                diff = gam[:, None] - gam[None, :]                  # gamma_t - gamma_i
                lower_strict = np.tril(np.ones((n, n), dtype=bool), -1)
                lower_incl = np.tril(np.ones((n, n), dtype=bool), 0)
                E_strict = np.where(lower_strict, np.exp(np.where(lower_strict, diff, 0.0)), 0.0)
                E_incl = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
                A = bc[:, None] * E_strict * (Kc @ Kc.T)
                T = np.linalg.inv(np.eye(n) + A)
                W = T @ ((bc * np.exp(gam))[:, None] * Kc)
                U = T @ (bc[:, None] * Vc)
                Delta = U - W @ S
                O = np.exp(gam)[:, None] * (Qc @ S) + ((Qc @ Kc.T) * E_incl) @ Delta
                S = np.exp(gam[-1]) * S + Kc.T @ (np.exp(gam[-1] - gam)[:, None] * Delta)
                o[b, c0:c1, h] = O
            S_out[b, h] = S
    return o, S_out

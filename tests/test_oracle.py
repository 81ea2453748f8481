"""Pins for the float64 oracle (CPU only).

The pages print no output values for this method, so the oracle is pinned against what the
mathematics fixes: closed forms of special regimes, exact invariants, and an independent
chunked formulation on tiny shapes. Each test names the mistake it is there to catch.
"""
import os

import numpy as np
import pytest
import torch

from oracle import gated_delta_rule, gated_delta_rule_chunked, l2norm, guard
from workloads import draw, CONFIGS


def rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def np_inputs(x):
    return (x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy(),
            x.g.double().numpy(), x.beta.double().numpy())


# ---------------------------------------------------------------- l2norm
def test_l2norm_eps_inside_rsqrt():
    # sum of squares 25e-6, plus eps 1e-6 -> sqrt(26e-6); F.normalize would give [0.6, 0.8].
    x = np.array([3e-3, 4e-3])
    got = l2norm(x)
    want = np.array([3e-3, 4e-3]) / 5.0990195135927845e-3
    assert np.allclose(got, want, rtol=1e-15, atol=0)
    assert abs(got[0] - 0.6) > 1e-2   # not max(|x|, eps) normalisation


# ---------------------------------------------------------------- closed forms
def one_key_closed_form(q, k, v, g, beta, s0):
    """O(L*D) algorithm for a single key per head (all k_t equal), any decay.

    With k_hat fixed, c = |k_hat|^2, m = S^T k_hat and n_t = sum_i exp(G_t - G_i) delta_i:
      delta_t = beta_t (v_t - exp(g_t) m_{t-1});  m_t = exp(g_t) m_{t-1} + c delta_t
      n_t = exp(g_t) n_{t-1} + delta_t;  G_t = G_{t-1} + g_t
      o_t = exp(G_t) S0^T q_hat_t + (k_hat . q_hat_t) n_t;  S_L = exp(G_L) S0 + k_hat n_L^T
    One row, one head: q [L, D], k [D], v [L, Dv], g, beta [L], s0 [D, Dv].
    """
    D = q.shape[-1]
    kh = k / np.sqrt(k @ k + 1e-6)
    c = kh @ kh
    m = s0.T @ kh
    n = np.zeros(v.shape[1])
    G = 0.0
    out = []
    for t in range(q.shape[0]):
        qh = q[t] / np.sqrt(q[t] @ q[t] + 1e-6) * D ** -0.5
        a = np.exp(g[t])
        delta = beta[t] * (v[t] - a * m)
        m = a * m + c * delta
        n = a * n + delta
        G += g[t]
        out.append(np.exp(G) * (s0.T @ qh) + (kh @ qh) * n)
    return np.array(out), np.exp(G) * s0 + np.outer(kh, n)


@pytest.mark.parametrize("decay", ["none", "weak", "strong"])
@pytest.mark.parametrize("scale", [1.0, 1e-3])
def test_one_key_closed_form(decay, scale):
    # Catches: decay applied after the read, output read before the update, S transposed,
    # eps outside the rsqrt (scale 1e-3 makes |k|^2 comparable to eps), missing D^-1/2.
    rng = np.random.default_rng(7)
    L, D, Dv, H = 150, 8, 8, 3
    k1 = rng.standard_normal((1, 1, H, D)) * scale
    k = np.broadcast_to(k1, (1, L, H, D)).copy()
    q = rng.standard_normal((1, L, H, D)) * scale
    v = rng.standard_normal((1, L, H, Dv))
    beta = rng.uniform(0.2, 0.9, (1, L, H))
    g = {"none": np.zeros((1, L, H)), "weak": -0.02 * rng.uniform(size=(1, L, H)),
         "strong": -rng.uniform(0.05, 3.0, (1, L, H))}[decay]
    s0 = 0.1 * rng.standard_normal((1, H, D, Dv))
    o, S = gated_delta_rule(q, k, v, g, beta, s0=s0)
    for h in range(H):
        o_cf, S_cf = one_key_closed_form(q[0, :, h], k[0, 0, h], v[0, :, h], g[0, :, h], beta[0, :, h], s0[0, h])
        assert rel(o[0, :, h], o_cf) < 1e-12
        assert rel(S[0, h], S_cf) < 1e-12


def test_one_key_regime_r4_full_width():
    # The page's R4 regime (one key for every token, beta = 0.5, g = 0) at D = 128, with S0.
    x = draw(1, 200, 2, 4, 128, "R4", 41, s0_rows=1)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    o, S = gated_delta_rule(q, k, v, g, beta, s0=s0)
    for h in range(4):
        kh = h // 2
        o_cf, S_cf = one_key_closed_form(q[0, :, kh], k[0, 0, kh], v[0, :, h], g[0, :, h], beta[0, :, h], s0[0, h])
        assert rel(o[0, :, h], o_cf) < 1e-12
        assert rel(S[0, h], S_cf) < 1e-12


def test_beta_zero_is_pure_decay():
    # beta = 0: nothing is written; o_t = exp(sum_{i<=t} g_i) S0^T q_hat_t, S_L = exp(sum g) S0.
    rng = np.random.default_rng(3)
    L, D, H = 40, 16, 2
    q = rng.standard_normal((1, L, H, D))
    k = rng.standard_normal((1, L, H, D))
    v = rng.standard_normal((1, L, H, D))
    g = -rng.uniform(0.0, 0.3, (1, L, H))
    s0 = rng.standard_normal((1, H, D, D))
    o, S = gated_delta_rule(q, k, v, g, np.zeros((1, L, H)), s0=s0)
    G = np.cumsum(g[0], axis=0)                                      # [L, H]
    qh = l2norm(q[0]) * D ** -0.5                                    # [L, H, D]
    want = np.exp(G)[..., None] * np.einsum("hkv,lhk->lhv", s0[0], qh)
    assert rel(o[0], want) < 1e-13
    assert rel(S[0], np.exp(G[-1])[:, None, None] * s0[0]) < 1e-13


def test_orthonormal_keys_is_causal_linear_attention():
    # k_t = e_t (distinct unit keys), g = 0, S0 = 0: every read S^T k_hat_t is 0 on a fresh
    # direction, so o_t = sum_{i<=t} beta_i (q_hat_t . k_hat_i) v_i.
    rng = np.random.default_rng(5)
    L, D, Dv = 24, 32, 16
    k = np.zeros((1, L, 1, D))
    for t in range(L):
        k[0, t, 0, t] = 1.0
    q = rng.standard_normal((1, L, 1, D))
    v = rng.standard_normal((1, L, 1, Dv))
    beta = rng.uniform(0.2, 0.9, (1, L, 1))
    o, S = gated_delta_rule(q, k, v, np.zeros((1, L, 1)), beta)
    kh = l2norm(k[0, :, 0])
    qh = l2norm(q[0, :, 0]) * D ** -0.5
    scores = np.tril(qh @ kh.T) * beta[0, :, 0][None, :]
    assert rel(o[0, :, 0], scores @ v[0, :, 0]) < 1e-13
    assert rel(S[0, 0], kh.T @ (beta[0, :, 0][:, None] * v[0, :, 0])) < 1e-13


# ---------------------------------------------------------------- invariants
def test_joint_linearity_2_pow_8_bitwise():
    # Scaling (v, S0) by 2^8 scales (o, S_final) by exactly 2^8 (kernel-test page docstring:
    # the delta rule is linear in (v, state) jointly). Catches a term missing v or S.
    x = draw(1, 130, 2, 4, 16, "R1", 12, s0_rows=1, Dv=16)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    o1, S1 = gated_delta_rule(q, k, v, g, beta, s0=s0)
    o2, S2 = gated_delta_rule(q, k, v * 256.0, g, beta, s0=s0 * 256.0)
    assert np.array_equal(o2, o1 * 256.0)
    assert np.array_equal(S2, S1 * 256.0)
    o3, _ = gated_delta_rule(q, k, v * 256.0, g, beta, s0=s0)         # the wrong contract
    assert not np.allclose(o3, o1 * 256.0, rtol=1e-6)


def test_pad_guard_equals_truncation_bitwise():
    # Positions at or past length[b] are exact no-ops even with garbage beta/g stored there:
    # S_final equals the state after the last valid token, outputs before are unchanged.
    B, L, D = 3, 37, 8
    x = draw(B, L, 1, 2, D, "R1", 13, s0_rows=B, zero_pads=False)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    lengths = np.array([37, 20, 0])
    o, S = gated_delta_rule(q, k, v, g, beta, lengths=lengths, s0=s0)
    for b, n in enumerate(lengths):
        if n:
            o_t, S_t = gated_delta_rule(q[b:b + 1, :n], k[b:b + 1, :n], v[b:b + 1, :n], g[b:b + 1, :n],
                                        beta[b:b + 1, :n], s0=s0[b:b + 1])
            assert np.array_equal(o[b, :n], o_t[0])
            assert np.array_equal(S[b], S_t[0])
        else:
            assert np.array_equal(S[b], s0[b])
        # at a pad, the output reads the frozen state: o_t = S_final^T q_hat_t
        qh = l2norm(q[b, n:]) * D ** -0.5                          # [L-n, 1, D]
        want = np.einsum("hkv,lhk->lhv", S[b], np.repeat(qh, 2, axis=1))
        assert rel(o[b, n:], want) < 1e-14 if n < L else True


def test_guard_multiplies_gates_by_valid():
    g = np.full((1, 4, 1), -0.5)
    beta = np.full((1, 4, 1), 0.7)
    gq, bq = guard(g, beta, [2])
    assert gq[0, :, 0].tolist() == [-0.5, -0.5, 0.0, 0.0]
    assert bq[0, :, 0].tolist() == [0.7, 0.7, 0.0, 0.0]


def test_split_continuation_bitwise():
    # Running [0, s) then [s, L) from the carried state equals one run (checkpoint/resume).
    x = draw(2, 90, 2, 4, 16, "R2", 14, s0_rows=2)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    o, S = gated_delta_rule(q, k, v, g, beta, s0=s0)
    s = 41
    oa, Sa = gated_delta_rule(q[:, :s], k[:, :s], v[:, :s], g[:, :s], beta[:, :s], s0=s0)
    ob, Sb = gated_delta_rule(q[:, s:], k[:, s:], v[:, s:], g[:, s:], beta[:, s:], s0=Sa)
    assert np.array_equal(np.concatenate([oa, ob], 1), o)
    assert np.array_equal(Sb, S)


def test_head_map_equals_repeat_interleave_copy():
    # Value head h reads key head h // r: same result as copying each key head r times
    # (model page, _linear_layer's repeat_interleave along the head axis). Catches h % Hk.
    x = draw(1, 50, 3, 6, 8, "R1", 15, s0_rows=1)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    o, S = gated_delta_rule(q, k, v, g, beta, s0=s0)
    qc, kc = np.repeat(q, 2, axis=2), np.repeat(k, 2, axis=2)
    o2, S2 = gated_delta_rule(qc, kc, v, g, beta, s0=s0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


def test_head_pairs_identical():
    # Kernel-test page: with identical v, beta, g per pair, the two value heads agree bitwise.
    x = draw(1, 64, 2, 4, 8, "R1", 16)
    q, k, v, g, beta = np_inputs(x)
    v[:, :, 1::2], g[:, :, 1::2], beta[:, :, 1::2] = v[:, :, 0::2], g[:, :, 0::2], beta[:, :, 0::2]
    o, S = gated_delta_rule(q, k, v, g, beta)
    assert np.array_equal(o[:, :, 0::2], o[:, :, 1::2]) and np.array_equal(S[:, 0::2], S[:, 1::2])


def test_s0_row_index_map():
    # Row b starts from s0[s0_row[b]] (the fork model's h0 / h0_idx), same as gathering first.
    x = draw(3, 20, 1, 2, 8, "R1", 17, s0_rows=2)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    rows = np.array([1, 0, 1])
    o, S = gated_delta_rule(q, k, v, g, beta, s0=s0, s0_row=rows)
    o2, S2 = gated_delta_rule(q, k, v, g, beta, s0=s0[rows])
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


def test_row_head_subset_is_exact():
    x = draw(3, 33, 2, 4, 8, "R1", 18, s0_rows=3)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    lengths = [33, 10, 25]
    o, S = gated_delta_rule(q, k, v, g, beta, lengths=lengths, s0=s0)
    os_, Ss = gated_delta_rule(q, k, v, g, beta, lengths=lengths, s0=s0, rows=[2, 0], heads=[3, 1])
    assert np.array_equal(os_, o[[2, 0]][:, :, [3, 1]])
    assert np.array_equal(Ss, S[[2, 0]][:, [3, 1]])


# ---------------------------------------------------------------- chunked vs sequential
@pytest.mark.parametrize("C", [1, 2, 4, 8, 64])
@pytest.mark.parametrize("regime", ["R1", "R2", "R3"])
def test_chunked_matches_recurrence(C, regime):
    # Pins the chunk algebra the kernels implement (C = 1 is the recurrence itself).
    D = 8 if C < 64 else 16
    L = 3 * C + 5 if C < 64 else 200
    x = draw(2, L, 1, 2, D, regime, 100 + C, s0_rows=2, zero_pads=False)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    lengths = [L, L - 7]
    o, S = gated_delta_rule(q, k, v, g, beta, lengths=lengths, s0=s0)
    oc, Sc = gated_delta_rule_chunked(q, k, v, g, beta, C, lengths=lengths, s0=s0)
    assert rel(oc, o) < 1e-12
    assert rel(Sc, S) < 1e-12


@pytest.mark.parametrize("L", [1, 2, 3, 63, 64, 65, 130])
def test_chunked_tails(L):
    x = draw(1, L, 2, 4, 16, "R1", 200 + L, s0_rows=1)
    q, k, v, g, beta = np_inputs(x)
    s0 = x.s0.double().numpy()
    o, S = gated_delta_rule(q, k, v, g, beta, s0=s0)
    oc, Sc = gated_delta_rule_chunked(q, k, v, g, beta, 64, s0=s0)
    assert rel(oc, o) < 1e-12 and rel(Sc, S) < 1e-12


# ---------------------------------------------------------------- generators
def test_generators_shapes_and_reproducible():
    for i in (1, 2, 3):
        spec = CONFIGS[i]
        a, b = spec.draw(), spec.draw()
        assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v) and torch.equal(a.g, b.g)
        B, L, Hk, Hv, D, Dv = a.shape
        assert (B, L, Hk, Hv, D, Dv) == (spec.B, spec.L, spec.Hk, spec.Hv, 128, 128)
        assert a.q.dtype == spec.dtype and a.g.dtype == torch.float32
        assert (a.g <= 0).all() and (a.beta >= 0).all() and (a.beta <= 1).all()
    c2 = CONFIGS[2].draw()
    assert c2.lengths.tolist() == [130]
    assert (c2.beta[:, 130:] == 0).all() and (c2.g[:, 130:] == 0).all()
    assert (c2.beta[:, :130] > 0).all()
    assert c2.s0.shape == (1, 32, 128, 128)


def test_generator_fork_lengths():
    x = draw(64, 0, 2, 4, 16, "R1", 41, lengths="random:32:1024", s0_rows=1, s0_row=[0] * 64)
    lens = x.lengths
    assert lens.min() >= 32 and lens.max() <= 1024
    assert x.q.shape[1] % 64 == 0 and x.q.shape[1] >= int(lens.max()) > x.q.shape[1] - 64
    pad = torch.arange(x.q.shape[1])[None] >= lens[:, None].long()
    assert (x.beta[pad] == 0).all() and (x.g[pad] == 0).all()
    assert x.s0_row.tolist() == [0] * 64


def test_generator_correlated_keys():
    x = draw(1, 512, 2, 4, 128, "R3", 31)
    k = x.k.double()
    u = k.mean(1, keepdim=True)
    cos = (k * u).sum(-1) / (k.norm(dim=-1) * u.norm(dim=-1))
    assert cos.min() > 0.8        # keys cluster around one direction per key head


def test_golden_regression_fixture():
    """The oracle still reproduces its frozen output on one tiny case (tests/golden)."""
    import json
    import importlib.util
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(here, "oracle_small.json")) as f:
        ref = json.load(f)
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(here, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.CASE == {k: (v if not isinstance(v, list) else v) for k, v in ref["case"].items()}
    o, s = mod.compute()
    np.testing.assert_allclose(o, np.array(ref["o"]), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(s, np.array(ref["s_final"]), rtol=1e-12, atol=1e-15)

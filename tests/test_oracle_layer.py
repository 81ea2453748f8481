"""Pins for the float64 oracle of the layer steps around the delta rule (CPU only).

Gate prologue, causal depthwise conv + SiLU with tail continuation, gated RMSNorm (model page
``model.py``: ``_dn_gates``, ``_conv_silu`` with the tail gather of ``_linear_layer``,
``_gated_rms``). The pages print no values for them, so each is pinned against closed forms,
a library routine on a different formulation, or an invariant; each test names the mistake it
catches.
"""
import math

import numpy as np
import pytest

from oracle.layer import conv_silu, dn_gates, gated_rmsnorm, sigmoid, silu, softplus


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- gates
def test_sigmoid_softplus_silu_special_values():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, softplus(0) = ln 2, softplus(ln 3) = ln 4,
    # silu(ln 3) = 0.75 ln 3; and the large-argument limits without overflow
    assert sigmoid(0.0) == 0.5
    assert math.isclose(sigmoid(math.log(3)), 0.75, rel_tol=1e-15)
    assert math.isclose(softplus(0.0), math.log(2), rel_tol=1e-15)
    assert math.isclose(softplus(math.log(3)), math.log(4), rel_tol=1e-15)
    assert math.isclose(silu(math.log(3)), 0.75 * math.log(3), rel_tol=1e-15)
    assert softplus(800.0) == 800.0 and softplus(-800.0) == 0.0
    assert sigmoid(-800.0) == 0.0 and sigmoid(800.0) == 1.0


def test_gates_closed_form_at_zero():
    # b = 0, a + dt_bias = 0, A_log = 0: beta = 1/2 and g = -ln 2 (catches a sign or a missing exp)
    B, L, H = 2, 3, 4
    beta, g = dn_gates(np.zeros((B, L, H)), np.full((B, L, H), 0.5), np.zeros(H), np.full(H, -0.5))
    assert np.all(beta == 0.5)
    assert np.allclose(g, -math.log(2), rtol=1e-15, atol=0)


def test_gates_decay_is_a_power_of_one_plus_exp():
    # e^g = (1 + e^{a + dt_bias})^(-e^{A_log}): pins the composition (exp of A_log, softplus of
    # the biased input, the minus sign) through an algebraically different form
    r = rng(1)
    B, L, H = 2, 5, 3
    a, b = r.normal(size=(B, L, H)), r.normal(size=(B, L, H))
    A_log, dt = r.normal(size=H) * 0.5, r.normal(size=H)
    beta, g = dn_gates(b, a, A_log, dt)
    want = (1.0 + np.exp(a + dt)) ** (-np.exp(A_log))
    assert np.allclose(np.exp(g), want, rtol=1e-13, atol=0)
    assert np.allclose(beta + sigmoid(-b), 1.0, rtol=0, atol=1e-15)   # sigmoid symmetry
    assert np.all(g < 0) and np.all((beta > 0) & (beta < 1))


def test_gates_per_head_parameters_follow_the_head_axis():
    # swapping two heads' parameters swaps exactly those heads' g (catches a head/token mixup)
    r = rng(2)
    a, b = r.normal(size=(1, 4, 3)), r.normal(size=(1, 4, 3))
    A_log, dt = np.array([0.1, -0.7, 1.2]), np.array([0.3, 0.0, -1.0])
    _, g = dn_gates(b, a, A_log, dt)
    a2 = a[..., [2, 1, 0]]
    _, g2 = dn_gates(b, a2, A_log[[2, 1, 0]], dt[[2, 1, 0]])
    assert np.array_equal(g2, g[..., [2, 1, 0]])


def test_gates_large_and_small_arguments():
    # softplus(x) -> x for large x and -> e^x for very negative x
    A_log, dt = np.array([0.0]), np.array([0.0])
    _, g = dn_gates(np.zeros((1, 2, 1)), np.array([[[40.0], [-40.0]]]), A_log, dt)
    assert math.isclose(g[0, 0, 0], -40.0, rel_tol=1e-15)
    assert math.isclose(g[0, 1, 0], -math.exp(-40.0), rel_tol=1e-12)


def test_gates_pads_are_exact_zeros():
    r = rng(3)
    a, b = r.normal(size=(3, 6, 2)), r.normal(size=(3, 6, 2))
    A_log, dt = r.normal(size=2), r.normal(size=2)
    lengths = [6, 2, 0]
    beta, g = dn_gates(b, a, A_log, dt, lengths)
    beta_all, g_all = dn_gates(b, a, A_log, dt)
    for bi, n in enumerate(lengths):
        assert np.all(beta[bi, n:] == 0) and np.all(g[bi, n:] == 0)
        assert np.array_equal(beta[bi, :n], beta_all[bi, :n]) and np.array_equal(g[bi, :n], g_all[bi, :n])


# ---------------------------------------------------------------- conv + SiLU
def conv_inputs(seed, B, L, Hk, Hv, D, K):
    r = rng(seed)
    Cm = (2 * Hk + Hv) * D
    return r.normal(size=(B, L, Cm)), r.normal(size=(B, K - 1, Cm)), r.normal(size=(Cm, K)) * 0.5


def join(q, k, v):
    B, L = q.shape[:2]
    return np.concatenate([q.reshape(B, L, -1), k.reshape(B, L, -1), v.reshape(B, L, -1)], -1)


def test_conv_matches_numpy_convolve():
    # np.convolve flips its second argument: the causal taps w[c, 0..K-1] multiply ext[t .. t+K-1],
    # so pre = convolve(ext, w[::-1], 'valid') (catches reversed taps or an off-by-one window)
    B, L, Hk, Hv, D, K = 2, 9, 1, 2, 4, 4
    mixed, tail, w = conv_inputs(4, B, L, Hk, Hv, D, K)
    q, k, v, _ = conv_silu(mixed, tail, w, Hk, Hv, D)
    out = join(q, k, v)
    ext = np.concatenate([tail, mixed], 1)
    for bi in range(B):
        for c in range(mixed.shape[2]):
            pre = np.convolve(ext[bi, :, c], w[c, ::-1], mode="valid")
            assert np.allclose(out[bi, :, c], pre / (1 + np.exp(-pre)), rtol=1e-13, atol=1e-15)


def test_conv_impulse_response_is_causal():
    # a unit input at (t0, c0) with a zero tail reaches outputs t0 .. t0 + K-1 of channel c0 only,
    # through w[c0, K-1], w[c0, K-2], ... (the last tap multiplies the current token)
    B, L, Hk, Hv, D, K, t0, c0 = 1, 10, 1, 1, 2, 4, 3, 5
    Cm = (2 * Hk + Hv) * D
    mixed = np.zeros((B, L, Cm))
    mixed[0, t0, c0] = 1.0
    w = np.arange(1, Cm * K + 1, dtype=np.float64).reshape(Cm, K) / 10.0
    q, k, v, _ = conv_silu(mixed, None, w, Hk, Hv, D)
    out = join(q, k, v)
    want = np.zeros((B, L, Cm))
    for s in range(t0, min(t0 + K, L)):
        want[0, s, c0] = silu(w[c0, K - 1 - (s - t0)])
    assert np.array_equal(out, want)


def test_conv_single_tap_is_elementwise():
    B, L, Hk, Hv, D = 2, 5, 1, 2, 4
    mixed, _, w = conv_inputs(5, B, L, Hk, Hv, D, 1)
    q, k, v, new_tail = conv_silu(mixed, None, w, Hk, Hv, D)
    assert np.allclose(join(q, k, v), silu(mixed * w[:, 0]), rtol=1e-15, atol=0)
    assert new_tail.shape == (B, 0, mixed.shape[2])


def test_conv_split_continuation():
    # one call over L1 + L2 tokens == a call over L1 then one over L2 that starts from the new tail
    # (catches a wrong tail gather or a tail applied at the wrong end)
    B, Hk, Hv, D, K, L1, L2 = 2, 1, 2, 4, 4, 7, 5
    mixed, tail, w = conv_inputs(6, B, L1 + L2, Hk, Hv, D, K)
    full = conv_silu(mixed, tail, w, Hk, Hv, D)
    a = conv_silu(mixed[:, :L1], tail, w, Hk, Hv, D)
    b = conv_silu(mixed[:, L1:], a[3], w, Hk, Hv, D)
    for i in range(3):
        assert np.allclose(np.concatenate([a[i], b[i]], 1), full[i], rtol=1e-13, atol=1e-15)
    assert np.array_equal(b[3], full[3])


def test_conv_tail_gather_short_rows():
    # new_tail = the last K-1 inputs up to the row's length, reaching into the old tail when the
    # row is shorter than K-1; a zero-length row keeps its tail
    B, L, Hk, Hv, D, K = 3, 6, 1, 1, 2, 4
    mixed, tail, w = conv_inputs(7, B, L, Hk, Hv, D, K)
    _, _, _, nt = conv_silu(mixed, tail, w, Hk, Hv, D, lengths=[6, 1, 0])
    assert np.array_equal(nt[0], mixed[0, 3:6])
    assert np.array_equal(nt[1], np.concatenate([tail[1, 1:], mixed[1, :1]]))
    assert np.array_equal(nt[2], tail[2])


def test_conv_channel_split():
    # q takes channels [0, Hk D), k the next Hk D, v the last Hv D, each reshaped head-major
    B, L, Hk, Hv, D = 1, 2, 2, 4, 3
    Cm = (2 * Hk + Hv) * D
    mixed = np.tile(np.arange(Cm, dtype=np.float64) / Cm, (B, L, 1))
    q, k, v, _ = conv_silu(mixed, None, np.ones((Cm, 1)), Hk, Hv, D)
    assert np.allclose(q[0, 0, 1, 2], silu((1 * D + 2) / Cm))
    assert np.allclose(k[0, 1, 0, 1], silu((Hk * D + 1) / Cm))
    assert np.allclose(v[0, 0, 3, 0], silu((2 * Hk * D + 3 * D) / Cm))


# ---------------------------------------------------------------- gated RMSNorm
def test_rmsnorm_constant_row():
    # x = c everywhere: x / sqrt(mean x^2 + eps) = c / sqrt(c^2 + eps)
    D, c, eps = 128, -0.3, 1e-6
    w = np.linspace(0.5, 1.5, D)
    z = np.full(D, math.log(3))
    y = gated_rmsnorm(np.full(D, c), z, w, eps)
    assert np.allclose(y, w * c / math.sqrt(c * c + eps) * 0.75 * math.log(3), rtol=1e-14, atol=0)


def test_rmsnorm_output_rms_is_the_gate():
    # eps = 0, w = 1, a constant gate z: the row's RMS is exactly silu(z) (catches sum for mean)
    x = rng(8).normal(size=(5, 128))
    z = np.full((5, 128), 2.0)
    y = gated_rmsnorm(x, z, np.ones(128), 0.0)
    assert np.allclose(np.sqrt((y * y).mean(-1)), silu(2.0), rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariant_and_zero_gate():
    r = rng(9)
    x, z, w = r.normal(size=(3, 128)), r.normal(size=(3, 128)), r.normal(size=128)
    assert np.allclose(gated_rmsnorm(7.5 * x, z, w, 0.0), gated_rmsnorm(x, z, w, 0.0), rtol=1e-13, atol=1e-15)
    assert np.all(gated_rmsnorm(x, np.zeros_like(z), w, 1e-6) == 0)

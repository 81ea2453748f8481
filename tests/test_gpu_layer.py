"""The layer steps around the delta rule (gdr_gates, gdr_conv_silu, gdr_gated_rmsnorm) vs the
float64 oracle, through the C ABI.

Tolerance, derived from the arithmetic: the kernels compute in float32 from the exact input
values and round each output once. A float32 output is then within a few float32 ulps of the
truth: max |gpu - oracle| / max |oracle| <= 1e-5. A bfloat16 output carries one rounding to 8
significant bits (relative error <= 2^-9) on top: the same ratio <= 4e-3, and every element
within 2^-8 of its own magnitude (plus 1e-6 absolute for values rounded near zero).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_gdr_amd as gdr
from oracle import conv_silu as conv_ref, dn_gates as gates_ref, gated_rmsnorm as norm_ref
from workloads import draw_layer
from gpu_helpers import rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 4e-3}


@pytest.fixture(autouse=True)
def _name_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def f64(t):
    return t.double().cpu().numpy()


def check(got, want, dtype, label):
    got = f64(got)
    e = rel_err(got, want)
    print(f"[parity] {label} rel={e:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert e <= TOL[dtype], (label, e)
    if dtype == torch.bfloat16:
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6), label


# ---------------------------------------------------------------- gates
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape,lengths", [((3, 130, 32), [130, 67, 0]), ((1, 1, 5), None), ((2, 4096, 32), [4096, 1])])
def test_gates_vs_oracle(dtype, shape, lengths):
    B, L, Hv = shape
    gen = torch.Generator("cpu").manual_seed(901 + L)
    b = torch.randn(B, L, Hv, generator=gen).to(dtype)
    a = torch.randn(B, L, Hv, generator=gen).to(dtype)
    A_log = torch.log(1 + 15 * torch.rand(Hv, generator=gen))
    dt = -2 + 0.5 * torch.randn(Hv, generator=gen)
    lens = None if lengths is None else torch.tensor(lengths, dtype=torch.int32)
    beta, g = gdr.gates(b.cuda(), a.cuda(), A_log.cuda(), dt.cuda(), None if lens is None else lens.cuda())
    torch.cuda.synchronize()
    assert beta.dtype == dtype and g.dtype == torch.float32
    beta_ref, g_ref = gates_ref(f64(b), f64(a), f64(A_log), f64(dt), None if lens is None else lens.numpy())
    check(beta, beta_ref, dtype, f"beta {shape} {dtype}")
    check(g, g_ref, torch.float32, f"g {shape} {dtype}")
    if lens is not None:   # pads are exact zeros
        for bi, n in enumerate(lengths):
            assert torch.all(beta[bi, n:] == 0) and torch.all(g[bi, n:] == 0)


def test_gates_bad_length_row_is_nan():
    b = torch.randn(2, 8, 4).cuda()
    a = torch.randn(2, 8, 4).cuda()
    lens = torch.tensor([8, 9], dtype=torch.int32).cuda()   # device-side: not checked on the host
    beta, g = gdr.gates(b, a, torch.zeros(4).cuda(), torch.zeros(4).cuda(), lens)
    torch.cuda.synchronize()
    assert torch.isfinite(beta[0]).all() and torch.isnan(beta[1]).all() and torch.isnan(g[1]).all()


def test_gates_full_size_long_prefill():
    # the long-prefill shape: B = 1, L = 16384, 32 value heads, bf16 projections
    x = draw_layer(1, 16384, 1, 32, 1, 951, torch.bfloat16, D=8)
    beta, g = gdr.gates(x.b_raw.cuda(), x.a_raw.cuda(), x.A_log.cuda(), x.dt_bias.cuda())
    torch.cuda.synchronize()
    beta_ref, g_ref = gates_ref(f64(x.b_raw), f64(x.a_raw), f64(x.A_log), f64(x.dt_bias))
    check(beta, beta_ref, torch.bfloat16, "beta full")
    check(g, g_ref, torch.float32, "g full")


# ---------------------------------------------------------------- conv + SiLU
def run_conv(x, Hk, Hv, tail=True, lengths=None, **kw):
    lens = None if lengths is None else torch.tensor(lengths, dtype=torch.int32).cuda()
    out = gdr.conv_silu(x.mixed.cuda(), x.conv_w.cuda(), Hk, Hv, x.tail.cuda() if tail else None, lens, **kw)
    torch.cuda.synchronize()
    return out


def conv_oracle(x, Hk, Hv, tail=True, lengths=None):
    return conv_ref(f64(x.mixed), f64(x.tail) if tail else None, f64(x.conv_w), Hk, Hv, 128, lengths)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,L,Hk,Hv,K,lengths", [
    (2, 200, 2, 4, 4, [200, 131]),     # several tiles, ragged last tile, ragged row
    (3, 5, 1, 2, 4, [5, 2, 0]),        # shorter than a tile; rows shorter than K-1; an empty row
    (1, 64, 1, 1, 1, None),            # a single tap: no tail
    (2, 77, 1, 2, 8, None),            # the widest filter
    (1, 130, 16, 32, 4, None),         # the model's channel count
])
def test_conv_vs_oracle(dtype, B, L, Hk, Hv, K, lengths):
    x = draw_layer(B, L, Hk, Hv, K, 960 + L + K, dtype, lengths=lengths)
    q, k, v, nt = run_conv(x, Hk, Hv, lengths=lengths)
    rq, rk, rv, rnt = conv_oracle(x, Hk, Hv, lengths=lengths)
    check(q, rq, dtype, f"conv q {B},{L},{Hk},{Hv},{K}")
    check(k, rk, dtype, "conv k")
    check(v, rv, dtype, "conv v")
    assert nt.shape == (B, K - 1, (2 * Hk + Hv) * 128)
    if K > 1:   # the tail is a gather: bit-exact
        assert np.array_equal(f64(nt), rnt)


def test_conv_no_tail_is_zero_history():
    x = draw_layer(2, 70, 1, 2, 4, 971, torch.float32)
    q, k, v, nt = run_conv(x, 1, 2, tail=False)
    rq, rk, rv, rnt = conv_oracle(x, 1, 2, tail=False)
    check(q, rq, torch.float32, "no-tail q")
    check(v, rv, torch.float32, "no-tail v")
    assert np.array_equal(f64(nt), rnt)


def test_conv_in_place_tail_and_chained_calls():
    # two chained calls with the tail updated in place equal one call over both halves
    x = draw_layer(2, 150, 1, 2, 4, 972, torch.bfloat16)
    mixed, w, tail = x.mixed.cuda(), x.conv_w.cuda(), x.tail.cuda().clone()
    full = gdr.conv_silu(mixed, w, 1, 2, tail.clone())
    a = gdr.conv_silu(mixed[:, :70].contiguous(), w, 1, 2, tail, new_tail=tail)
    b = gdr.conv_silu(mixed[:, 70:].contiguous(), w, 1, 2, tail, new_tail=tail)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(torch.cat([a[i], b[i]], 1), full[i])
    assert torch.equal(tail, full[3])


def test_conv_empty_sequence_carries_tail():
    x = draw_layer(2, 0, 1, 2, 4, 973, torch.float32)
    q, k, v, nt = run_conv(x, 1, 2)
    assert q.shape[1] == 0 and torch.equal(nt.cpu(), x.tail)


def test_conv_bad_length_row_gets_nan_tail():
    x = draw_layer(2, 10, 1, 2, 4, 974, torch.float32)
    lens = torch.tensor([10, 11], dtype=torch.int32).cuda()
    q, k, v, nt = gdr.conv_silu(x.mixed.cuda(), x.conv_w.cuda(), 1, 2, x.tail.cuda(), lens)
    torch.cuda.synchronize()
    assert torch.isfinite(nt[0]).all() and torch.isnan(nt[1]).all()


def test_conv_full_size_long_prefill_sampled():
    # the long-prefill shape (B = 1, L = 16384, 16 key / 32 value heads, K = 4, bf16), checked on
    # windows of tokens the oracle computes from the preceding K-1 inputs (exact by continuation)
    Hk, Hv, K, L = 16, 32, 4, 16384
    x = draw_layer(1, L, Hk, Hv, K, 975, torch.bfloat16)
    q, k, v, nt = run_conv(x, Hk, Hv)
    mixed = f64(x.mixed)
    for t0 in (0, 61, 4096, 9000, L - 16):
        n = 16
        tail = f64(x.tail) if t0 == 0 else mixed[:, t0 - K + 1:t0]
        rq, rk, rv, _ = conv_ref(mixed[:, t0:t0 + n], tail, f64(x.conv_w), Hk, Hv, 128)
        check(q[:, t0:t0 + n], rq, torch.bfloat16, f"full q @{t0}")
        check(k[:, t0:t0 + n], rk, torch.bfloat16, f"full k @{t0}")
        check(v[:, t0:t0 + n], rv, torch.bfloat16, f"full v @{t0}")
    assert np.array_equal(f64(nt), mixed[:, L - K + 1:])


# ---------------------------------------------------------------- gated RMSNorm
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,L,Hv", [(2, 130, 4), (1, 1, 1), (1, 3, 3)])
def test_rmsnorm_vs_oracle(dtype, B, L, Hv):
    x = draw_layer(B, L, 1, Hv, 1, 980 + L + Hv, dtype)
    y = gdr.gated_rmsnorm(x.x.cuda(), x.z.cuda(), x.norm_w.cuda(), 1e-6)
    torch.cuda.synchronize()
    check(y, norm_ref(f64(x.x), f64(x.z), f64(x.norm_w), 1e-6), dtype, f"norm {B},{L},{Hv} {dtype}")


def test_rmsnorm_in_place_and_eps():
    x = draw_layer(1, 40, 1, 8, 1, 985, torch.bfloat16)
    buf = (x.x * 1e-3).cuda()   # small rows, where eps matters
    want = norm_ref(f64(buf), f64(x.z), f64(x.norm_w), 1e-5)
    y = gdr.gated_rmsnorm(buf, x.z.cuda(), x.norm_w.cuda(), 1e-5, out=buf)
    torch.cuda.synchronize()
    assert y.data_ptr() == buf.data_ptr()
    check(buf, want, torch.bfloat16, "norm in place")


def test_rmsnorm_full_size_long_prefill_sampled():
    x = draw_layer(1, 16384, 1, 32, 1, 986, torch.bfloat16)
    y = gdr.gated_rmsnorm(x.x.cuda(), x.z.cuda(), x.norm_w.cuda(), 1e-6)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(16384 * 32, 4096, replace=False)
    xr, zr = f64(x.x).reshape(-1, 128)[rows], f64(x.z).reshape(-1, 128)[rows]
    check(y.reshape(-1, 128)[torch.as_tensor(rows)], norm_ref(xr, zr, f64(x.norm_w), 1e-6), torch.bfloat16,
          "norm full sampled")

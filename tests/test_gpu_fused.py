"""gdr_prefill_ex (gate prologue and gated RMSNorm fused into the prefill) vs the float64 oracle,
through the C ABI.

Oracle: oracle.dn_gates -> oracle.gated_delta_rule -> oracle.gated_rmsnorm on the same inputs
(the layer order of the model page, model.py, _linear_layer). Bar: the delta rule's, on the
fused result: max |gpu - oracle| / max |oracle| <= 1e-4 for float32 inputs and <= 2e-2 for
bfloat16 inputs, on the output and on the final state. The normalised output divides each
(token, head) row by its own RMS, so its error is the row's relative error of o, which for a
row much smaller than the largest can exceed the global ratio; row by row (each row's max
|difference| over that row's max |truth|) the check is a bug detector instead: ROW_TOL, far
below the O(1) error of a dropped, misplaced or wrongly scaled row sum.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_gdr_amd as gdr
from oracle import dn_gates, gated_delta_rule, gated_rmsnorm
from workloads import draw, draw_layer
from gpu_helpers import TOL, rel_err

pytestmark = pytest.mark.gpu

ROW_TOL = {torch.float32: 1e-3, torch.bfloat16: 0.1}


@pytest.fixture(autouse=True)
def _name_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def f64(t):
    return None if t is None else t.double().cpu().numpy()


def layer_inputs(B, L, Hk, Hv, dtype, seed, lengths=None, s0_rows=0, raw_dtype=None):
    x = draw(B, L, Hk, Hv, 128, "R1", seed, dtype, lengths=lengths, s0_rows=s0_rows)
    y = draw_layer(B, L, 1, Hv, 1, seed + 1, raw_dtype or dtype, D=128)
    return x, y


def oracle(x, y, gates, norm, eps=1e-6, heads=None):
    lens = None if x.lengths is None else x.lengths.numpy()
    if gates:
        beta, g = dn_gates(f64(y.b_raw), f64(y.a_raw), f64(y.A_log), f64(y.dt_bias), lens)
    else:
        beta, g = f64(x.beta), f64(x.g)
    o, s = gated_delta_rule(f64(x.q), f64(x.k), f64(x.v), g, beta, lengths=lens, s0=f64(x.s0),
                            s0_row=None if x.s0_row is None else x.s0_row.numpy(), heads=heads)
    if norm:
        z = f64(y.x) if heads is None else f64(y.x)[:, :, heads]
        o = gated_rmsnorm(o, z, f64(y.norm_w), eps)
    return o, s


def run(x, y, gates, norm, eps=1e-6):
    d = lambda t: None if t is None else t.cuda()
    kw = {}
    if gates:
        kw["gates"] = (d(y.b_raw), d(y.a_raw), d(y.A_log), d(y.dt_bias))
    if norm:
        kw["norm"] = (d(y.x).to(x.v.dtype), d(y.norm_w), eps)   # y.x serves as the gate z
    o, s = gdr.prefill(d(x.q), d(x.k), d(x.v), None if gates else d(x.g), None if gates else d(x.beta),
                       valid=d(x.lengths), s0=d(x.s0), **kw)
    torch.cuda.synchronize()
    return o, s


def check(o, s, o_ref, s_ref, dtype, label, heads=None):
    o, s = f64(o), f64(s)
    if heads is not None:
        o, s = o[:, :, heads], s[:, heads]
    tol = TOL[dtype]
    e_o, e_s = rel_err(o, o_ref), rel_err(s, s_ref)
    rows = (np.abs(o - o_ref).max(-1) / np.maximum(np.abs(o_ref).max(-1), 1e-30)).max()
    print(f"[parity] {label} o={e_o:.3e} rows={rows:.3e} S={e_s:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert e_o <= tol and e_s <= tol, (label, e_o, e_s)
    return rows


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gates,norm", [(True, False), (False, True), (True, True)])
def test_fused_vs_oracle(dtype, gates, norm):
    # several chunks, a ragged last chunk, ragged rows and an initial state
    x, y = layer_inputs(2, 200, 2, 4, dtype, 1100, lengths=[200, 77], s0_rows=2)
    o, s = run(x, y, gates, norm)
    o_ref, s_ref = oracle(x, y, gates, norm)
    rows = check(o, s, o_ref, s_ref, dtype, f"fused gates={gates} norm={norm} {dtype}")
    if norm:
        assert rows <= ROW_TOL[dtype]


def test_fused_gates_float32_projections_with_bf16_qkv():
    x, y = layer_inputs(1, 130, 1, 2, torch.bfloat16, 1110, raw_dtype=torch.float32)
    o, s = run(x, y, True, False)
    o_ref, s_ref = oracle(x, y, True, False)
    check(o, s, o_ref, s_ref, torch.bfloat16, "fused gates fp32 raw")


def test_fused_pads_are_no_ops():
    # the fused gates make pads exact no-ops: garbage raw projections past each length change nothing
    x, y = layer_inputs(2, 150, 1, 2, torch.bfloat16, 1120, lengths=[150, 40])
    o1, s1 = run(x, y, True, True)
    y.b_raw[1, 40:] = 7.0
    y.a_raw[1, 40:] = -9.0
    o2, s2 = run(x, y, True, True)
    assert torch.equal(s1, s2) and torch.equal(o1[:, :40], o2[:, :40]) and torch.equal(o1[0], o2[0])


def test_fused_norm_eps_and_small_outputs():
    # strong decay keeps o small; a large eps then dominates the row RMS
    x, y = layer_inputs(1, 100, 1, 2, torch.bfloat16, 1130)
    o, s = run(x, y, False, True, eps=0.5)
    o_ref, s_ref = oracle(x, y, False, True, eps=0.5)
    check(o, s, o_ref, s_ref, torch.bfloat16, "fused norm eps=0.5")


def test_fused_long_prefill_sampled_heads():
    # the long-prefill shape (B = 1, L = 16384, 16 key / 32 value heads, bf16; segment-parallel
    # scan), both fusions, on sampled value heads
    x = draw(1, 16384, 16, 32, 128, "LONG", 1140, torch.bfloat16)
    y = draw_layer(1, 16384, 1, 32, 1, 1141, torch.bfloat16, D=128)
    o, s = run(x, y, True, True)
    heads = [0, 13, 31]
    o_ref, s_ref = oracle(x, y, True, True, heads=heads)
    rows = check(o, s, o_ref, s_ref, torch.bfloat16, "fused long heads", heads=heads)
    assert rows <= ROW_TOL[torch.bfloat16]


def test_fused_equals_unfused_composition_float32():
    # float32: the fused norm is the same kernel run in place after the scan, so fused and composed
    # results agree to rounding
    x, y = layer_inputs(2, 90, 1, 2, torch.float32, 1150, lengths=[90, 31])
    o, _ = run(x, y, False, True)
    o_plain, _ = run(x, y, False, False)
    comp = gdr.gated_rmsnorm(o_plain, y.x.cuda(), y.norm_w.cuda(), 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(o, comp)


# ---------------------------------------------------------------- gdr_decode_ex
def run_decode(x, y, gates, norm, eps=1e-6):
    d = lambda t: None if t is None else t.cuda()
    kw = {}
    if gates:
        kw["gates"] = (d(y.b_raw), d(y.a_raw), d(y.A_log), d(y.dt_bias))
    if norm:
        kw["norm"] = (d(y.x).to(x.v.dtype), d(y.norm_w), eps)
    o, s = gdr.decode(d(x.q), d(x.k), d(x.v), None if gates else d(x.g), None if gates else d(x.beta),
                      valid=d(x.lengths), s0=d(x.s0), s0_row=d(x.s0_row), **kw)
    torch.cuda.synchronize()
    return o, s


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L", [1, 5, 64])
def test_fused_decode_vs_oracle(dtype, L):
    x, y = layer_inputs(3, L, 2, 4, dtype, 1160 + L, lengths=[L, max(L - 2, 0), 0], s0_rows=3)
    o, s = run_decode(x, y, True, True)
    o_ref, s_ref = oracle(x, y, True, True)
    rows = check(o, s, o_ref, s_ref, dtype, f"fused decode L={L} {dtype}")
    assert rows <= ROW_TOL[dtype]


def test_fused_decode_fork_rows():
    # a decode step of 64 fork rows that all continue one shared state row, both fusions
    x = draw(64, 1, 16, 32, 128, "R1", 1170, torch.bfloat16, s0_rows=1, s0_row=[0] * 64)
    y = draw_layer(64, 1, 1, 32, 1, 1171, torch.bfloat16, D=128)
    o, s = run_decode(x, y, True, True)
    rows = [0, 17, 63]
    lens = None
    beta, g = dn_gates(f64(y.b_raw)[rows], f64(y.a_raw)[rows], f64(y.A_log), f64(y.dt_bias), lens)
    o_ref, s_ref = gated_delta_rule(f64(x.q)[rows], f64(x.k)[rows], f64(x.v)[rows], g, beta,
                                    s0=f64(x.s0), s0_row=np.zeros(len(rows), dtype=np.int64))
    o_ref = gated_rmsnorm(o_ref, f64(y.x)[rows], f64(y.norm_w), 1e-6)
    check(o[rows], s[rows], o_ref, s_ref, torch.bfloat16, "fused decode fork rows")


def test_fused_decode_equals_fused_prefill():
    # the two entry points compute the same thing; in float32 they agree to accumulated rounding
    x, y = layer_inputs(2, 70, 1, 2, torch.float32, 1180, lengths=[70, 33], s0_rows=2)
    o1, s1 = run_decode(x, y, True, True)
    o2, s2 = run(x, y, True, True)
    assert rel_err(f64(o1), f64(o2)) <= 1e-5 and rel_err(f64(s1), f64(s2)) <= 1e-5

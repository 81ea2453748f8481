"""The token-by-token entry point (gdr_decode) vs the float64 oracle, through the C ABI.

Same bar as the prefill: max |o_gpu - o_oracle| / max |o_oracle| <= 1e-4 for float32 inputs and
<= 2e-2 for bfloat16 inputs, and the same ratio for the final state. The workloads are the
decode steps and short fork continuations of the fork model: many rows, a few tokens each,
states gathered by row index and continued in place.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_gdr_amd as gdr
from workloads import draw
from gpu_helpers import TOL, compare, rel_err, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def run_decode(x, **kw):
    d = to_dev(x)
    o, s = gdr.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], valid=d["lengths"], s0=d["s0"],
                      s0_row=d["s0_row"], **kw)
    torch.cuda.synchronize()
    return o, s


def check(x, o, s, label=""):
    tol = TOL[x.q.dtype]
    e_all, e_valid, e_s = compare(x, o, s, label=label)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert e_all <= tol and e_valid <= tol and e_s <= tol, (e_all, e_valid, e_s)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L", [1, 2, 7, 64])
def test_decode_vs_oracle(dtype, L):
    x = draw(3, L, 2, 4, 128, "R1", 700 + L, dtype, lengths=[L, max(L - 1, 0), 0], s0_rows=3)
    o, s = run_decode(x)
    check(x, o, s, label=f"decode L={L} {dtype}")


def test_decode_fork_rows_shared_state():
    # 64 fork rows, one token each, every row continuing from the same prefix state (s0_row = 0)
    x = draw(64, 1, 16, 32, 128, "R1", 777, torch.bfloat16, s0_rows=1, s0_row=[0] * 64)
    o, s = run_decode(x)
    check(x, o, s, label="fork decode B=64 L=1 shared s0")


@pytest.mark.parametrize("regime", ["R2", "R3", "R4"])
def test_decode_regimes(regime):
    x = draw(2, 5, 1, 2, 128, regime, 720, torch.float32, s0_rows=2)
    o, s = run_decode(x)
    check(x, o, s, label=f"decode {regime}")


def test_decode_equals_prefill():
    x = draw(4, 9, 2, 4, 128, "R2", 731, torch.float32, lengths=[9, 4, 1, 0], s0_rows=4)
    od, sd = run_decode(x)
    op, sp = run_gpu(x)
    assert rel_err(od.cpu(), op.cpu()) <= 1e-5 and rel_err(sd.cpu(), sp.cpu()) <= 1e-5


def test_decode_in_place_continuation():
    x = draw(2, 3, 1, 2, 128, "R1", 741, torch.float32, s0_rows=2)
    d = to_dev(x)
    state = d["s0"].clone()
    o, s = gdr.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=state, s_final=state)
    torch.cuda.synchronize()
    assert s.data_ptr() == state.data_ptr()
    check(x, o, s, label="decode in place")


def test_decode_steps_chain_to_one_call():
    # three single-token steps, each continuing the previous state in place, equal one 3-token call
    x = draw(2, 3, 2, 4, 128, "R1", 751, torch.float32, s0_rows=2)
    d = to_dev(x)
    state = d["s0"].clone()
    outs = []
    for t in range(3):
        sl = lambda a: a[:, t:t + 1].contiguous()
        o, _ = gdr.decode(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), s0=state, s_final=state)
        outs.append(o)
    torch.cuda.synchronize()
    o_all, s_all = run_decode(x)
    assert rel_err(torch.cat(outs, 1).cpu(), o_all.cpu()) <= 1e-6 and rel_err(state.cpu(), s_all.cpu()) <= 1e-6


def test_decode_bad_row_index_gives_nan_rows():
    x = draw(3, 2, 1, 2, 128, "R1", 761, torch.float32, s0_rows=2, s0_row=[0, 5, 1])
    d = to_dev(x)
    o, s = gdr.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], s0_row=d["s0_row"])
    torch.cuda.synchronize()
    assert torch.isnan(o[1]).all() and torch.isnan(s[1]).all()
    assert torch.isfinite(o[0]).all() and torch.isfinite(o[2]).all()

"""gdr_prefill_noalloc (the prefill with the library's device-resident workspace, for callers that
cannot allocate) against gdr_prefill with a workspace of the caller's, through the C ABI, on an
MI355X. Both run the same kernels on the same inputs, so the results must agree to the oracle
parity bar (max |difference| / max |reference| <= 2e-2 for bf16, 1e-4 for float32); they are in
fact expected to be identical. Two calls in a row, the second on a smaller input (the array keeps
the first call's contents, which the second must not depend on), then a float32 call, then a shape
whose workspace exceeds the array, which must be rejected before anything runs.
"""
import ctypes

import pytest
import torch

import gated_deltanet_prefill_gdr_amd as gdr
from workloads import draw
from gpu_helpers import TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def both(x):
    d = to_dev(x)
    B, L, Hk, Hv, Dk, Dv = x.shape
    o_ref, s_ref = gdr.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], valid=d["lengths"], s0=d["s0"],
                               s0_row=d["s0_row"])
    o = torch.full_like(o_ref, float("nan"))
    s = torch.full_like(s_ref, float("nan"))
    gdr.prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], valid=d["lengths"], s0=d["s0"],
                        s0_row=d["s0_row"], out=o, s_final=s)
    torch.cuda.synchronize()
    return o, s, o_ref, s_ref


def agree(x, label):
    o, s, o_ref, s_ref = both(x)
    tol = TOL[x.q.dtype]
    eo = rel_err(o.double().cpu().numpy(), o_ref.double().cpu().numpy())
    es = rel_err(s.double().cpu().numpy(), s_ref.double().cpu().numpy())
    same = torch.equal(o, o_ref) and torch.equal(s, s_ref)
    print(f"[noalloc] {label}: o {eo:.3e} S {es:.3e} identical={same}", flush=True)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert eo <= tol and es <= tol


def test_noalloc_two_calls_second_smaller():
    # segments, truncated starts, 16 key / 32 value heads, 4096 tokens (about 26 MB of workspace)
    agree(draw(1, 4096, 16, 32, 128, "LONG", 901, torch.bfloat16), "bf16 L=4096 32 heads")
    # a smaller one right after: ragged rows, an initial state, fewer heads
    agree(draw(2, 700, 2, 4, 128, "R1", 902, torch.bfloat16, lengths=[700, 333], s0_rows=2), "bf16 ragged small")


def test_noalloc_float32():
    agree(draw(1, 300, 2, 4, 128, "R2", 903, torch.float32, s0_rows=1), "f32 L=300")


def test_noalloc_rejects_oversized_workspace():
    desc = gdr.make_desc(4, 16384, 16, 32, 0, True, False)   # about 400 MB of workspace
    assert gdr.workspace_size(desc) > (128 << 20)
    st = gdr.library().gdr_prefill_noalloc(ctypes.byref(desc), *([None] * 10), None)
    assert st == -2 and "workspace" in gdr.last_error(), gdr.last_error()

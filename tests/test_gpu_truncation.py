"""Truncated segment starts against the float64 oracle, through the C ABI, on an MI355X.

For bf16 sequences cut into segments, the state entering a segment may be taken from the last few
chunks of the segment before it, run from zero, when their decay bounds the dropped term by 2^-40
of the state where that window starts; a finalize pass checks the carried bound against the measured
state norms and reruns a (row, head) in one piece where it exceeds 2^-24. These tests check the results against the oracle on both paths, and read the status word (the
number of (row, head) pairs rerun) and the plan entries from the workspace.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_gdr_amd as gdr
from workloads import CONFIGS, draw
from gpu_helpers import TOL, compare, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.set_truncation(True)
    yield
    gdr.set_truncation(True)


def seg_plan(B, Hv, NC):
    """Segments per (row, head) and chunks per segment, as the library cuts bf16 sequences."""
    P = min(NC, max(1, -(-256 // (B * Hv))))
    Ls = -(-NC // P)
    return -(-NC // Ls), Ls


def run(x, in_place=False):
    """Prefill through the binding with a workspace of our own, filled with NaN bytes first (so that
    reading a slot no kernel of the call wrote spoils the results); returns o, s_final, the status word
    and the per-(row, head) truncation flags (None without segments)."""
    d = to_dev(x)
    B, L, Hk, Hv, Dk, Dv = x.shape
    desc = gdr.make_desc(B, L, Hk, Hv, 0 if x.s0 is None else x.s0.shape[0], True, False)
    ws = torch.full((gdr.workspace_size(desc),), 0xFF, device="cuda", dtype=torch.uint8)
    kw = {}
    if in_place:
        kw["s_final"] = d["s0"]
    o, s = gdr.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], valid=d["lengths"], s0=d["s0"],
                       s0_row=d["s0_row"], workspace=ws, **kw)
    torch.cuda.synchronize()
    off = gdr.status_offset(desc)
    if off is None:
        return o, s, None, None
    wsc = ws.cpu()
    status = int(wsc[off:off + 4].view(torch.int32)[0])
    P, _ = seg_plan(B, Hv, -(-L // 64))
    plan = wsc[off + 256: off + 256 + B * Hv * P * 16].view(torch.int32).view(B, Hv, P, 4)
    trunc = plan[:, :, 1, 2].numpy().astype(bool) if P > 1 else None
    return o, s, status, trunc


def check(x, o, s, label, heads=None, rows=None):
    tol = TOL[x.q.dtype]
    e_all, e_valid, e_s = compare(x, o, s, rows=rows, heads=heads, label=label)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert e_all <= tol and e_valid <= tol and e_s <= tol, (e_all, e_valid, e_s)


def test_long_prefill_truncated_all_heads():
    """The long prefill (L = 16384, 32 value heads, g ~ -U(0, 0.5)): every head takes the truncated
    path, none is rerun, and all 32 heads match the oracle."""
    x = CONFIGS[5].draw()
    o, s, status, trunc = run(x)
    assert status == 0 and trunc.all(), (status, trunc)
    check(x, o, s, "long prefill truncated, all heads")


def test_long_prefill_exact_all_heads():
    """The same workload with truncation switched off: the exact segment transitions and combine."""
    x = CONFIGS[5].draw()
    gdr.set_truncation(False)
    o, s, status, trunc = run(x)
    assert not trunc.any()
    check(x, o, s, "long prefill exact, all heads")


def test_weak_decay_takes_exact_path():
    """g ~ -0.02 U(0, 1): no window within the 2-chunk segments here decays by 2^-40, so no head is
    truncated."""
    x = draw(1, 4096, 4, 8, 128, "R2", 811, torch.bfloat16)
    o, s, status, trunc = run(x)
    assert not trunc.any()
    check(x, o, s, "weak decay bf16 L=4096")


@pytest.mark.parametrize("regime,seed", [("LONG", 821), ("R2", 822)])
def test_long_sequence_many_segments(regime, seed):
    """L = 65536 on two value heads: 128 segments of 8 chunks, far past the benchmark shapes in sequence
    length and segment count. LONG: every boundary takes a window; R2 (weak decay): the exact path, whose
    combine chains 127 segment maps. Every output and the final states against the oracle."""
    x = draw(1, 65536, 1, 2, 128, regime, seed, torch.bfloat16)
    assert seg_plan(1, 2, 1024) == (128, 8)
    o, s, status, trunc = run(x)
    assert status == 0
    assert trunc.all() if regime == "LONG" else not trunc.any(), trunc
    check(x, o, s, f"L=65536, 128 segments, {regime}")


def test_exact_path_from_shared_s0_rows():
    """Weak decay (the exact path) with initial states: three rows start from two s0 rows, so the combine
    chains the segment maps from s0 rows shared between batch rows."""
    x = draw(3, 2048, 2, 4, 128, "R2", 817, torch.bfloat16, s0_rows=2, s0_row=[1, 0, 1])
    o, s, status, trunc = run(x)
    assert not trunc.any() and status == 0
    check(x, o, s, "exact path from shared s0 rows")


def test_exact_path_in_place():
    """Weak decay with s_final written over s0: the combine chains the segment maps from the copy of s0
    it keeps in slot 0, and the last segment overwrites s0 with the final state."""
    x = draw(2, 2048, 2, 4, 128, "R2", 818, torch.bfloat16, s0_rows=2)
    o, s, status, trunc = run(x, in_place=True)
    assert not trunc.any() and status == 0
    check(x, o, s, "exact path in place")


def test_medium_decay_long_windows():
    """g ~ -U(0.03, 0.05) (about 3.7 in log2 per chunk): a boundary needs a window of about 11 chunks to
    decay by 2^-40, longer than one batch of plan loads (8) and within the 16-chunk segments here
    (B Hv = 32: 8 segments)."""
    x = draw(4, 8192, 4, 8, 128, "LONG", 823, torch.bfloat16)
    gen = torch.Generator().manual_seed(9)
    x.g = (-(0.03 + 0.02 * torch.rand(x.g.shape, generator=gen))).contiguous()
    assert seg_plan(4, 8, 128) == (8, 16)
    o, s, status, trunc = run(x)
    assert trunc.all() and status == 0, (trunc, status)
    check(x, o, s, "medium decay, long windows", rows=[0, 3], heads=[0, 7])


@pytest.mark.parametrize("lo,width,truncated", [(0.027, 0.002, True), (0.0136, 0.0002, True), (0.012, 0.0005, False)])
def test_window_limit(lo, width, truncated):
    """The long prefill's shape (8 segments of 32 chunks) with g ~ -U(lo, lo + width): windows of 16
    chunks (two batches of plan loads), of 32 (four batches; the whole segment before the boundary, the
    longest allowed: every head truncated) and of 36 (past it: every head takes the exact path), the
    window lengths worked out from the drawn gates beforehand."""
    x = draw(1, 16384, 16, 32, 128, "LONG", 824, torch.bfloat16)
    gen = torch.Generator().manual_seed(10)
    x.g = (-(lo + width * torch.rand(x.g.shape, generator=gen))).contiguous()
    assert seg_plan(1, 32, 256) == (8, 32)
    o, s, status, trunc = run(x)
    assert status == 0
    assert trunc.all() if truncated else not trunc.any(), trunc
    check(x, o, s, f"window limit, g ~ -U({lo:.3f}, {lo + width:.3f})", heads=[0, 31])


def test_mixed_heads():
    """Heads with strong decay are truncated, heads without decay are not, in one call."""
    x = draw(1, 2048, 2, 4, 128, "LONG", 812, torch.bfloat16)
    g = x.g.clone()
    g[:, :, 0] = -(0.5 + 0.5 * torch.rand(g[:, :, 0].shape, generator=torch.Generator().manual_seed(5)))
    g[:, :, 2] = -(0.5 + 0.5 * torch.rand(g[:, :, 2].shape, generator=torch.Generator().manual_seed(6)))
    g[:, :, 1] = 0.0
    g[:, :, 3] = -1e-3
    x.g = g.contiguous()
    o, s, status, trunc = run(x)
    assert trunc[0].tolist() == [True, False, True, False], trunc
    assert status == 0
    check(x, o, s, "mixed heads")


def test_certificate_failure_reruns():
    """A state 1e8 times larger just before a boundary's window than after it: the a-priori decay
    test passes (2^-44 per chunk) but the measured bound does not, so the finalize pass reruns
    that (row, head) in one piece; results match the oracle."""
    B, L, Hk, Hv = 1, 1024, 1, 2
    x = draw(B, L, Hk, Hv, 128, "LONG", 813, torch.bfloat16)
    gen = torch.Generator().manual_seed(7)
    x.g = (-(0.48 + 0.02 * torch.rand(B, L, Hv, generator=gen))).contiguous()   # about 2^-44 per chunk
    v = x.v.float()
    v[:, 64 * 6:64 * 7] *= 1e4    # chunk 6: large values
    v[:, 64 * 7:] *= 1e-4         # from chunk 7 on: small ones
    x.v = v.to(torch.bfloat16).contiguous()
    o, s, status, trunc = run(x)
    assert trunc.all() and status == 2, (trunc, status)
    check(x, o, s, "certificate failure rerun")


def test_in_place_with_truncation_and_rerun():
    """s_final written over s0: the rerun starts from the copy of s0 the combine keeps in slot 0."""
    B, L, Hk, Hv = 2, 1024, 1, 2
    x = draw(B, L, Hk, Hv, 128, "LONG", 814, torch.bfloat16, s0_rows=B)
    gen = torch.Generator().manual_seed(8)
    x.g = (-(0.48 + 0.02 * torch.rand(B, L, Hv, generator=gen))).contiguous()
    v = x.v.float()
    v[1, 64 * 6:64 * 7] *= 1e4    # row 1 fails its certificate, row 0 does not
    v[1, 64 * 7:] *= 1e-4
    x.v = v.to(torch.bfloat16).contiguous()
    o, s, status, trunc = run(x, in_place=True)
    assert trunc.all() and status == 2, (trunc, status)
    check(x, o, s, "in place, truncated and rerun")


def test_ragged_rows_with_segments():
    """Rows whose boundaries fall in their right pads are not truncated; the others are."""
    x = draw(2, 1024, 1, 2, 128, "R1", 815, torch.bfloat16, lengths=[1024, 300], s0_rows=2)
    o, s, status, trunc = run(x)
    assert trunc[0].all() and not trunc[1].any(), trunc
    assert status == 0
    check(x, o, s, "ragged rows with segments")


def test_fused_norm_with_truncation():
    """The fused gated RMSNorm of the output pass on the truncated path (long shape, sampled heads)."""
    import oracle
    from workloads import draw_layer
    x = CONFIGS[5].draw()
    y = draw_layer(1, x.q.shape[1], 1, 32, 1, 816, torch.bfloat16)
    d = to_dev(x)
    z, nw = y.x.cuda(), y.norm_w.cuda()
    o, s = gdr.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], norm=(z, nw, 1e-6))
    torch.cuda.synchronize()
    heads = [0, 13, 31]
    o_ref, s_ref = oracle.gated_delta_rule(x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy(),
                                           x.g.double().numpy(), x.beta.double().numpy(), heads=heads)
    n_ref = oracle.gated_rmsnorm(o_ref, y.x.double().numpy()[:, :, heads], y.norm_w.double().numpy(), 1e-6)
    got = o.double().cpu().numpy()[:, :, heads]
    err = np.abs(got - n_ref).max() / np.abs(n_ref).max()
    es = np.abs(s.double().cpu().numpy()[:, heads] - s_ref).max() / np.abs(s_ref).max()
    print(f"[parity] fused norm truncated: o {err:.3e} S {es:.3e}", flush=True)
    assert err <= 2e-2 and es <= 2e-2


def test_fused_norm_exact_path():
    """The fused gated RMSNorm of the output pass on the exact path (segment maps combined), with s0."""
    import oracle
    from workloads import draw_layer
    x = draw(1, 2048, 2, 8, 128, "R2", 819, torch.bfloat16, s0_rows=1)
    y = draw_layer(1, x.q.shape[1], 1, 8, 1, 820, torch.bfloat16)
    d = to_dev(x)
    z, nw = y.x.cuda(), y.norm_w.cuda()
    gdr.set_truncation(False)
    o, s = gdr.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], norm=(z, nw, 1e-6))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gated_delta_rule(x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy(),
                                           x.g.double().numpy(), x.beta.double().numpy(),
                                           s0=x.s0.double().numpy())
    n_ref = oracle.gated_rmsnorm(o_ref, y.x.double().numpy(), y.norm_w.double().numpy(), 1e-6)
    err = np.abs(o.double().cpu().numpy() - n_ref).max() / np.abs(n_ref).max()
    es = np.abs(s.double().cpu().numpy() - s_ref).max() / np.abs(s_ref).max()
    print(f"[parity] fused norm exact: o {err:.3e} S {es:.3e}", flush=True)
    assert err <= 2e-2 and es <= 2e-2

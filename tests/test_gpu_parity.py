"""HIP path vs the float64 oracle, through the C ABI, on an MI355X.

Bar: max |o_gpu - o_oracle| / max |o_oracle| <= 1e-4 for float32 inputs and <= 2e-2 for
bfloat16 inputs, over all positions and over valid positions only; the same ratio for the
final state. Large workloads are checked on sampled rows / heads (each (row, value head) is an
independent recurrence, so the oracle on a subset is exact).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_gdr_amd as gdr
from workloads import CONFIGS, draw
from gpu_helpers import TOL, compare, run_gpu, run_oracle, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def check(x, o, s, rows=None, heads=None, label=""):
    tol = TOL[x.q.dtype]
    e_all, e_valid, e_s = compare(x, o, s, rows=rows, heads=heads, label=label)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert e_all <= tol and e_valid <= tol and e_s <= tol, (e_all, e_valid, e_s)


# ------------------------------------------------------------------ the five workloads
@pytest.mark.parametrize("i", [1, 2, 3])
def test_config_full(i):
    x = CONFIGS[i].draw()
    o, s = run_gpu(x)
    check(x, o, s, label=CONFIGS[i].name)


def test_config4_forks_sampled_rows():
    x = CONFIGS[4].draw()
    o, s = run_gpu(x)
    lens = x.lengths.numpy()
    rows = sorted({int(lens.argmin()), int(lens.argmax()), 0, 33})
    check(x, o, s, rows=rows, label=f"{CONFIGS[4].name} rows={rows}")


def test_config4_forks_all_rows():
    x = CONFIGS[4].draw()
    o, s = run_gpu(x)
    check(x, o, s, label=f"{CONFIGS[4].name} all 64 rows")


def test_config5_long_sampled_heads():
    x = CONFIGS[5].draw()
    o, s = run_gpu(x)
    heads = [0, 1, 17, 31]
    check(x, o, s, heads=heads, label=f"{CONFIGS[5].name} heads={heads}")


# ------------------------------------------------------------------ shapes and tails
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 130, 200, 333])
def test_lengths_and_tails(dtype, L):
    x = draw(2, L, 2, 4, 128, "R1", 300 + L, dtype, lengths=[L, max(L // 2, 1) - 1 if L > 1 else 0],
             s0_rows=2)
    o, s = run_gpu(x)
    check(x, o, s, label=f"L={L} {dtype}")


@pytest.mark.parametrize("regime", ["R2", "R3", "R4", "LONG"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_regimes(regime, dtype):
    x = draw(1, 256, 2, 4, 128, regime, 400, dtype, s0_rows=1 if regime == "R4" else 0)
    o, s = run_gpu(x)
    check(x, o, s, label=f"{regime} {dtype}")


def test_no_head_sharing_and_ratio_4():
    for Hk, Hv in ((3, 3), (1, 4)):
        x = draw(1, 150, Hk, Hv, 128, "R1", 500 + Hv, torch.bfloat16, s0_rows=1)
        o, s = run_gpu(x)
        check(x, o, s, label=f"Hk={Hk} Hv={Hv}")


def test_odd_value_heads_per_key_head():
    # the bf16 prep forms the records of a key head's value heads two at a time: an odd count
    # leaves one head alone (3 = pair + single; 5 = a batch of four gates, then one more)
    for Hk, Hv, seed in ((2, 6, 514), (1, 5, 515)):
        x = draw(2, 200, Hk, Hv, 128, "R1", seed, torch.bfloat16, lengths=[200, 90], s0_rows=2)
        o, s = run_gpu(x)
        check(x, o, s, label=f"Hk={Hk} Hv={Hv}")


def test_eight_value_heads_per_key_head():
    # more than four value heads share a key head: the prep forms their records in two batches
    # of gates (both dtypes, with ragged rows and initial states)
    for dtype in (torch.bfloat16, torch.float32):
        x = draw(2, 150, 1, 8, 128, "R1", 511, dtype, lengths=[150, 70], s0_rows=2)
        o, s = run_gpu(x)
        check(x, o, s, label=f"Hk=1 Hv=8 {dtype}")


def test_bf16_beta():
    x = draw(1, 200, 2, 4, 128, "R1", 501, torch.bfloat16)
    x.beta = x.beta.to(torch.bfloat16)
    o, s = run_gpu(x)
    check(x, o, s, label="bf16 beta")


# ------------------------------------------------------------------ edge cases
def test_zero_length_rows_keep_state():
    x = draw(3, 100, 2, 4, 128, "R1", 502, torch.float32, lengths=[0, 100, 0], s0_rows=3)
    o, s = run_gpu(x)
    check(x, o, s, label="zero-length rows")
    assert torch.equal(s[0].cpu(), x.s0[0]) and torch.equal(s[2].cpu(), x.s0[2])


def test_bf16_padded_segments():
    # many chunks past the row lengths, spread over the segments of the bf16 scan: whole pad
    # segments (identity transitions), a segment that starts in the pad, and a zero-length row
    x = draw(3, 700, 2, 4, 128, "R1", 508, torch.bfloat16, lengths=[700, 0, 129], s0_rows=3)
    o, s = run_gpu(x)
    check(x, o, s, label="bf16 padded segments")


def test_bf16_ragged_rows():
    # sixteen ragged rows, some empty, one full: the chunk list of the prep, the pad loop of the
    # output pass and the row-to-workgroup mapping together
    lens = [200, 3, 64, 65, 0, 128, 199, 1, 150, 77, 100, 190, 12, 129, 63, 180]
    x = draw(16, 200, 1, 2, 128, "R1", 509, torch.bfloat16, lengths=lens, s0_rows=16)
    o, s = run_gpu(x)
    check(x, o, s, label="bf16 ragged rows")


def test_bf16_many_ragged_rows():
    # 300 ragged rows: the prep's chunk list is built over two blocks of 256 rows; rows on both
    # sides of the block boundary, an empty one and a full one are checked against the oracle
    rng = np.random.default_rng(510)
    lens = rng.integers(0, 131, size=300).tolist()
    lens[255], lens[256], lens[257] = 0, 130, 1
    x = draw(300, 130, 1, 2, 128, "R1", 510, torch.bfloat16, lengths=lens, s0_rows=300)
    o, s = run_gpu(x)
    check(x, o, s, rows=[0, 1, 254, 255, 256, 257, 299], label="bf16 300 ragged rows")


def test_empty_sequence_copies_state():
    x = draw(2, 0, 2, 4, 128, "R1", 503, torch.float32, s0_rows=2)
    o, s = run_gpu(x)
    assert o.shape == (2, 0, 4, 128)
    assert torch.equal(s.cpu(), x.s0)


def test_empty_batch():
    x = draw(0, 64, 2, 4, 128, "R1", 504, torch.bfloat16)
    o, s = run_gpu(x)
    assert o.shape == (0, 64, 4, 128) and s.shape == (0, 4, 128, 128)


def test_out_of_range_device_indices_give_nan_rows():
    import gated_deltanet_prefill_gdr_amd as gdr
    x = draw(3, 70, 1, 2, 128, "R1", 505, torch.bfloat16, s0_rows=2)
    dev = "cuda"
    lengths = torch.tensor([70, 71, 5], dtype=torch.int32, device=dev)        # row 1 invalid
    s0_row = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)           # row 2 invalid
    o, s = gdr.prefill(x.q.to(dev), x.k.to(dev), x.v.to(dev), x.g.to(dev), x.beta.to(dev), valid=lengths,
                       s0=x.s0.to(dev), s0_row=s0_row)
    torch.cuda.synchronize()
    assert torch.isnan(o[1].float()).all() and torch.isnan(s[1]).all()
    assert torch.isnan(o[2].float()).all() and torch.isnan(s[2]).all()
    assert torch.isfinite(o[0].float()).all() and torch.isfinite(s[0]).all()


def test_valid_mask_equals_lengths():
    x = draw(2, 150, 2, 4, 128, "R1", 506, torch.bfloat16, lengths=[150, 77])
    o1, s1 = run_gpu(x)
    import gated_deltanet_prefill_gdr_amd as gdr
    mask = (torch.arange(150)[None] < x.lengths[:, None]).float().cuda()
    o2, s2 = gdr.prefill(x.q.cuda(), x.k.cuda(), x.v.cuda(), x.g.cuda(), x.beta.cuda(), valid=mask)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ------------------------------------------------------------------ properties
def test_deterministic_bitwise():
    x = draw(2, 300, 2, 4, 128, "R1", 507, torch.bfloat16, lengths=[300, 123], s0_rows=2)
    o1, s1 = run_gpu(x)
    o2, s2 = run_gpu(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_batch_invariance_bitwise():
    # A row's result does not depend on the other rows of the batch (fork rows).
    x = draw(5, 256, 2, 4, 128, "R1", 508, torch.bfloat16, lengths=[256, 40, 200, 1, 129], s0_rows=1,
             s0_row=[0] * 5)
    o, s = run_gpu(x)
    for b in (1, 3):
        xb = draw(5, 256, 2, 4, 128, "R1", 508, torch.bfloat16, lengths=[256, 40, 200, 1, 129], s0_rows=1,
                  s0_row=[0] * 5)
        for n in ("q", "k", "v", "g", "beta", "lengths", "s0_row"):
            setattr(xb, n, getattr(xb, n)[b:b + 1].contiguous())
        ob, sb = run_gpu(xb)
        assert torch.equal(ob[0], o[b]) and torch.equal(sb[0], s[b])


@pytest.mark.parametrize("B", [64, 128])
def test_row_order_invariance_bitwise(B):
    """Without segments (B Hv >= 256) ragged rows are taken longest first, ties in any order, by the
    single-head pass (B = 64) or the pair pass (B = 128): a row's results do not depend on the run nor
    on where the row sits in the batch."""
    gen = torch.Generator().manual_seed(3)
    lens = [int(v) for v in torch.randint(1, 1025, (B,), generator=gen)]
    lens[:8] = [1024, 1024, 64, 64, 1, 1, 700, 700]   # ties
    x = draw(B, 1024, 2, 4, 128, "R1", 510, torch.bfloat16, lengths=lens, s0_rows=B)
    o1, s1 = run_gpu(x)
    o2, s2 = run_gpu(x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    perm = torch.randperm(B, generator=gen)
    xp = draw(B, 1024, 2, 4, 128, "R1", 510, torch.bfloat16, lengths=lens, s0_rows=B)
    for n in ("q", "k", "v", "g", "beta", "lengths", "s0"):
        setattr(xp, n, getattr(xp, n)[perm].contiguous())
    op, sp = run_gpu(xp)
    assert torch.equal(op, o1[perm]) and torch.equal(sp, s1[perm])


def test_pad_garbage_is_ignored():
    kw = dict(lengths=[200, 90], s0_rows=2)
    x = draw(2, 200, 2, 4, 128, "R1", 509, torch.bfloat16, **kw)
    y = draw(2, 200, 2, 4, 128, "R1", 509, torch.bfloat16, zero_pads=False, **kw)
    assert not torch.equal(x.beta, y.beta)
    o1, s1 = run_gpu(x)
    o2, s2 = run_gpu(y)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_head_pairs_identical():
    x = draw(1, 200, 2, 4, 128, "R1", 510, torch.bfloat16)
    x.v[:, :, 1::2] = x.v[:, :, 0::2]
    x.g[:, :, 1::2] = x.g[:, :, 0::2]
    x.beta[:, :, 1::2] = x.beta[:, :, 0::2]
    o, s = run_gpu(x)
    assert torch.equal(o[:, :, 0::2], o[:, :, 1::2]) and torch.equal(s[:, 0::2], s[:, 1::2])


# ------------------------------------------------------------------ value-head pairs
# Without segments and with B Hv / 2 >= 256, the bf16 output pass runs the two value heads of a key head
# in one workgroup (each column with the single-head pass's arithmetic, in the same order). A batch that
# takes it must equal, bit for bit, the same rows run in halves, which are too few for the pair pass.
PAIR_KW = dict(lengths=[200, 0, 64, 65, 1, 130, 199, 128] * 4, s0_rows=3, s0_row=[0, 1, 2] * 10 + [1, 0])


def _rows(x, lo, hi):
    """Rows lo .. hi - 1 of x (the same initial-state rows)."""
    from dataclasses import replace
    return replace(x, **{n: getattr(x, n)[lo:hi].contiguous()
                         for n in ("q", "k", "v", "g", "beta", "lengths", "s0_row")})


def test_pair_pass_equals_single_head_pass_bitwise():
    x = draw(32, 200, 4, 16, 128, "R1", 520, torch.bfloat16, **PAIR_KW)   # 32 x 8 pairs: the pair pass
    o, s = run_gpu(x)
    for lo in (0, 16):   # 16 x 16 heads: 128 pairs, the single-head pass, still without segments
        oh, sh = run_gpu(_rows(x, lo, lo + 16))
        assert torch.equal(oh, o[lo:lo + 16]) and torch.equal(sh, s[lo:lo + 16]), lo


def test_pair_pass_against_oracle():
    x = draw(32, 200, 4, 16, 128, "R1", 521, torch.bfloat16, **PAIR_KW)
    o, s = run_gpu(x)
    rows = [0, 1, 2, 3, 4, 7, 29, 31]   # full, empty, one chunk, ragged, one token, ...
    check(x, o, s, rows=rows, label=f"pair pass rows={rows}")


def test_pair_pass_nan_rows():
    import gated_deltanet_prefill_gdr_amd as gdr
    x = draw(32, 200, 4, 16, 128, "R1", 522, torch.bfloat16, **PAIR_KW)
    dev = "cuda"
    lengths = x.lengths.clone()
    lengths[5] = 201                   # past L: a bad row
    s0_row = x.s0_row.clone()
    s0_row[9] = 3                      # past the state rows: a bad row
    o, s = gdr.prefill(x.q.to(dev), x.k.to(dev), x.v.to(dev), x.g.to(dev), x.beta.to(dev),
                       valid=lengths.to(dev), s0=x.s0.to(dev), s0_row=s0_row.to(dev))
    ref_o, ref_s = run_gpu(x)
    torch.cuda.synchronize()
    for b in (5, 9):
        assert torch.isnan(o[b].float()).all() and torch.isnan(s[b]).all(), b
    good = [b for b in range(32) if b not in (5, 9)]
    assert torch.equal(o[good], ref_o[good]) and torch.equal(s[good], ref_s[good])


def test_split_continuation():
    x = draw(1, 320, 2, 4, 128, "R2", 511, torch.float32, s0_rows=1)
    o, s = run_gpu(x)
    cut = 130   # not a chunk boundary
    xa = draw(1, 320, 2, 4, 128, "R2", 511, torch.float32, s0_rows=1)
    xb = draw(1, 320, 2, 4, 128, "R2", 511, torch.float32, s0_rows=1)
    for n in ("q", "k", "v", "g", "beta"):
        setattr(xa, n, getattr(x, n)[:, :cut].contiguous())
        setattr(xb, n, getattr(x, n)[:, cut:].contiguous())
    oa, sa = run_gpu(xa)
    xb.s0 = sa.cpu()
    ob, sb = run_gpu(xb)
    assert rel_err(torch.cat([oa, ob], 1).cpu().numpy(), o.cpu().numpy()) < 1e-4
    assert rel_err(sb.cpu().numpy(), s.cpu().numpy()) < 1e-4


def test_joint_linearity_2_pow_8():
    # Scaling (v, S0) by 2^8 scales (o, S_final) by 2^8; power-of-two scaling commutes with
    # every rounding on the path, so the GPU result scales exactly.
    x = draw(1, 200, 2, 4, 128, "R2", 512, torch.bfloat16, s0_rows=1)   # nothing subnormal
    o1, s1 = run_gpu(x)
    x.v = x.v * 256
    x.s0 = x.s0 * 256
    o2, s2 = run_gpu(x)
    assert torch.equal(o2, o1 * 256) and torch.equal(s2, s1 * 256)


def test_in_place_state_continuation():
    import gated_deltanet_prefill_gdr_amd as gdr
    x = draw(2, 100, 2, 4, 128, "R1", 513, torch.float32, s0_rows=2)
    o_ref, s_ref = run_gpu(x)
    st = x.s0.cuda()
    o, s = gdr.prefill(x.q.cuda(), x.k.cuda(), x.v.cuda(), x.g.cuda(), x.beta.cuda(), s0=st, s_final=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)


def test_kernel_timing_records_both_kernels():
    import gated_deltanet_prefill_gdr_amd as gdr
    x = draw(1, 256, 2, 4, 128, "R1", 514, torch.bfloat16)
    gdr.timing_enable(True)
    try:
        run_gpu(x)
        run_gpu(x)
        t = gdr.timing_read()
    finally:
        gdr.timing_enable(False)
    assert t["gdr_prep"][1] == 2 and t["gdr_scan"][1] == 2
    assert t["gdr_prep"][0] > 0 and t["gdr_scan"][0] > 0


def test_graph_capture_replays_equal_eager():
    # the library launches only kernels (no allocation, no memset), so a call can be captured in a
    # HIP graph; every replay, with eager work and synchronisations in between, equals the eager call
    x = draw(1, 1000, 2, 4, 128, "R1", 1201, torch.bfloat16, s0_rows=1)
    d = to_dev(x)
    B, L, Hk, Hv, D, Dv = x.shape
    o = torch.empty(B, L, Hv, Dv, device="cuda", dtype=torch.bfloat16)
    sf = torch.empty(B, Hv, D, Dv, device="cuda")
    desc = gdr.make_desc(B, L, Hk, Hv, 1, True, False)
    ws = torch.empty(gdr.workspace_size(desc), device="cuda", dtype=torch.uint8)
    step = lambda: gdr.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], out=o, s_final=sf, workspace=ws)
    step()
    torch.cuda.synchronize()
    o_ref, s_ref = o.clone(), sf.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        o.zero_()
        sf.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(sf, s_ref), f"replay {i}"

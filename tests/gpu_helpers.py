"""Shared helpers for the GPU tests: run the HIP path through the binding, run the oracle on
the same inputs, and compare with the max-relative-error metric of the kernel-test page
(max |difference| / max |truth|, function main's summary)."""
import numpy as np
import torch

import gated_deltanet_prefill_gdr_amd as gdr
from oracle import gated_delta_rule

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to_dev(x, dev="cuda"):
    return {n: (None if t is None else t.to(dev)) for n, t in
            (("q", x.q), ("k", x.k), ("v", x.v), ("g", x.g), ("beta", x.beta), ("lengths", x.lengths),
             ("s0", x.s0), ("s0_row", x.s0_row))}


def run_gpu(x, dev="cuda", **kw):
    d = to_dev(x, dev)
    o, s = gdr.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], valid=d["lengths"], s0=d["s0"],
                       s0_row=d["s0_row"], **kw)
    torch.cuda.synchronize()
    return o, s


def run_oracle(x, rows=None, heads=None):
    return gated_delta_rule(x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy(),
                            x.g.double().numpy(), x.beta.double().numpy(),
                            lengths=None if x.lengths is None else x.lengths.numpy(),
                            s0=None if x.s0 is None else x.s0.double().numpy(),
                            s0_row=None if x.s0_row is None else x.s0_row.numpy(), rows=rows, heads=heads)


def rel_err(got, want, mask=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if mask is not None:
        got, want = got[mask], want[mask]
    if want.size == 0:
        return 0.0
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-30))


def valid_mask(x, rows=None):
    """[B', L] bool: positions before each row's length."""
    B, L = x.q.shape[:2]
    lens = np.full(B, L) if x.lengths is None else x.lengths.numpy()
    if rows is not None:
        lens = lens[np.asarray(rows)]
    return np.arange(L)[None, :] < lens[:, None]


def compare(x, o_gpu, s_gpu, rows=None, heads=None, label=""):
    """Oracle on the selected rows/heads; returns (err_o_all, err_o_valid, err_s)."""
    o_ref, s_ref = run_oracle(x, rows=rows, heads=heads)
    o = o_gpu.double().cpu().numpy()
    s = s_gpu.double().cpu().numpy()
    if rows is not None:
        o, s = o[rows], s[rows]
    if heads is not None:
        o, s = o[:, :, heads], s[:, heads]
    m = valid_mask(x, rows)
    e_all = rel_err(o, o_ref)
    e_valid = rel_err(o, o_ref, mask=m)
    e_s = rel_err(s, s_ref)
    print(f"[parity] {label} o(all)={e_all:.3e} o(valid)={e_valid:.3e} S={e_s:.3e}", flush=True)
    return e_all, e_valid, e_s

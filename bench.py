"""Benchmark of the chunked gated delta rule prefill on one MI355X.

One step = one gdr_prefill call (all its kernels: the per-chunk prep, the segment transitions and
their combine, the output scan) over the long-prefill workload: B = 1, 16 key / 32 value heads, Dk = Dv = 128, L = 16384,
bf16 q/k/v, fp32 g/beta/state, zero initial state, final state returned. Inputs, outputs and
the workspace are resident in HBM before the timed region. Before the W warm-up steps the step
runs untimed for 0.3 s so that the GPU's clocks have settled. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --decode          # one fork decode step instead (gdr_decode, 64 rows x 1 token)
  python bench.py --layer           # the layer steps around it (gates, conv + SiLU, gated RMSNorm)
  python bench.py --fused           # the prefill with the gate prologue and gated RMSNorm fused in
  python bench.py --all-configs     # every named workload: median call time, throughput, rooflines,
                                    # per-kernel times (--config N for one of them)
  python bench.py --copy-probe      # a plain device copy of known size, for HBM counter scaling
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated-delta prefill tokens·heads/s and % MFMA roofline at L=16384, H=32, D=128"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3    # fp32 matrix
CHUNK, D = 64, 128


def algorithmic(B, L, Hk, Hv, esz, n_s0, want_state):
    """Algorithmic bytes and flops of one call (the whole path).

    Bytes: read q, k, v, g, beta, s0 (if any), lengths; write o and s_final (if wanted).
    Flops per (token, value head): 6 D^2 + 10 C D (the chunked method counted with full 64x64
    tiles: W S, Q S, K^T Delta over the state, plus Gram, W, U, Q K^T, P Delta within a chunk).
    """
    units = B * L * Hv
    nbytes = (2 * B * L * Hk * D * esz          # q, k
              + 2 * B * L * Hv * D * esz        # v, o
              + 2 * B * L * Hv * 4              # g, beta (fp32)
              + n_s0 * Hv * D * D * 4
              + (B * Hv * D * D * 4 if want_state else 0))
    flops = units * (6 * D * D + 10 * CHUNK * D)
    return units, nbytes, flops


def kernel_bytes(name, B, L, Hk, Hv, esz, P, fused=False):
    """Bytes a kernel of the path must read and write through its own interface, one launch.

    Intermediates count where they cross HBM: the per-chunk record (T diag(beta) in q's dtype,
    for float32 also the decayed scores, then 8 x 64 fp32 scalars) and the segment slots
    (128 x 256 fp32 each).
    """
    NC = (L + CHUNK - 1) // CHUNK
    rec = (1 if esz == 2 else 2) * 6 * 512 * esz + 8 * CHUNK * 4
    rec_tb = 6 * 512 * esz + 8 * CHUNK * 4          # the part the transitions read
    slot = D * 2 * D * 4
    qk = B * L * Hk * D * esz
    vo = B * L * Hv * D * esz
    gb = 2 * B * L * Hv * 4
    recs = B * Hv * NC * rec
    frac = (P - 1) / P if P > 1 else 0.0                 # share of chunks in the first P-1 segments
    if fused:   # raw bf16 gate projections read by the prep, the gate z by the output pass
        gb = 2 * B * L * Hv * 2
    if name == "gdr_prep":
        return 2 * qk + gb + recs
    if name == "gdr_transition":
        return frac * (qk + vo + B * Hv * NC * rec_tb) + B * Hv * (P - 1) * slot
    if name == "gdr_combine":
        return B * Hv * (P - 1) * (slot * 3 // 2) + B * Hv * P * slot // 2
    if name == "gdr_scan":
        return (2 * qk + 2 * vo + recs + B * Hv * D * D * 4 + (B * Hv * P * slot // 2 if P > 1 else 0)
                + (vo if fused else 0))
    if name == "gdr_gated_rmsnorm":   # o and z read, o written
        return 3 * vo
    raise KeyError(name)


def seg_plan(B, Hv, NC, bf16=True):
    """Number of segments the library cuts each (row, head) into (mirrors the C side)."""
    if not bf16 or NC <= 1:
        return 1
    P = min(NC, max(1, -(-256 // (B * Hv))))
    Ls = -(-NC // P)
    return -(-NC // Ls)


def source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_prefill_gdr_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


_CPU_X = None   # the inputs of the CPU baseline, shared with its forked worker processes


def _oracle_pair(bh):
    """Worker: the float64 oracle on one (row, value head) of _CPU_X; returns its CPU seconds."""
    from threadpoolctl import threadpool_limits
    from oracle import gated_delta_rule
    b, h = bh
    x = _CPU_X
    t0 = time.process_time()
    with threadpool_limits(limits=1):
        gated_delta_rule(x["q"], x["k"], x["v"], x["g"], x["beta"], lengths=x["lengths"], s0=x["s0"],
                         s0_row=x["s0_row"], rows=[b], heads=[h])
    return time.process_time() - t0


def cpu_workers():
    """Worker processes for the oracle: one per host core this process may use, at most 16 (a
    one-GPU share of the GPU machine's host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, pairs=None):
    """The float64 oracle as it stands, over the (row, value head) pairs of the workload (all of them
    unless `pairs` is given), one worker process per host core, each pair's token loop inside one
    process; wall time end to end. Must run before this process touches the GPU (the workers are
    forked)."""
    import multiprocessing as mp
    import numpy as np
    global _CPU_X
    B, L, Hk, Hv = x.q.shape[0], x.q.shape[1], x.q.shape[2], x.v.shape[2]
    _CPU_X = {"q": x.q.double().numpy(), "k": x.k.double().numpy(), "v": x.v.double().numpy(),
              "g": x.g.double().numpy(), "beta": x.beta.double().numpy(),
              "lengths": None if x.lengths is None else x.lengths.numpy(),
              "s0": None if x.s0 is None else x.s0.double().numpy(),
              "s0_row": None if x.s0_row is None else x.s0_row.numpy()}
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hv)]
    workers = min(cpu_workers(), len(pairs))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        cpu_s = sum(pool.map(_oracle_pair, pairs, chunksize=1))
    wall = time.perf_counter() - t0
    _CPU_X = None
    units = len(pairs) * L
    return {"value": units / wall, "unit": "tokens·heads/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(pairs)} of {B * Hv} (row, value head) pairs, all {L} tokens each, float64 numpy, "
                      f"{workers} processes x 1 thread, {wall:.1f} s wall, {cpu_s:.1f} s CPU",
            "cpu_model": cpu_model(), "numpy": np.__version__, "wall_s": wall, "cpu_s": cpu_s}


def copy_probe(nbytes=1 << 30, reps=3):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes, "reps": reps}))


def settle(step, seconds=0.3):
    """Run the step untimed until `seconds` have passed: the GPU's clocks ramp up over the first
    tens of milliseconds of load, and the few warm-up steps alone (a few ms) do not get there.
    Measured on the long prefill: 317-325 us per step right after 10 warm-up steps, 282 us once
    the clocks have settled; the step's work is the same."""
    import torch
    t0 = time.perf_counter()
    while seconds > 0 and time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()


def run_timed(step, steps):
    """Time `steps` calls of step(): first with nothing but two events around the loop (the step
    time), then again with the library's per-kernel HIP events on (kernel averages; those events
    sit between the kernels, so they are kept out of the step time)."""
    import torch
    import gated_deltanet_prefill_gdr_amd as gdr
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    gdr.timing_enable(True)
    gdr.timing_read()                      # drop anything recorded before
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = gdr.timing_read()
    gdr.timing_enable(False)
    return ms, kern


def bench_decode(a):
    """One decode step of the fork workload: every row continues its own state by one token, in
    place (s_final is s0). Bound by the state read and write; the token rows are tiny."""
    import torch
    import gated_deltanet_prefill_gdr_amd as gdr
    from workloads import draw
    B, L, Hk, Hv = a.rows, 1, 16, 32
    x = draw(B, L, Hk, Hv, D, "R1", 4242, torch.bfloat16, s0_rows=B)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v, g, beta, s0 = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta, x.s0))
    o = torch.empty(B, L, Hv, D, device=dev, dtype=v.dtype)
    fused = {}
    if a.fused:   # raw gate projections in place of g and beta, and the gated RMSNorm of o
        from workloads import draw_layer
        y = draw_layer(B, L, 1, Hv, 1, 4343, torch.bfloat16, D=D)
        fused = {"gates": tuple(t.to(dev) for t in (y.b_raw, y.a_raw, y.A_log, y.dt_bias)),
                 "norm": (y.x.to(dev), y.norm_w.to(dev), 1e-6)}
        g = beta = None

    def step():
        gdr.decode(q, k, v, g, beta, s0=s0, out=o, s_final=s0, **fused)

    settle(step, a.settle)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ms, kern = run_timed(step, a.steps)
    k_ms = kern["gdr_decode"][0] / max(kern["gdr_decode"][1], 1)
    units, nbytes, _ = algorithmic(B, L, Hk, Hv, 2, B, True)
    achieved = nbytes / (k_ms * 1e-3) / 1e9
    line = {
        "metric": "gated-delta fork decode step tokens·heads/s (64 rows x 1 token, H=32, D=128)"
                  + (", gate prologue and gated RMSNorm fused" if a.fused else ""),
        "value": units / (ms * 1e-3), "unit": "tokens·heads/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, beta~U(0.2,0.9), g~-U(0.05,3), state 0.1 N(0,1))",
        "config": {"workload": f"fork decode B={B} L=1 Hk={Hk} Hv={Hv} Dk=Dv=128 bf16 q/k/v, per-row fp32 "
                               "state continued in place", "B": B, "L": L, "Hk": Hk, "Hv": Hv, "D": D},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "gdr_decode",
                     "kernel_bytes": nbytes, "kernel_ms": k_ms},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def layer_bytes(B, L, Hk, Hv, K, esz):
    """Algorithmic bytes of one launch of each layer step (read inputs once, write outputs once)."""
    tok, Cm = B * L, (2 * Hk + Hv) * D
    return {
        "gdr_gates": tok * Hv * (2 * esz + esz + 4) + 2 * Hv * 4 + B * 4,
        "gdr_conv_silu": 2 * tok * Cm * esz + 2 * B * (K - 1) * Cm * esz + Cm * K * 4,
        "gdr_gated_rmsnorm": 3 * tok * Hv * D * esz + D * 4,
    }


def bench_layer(a):
    """The layer steps at the long-prefill shape (B = 1, L = 16384, 16 key / 32 value heads, K = 4,
    bf16): one step = gates + conv + SiLU (with the tail carried) + gated RMSNorm, each its own launch."""
    import torch
    import gated_deltanet_prefill_gdr_amd as gdr
    from workloads import draw_layer
    B, L, Hk, Hv, K = 1, 16384, 16, 32, 4
    x = draw_layer(B, L, Hk, Hv, K, 5151, torch.bfloat16)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t = {n: getattr(x, n).to(dev) for n in ("b_raw", "a_raw", "A_log", "dt_bias", "mixed", "tail", "conv_w", "x",
                                             "z", "norm_w")}
    beta = torch.empty(B, L, Hv, device=dev, dtype=torch.bfloat16)
    g = torch.empty(B, L, Hv, device=dev, dtype=torch.float32)
    q = torch.empty(B, L, Hk, D, device=dev, dtype=torch.bfloat16)
    k, v = torch.empty_like(q), torch.empty(B, L, Hv, D, device=dev, dtype=torch.bfloat16)
    new_tail, y = torch.empty_like(t["tail"]), torch.empty_like(t["x"])

    def step():
        gdr.gates(t["b_raw"], t["a_raw"], t["A_log"], t["dt_bias"], beta_out=beta, g_out=g)
        gdr.conv_silu(t["mixed"], t["conv_w"], Hk, Hv, t["tail"], out=(q, k, v), new_tail=new_tail)
        gdr.gated_rmsnorm(t["x"], t["z"], t["norm_w"], 1e-6, out=y)

    settle(step, a.settle)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ms, kern = run_timed(step, a.steps)
    kern = {n: (t / c, c) for n, (t, c) in kern.items() if c > 0}
    nb = layer_bytes(B, L, Hk, Hv, K, 2)
    per = {n: {"ms": kern[n][0], "bytes": nb[n], "GB/s": nb[n] / (kern[n][0] * 1e-3) / 1e9,
               "frac": nb[n] / (kern[n][0] * 1e-3) / 1e9 / HBM_PEAK_GBS} for n in nb}
    dom = max(per, key=lambda n: per[n]["ms"])
    line = {
        "metric": "gated-delta layer steps (gates, conv + SiLU, gated RMSNorm) tokens·heads/s at L=16384, H=32",
        "value": B * L * Hv / (ms * 1e-3), "unit": "tokens·heads/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) projections, mixed, z; U(-1,1)/2 conv taps)",
        "config": {"workload": "layer steps B=1 L=16384 Hk=16 Hv=32 D=128 K=4 bf16", "B": B, "L": L, "Hk": Hk,
                   "Hv": Hv, "K": K},
        "roofline": {"bound": "hbm", "achieved": per[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": per[dom]["frac"], "traffic": None, "kernel": dom, "kernel_bytes": nb[dom],
                     "kernel_ms": per[dom]["ms"]},
        "kernels": per,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_all_configs(a):
    """Every named workload of workloads.CONFIGS: median call time over 50 calls after 10 warm-up calls
    (HIP events around each call, inputs resident), throughput, TFLOP/s, algorithmic GB/s and
    both roofline fractions. One JSON line per config; a report, not the step metric."""
    import statistics
    import torch
    import gated_deltanet_prefill_gdr_amd as gdr
    from workloads import CONFIGS
    which = sorted(a.config) if a.config else sorted(CONFIGS)
    cpu = {}
    if not a.no_cpu_baseline:   # every config's oracle time first: its workers are forked
        for i in which:
            cpu[i] = cpu_baseline(CONFIGS[i].draw())
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    for i in which:
        x = CONFIGS[i].draw()
        B, L, Hk, Hv, Dk, Dv = x.shape
        esz = 2 if x.q.dtype == torch.bfloat16 else 4
        t = {n: (None if v is None else v.to(dev)) for n, v in
             (("q", x.q), ("k", x.k), ("v", x.v), ("g", x.g), ("beta", x.beta), ("lengths", x.lengths),
              ("s0", x.s0), ("s0_row", x.s0_row))}
        o = torch.empty(B, L, Hv, Dv, device=dev, dtype=x.v.dtype)
        sf = torch.empty(B, Hv, Dk, Dv, device=dev, dtype=torch.float32)
        n_s0 = 0 if x.s0 is None else x.s0.shape[0]
        desc = gdr.make_desc(B, L, Hk, Hv, n_s0, esz == 2, False)
        ws = torch.empty(max(gdr.workspace_size(desc), 1), device=dev, dtype=torch.uint8)

        def step():
            gdr.prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], valid=t["lengths"], s0=t["s0"],
                        s0_row=t["s0_row"], out=o, s_final=sf, workspace=ws)

        settle(step, a.settle)
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
        for e0, e1 in ev:
            e0.record()
            step()
            e1.record()
        torch.cuda.synchronize()
        ms = statistics.median(e0.elapsed_time(e1) for e0, e1 in ev)
        gdr.timing_enable(True)   # per-kernel averages, in a loop of their own
        gdr.timing_read()
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        kern = {n: t / c for n, (t, c) in gdr.timing_read().items() if c > 0}
        gdr.timing_enable(False)
        units, nbytes, flops = algorithmic(B, L, Hk, Hv, esz, n_s0, True)
        nbytes += 4 * B if x.lengths is not None else 0
        valid_units = units if x.lengths is None else int(x.lengths.sum()) * Hv
        peak = MFMA_BF16_PEAK_TFLOPS if esz == 2 else MFMA_FP32_PEAK_TFLOPS
        line = {"config": i, "workload": CONFIGS[i].name, "dtype": "bf16" if esz == 2 else "f32",
                "us": ms * 1e3, "tokens_heads_per_s": units / (ms * 1e-3),
                "valid_tokens_heads_per_s": valid_units / (ms * 1e-3), "tflops": flops / (ms * 1e-3) / 1e12,
                "alg_GBs": nbytes / (ms * 1e-3) / 1e9, "mfma_frac": flops / (ms * 1e-3) / 1e12 / peak,
                "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes": nbytes, "alg_flops": flops,
                "kernel_ms": kern, "cpu_baseline": cpu.get(i)}
        print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--decode", action="store_true")
    ap.add_argument("--rows", type=int, default=64)
    ap.add_argument("--layer", action="store_true")
    ap.add_argument("--fused", action="store_true")
    ap.add_argument("--all-configs", action="store_true", help="time every named workload (a report)")
    ap.add_argument("--config", type=int, action="append", choices=[1, 2, 3, 4, 5],
                    help="with or instead of --all-configs: only these named workloads (repeatable)")
    ap.add_argument("--no-exact", action="store_true",
                    help="skip timing the call with truncated segment starts switched off (profiler runs)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up (0 for counter runs)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if a.copy_probe:
        copy_probe()
        return
    if a.decode:
        bench_decode(a)
        return
    if a.layer:
        bench_layer(a)
        return
    if a.all_configs or a.config:
        bench_all_configs(a)
        return
    import gated_deltanet_prefill_gdr_amd as gdr
    from workloads import CONFIGS

    spec = CONFIGS[5]
    x = spec.draw()
    B, L, Hk, Hv, Dk, Dv = x.shape
    cpu = None
    if not a.no_cpu_baseline and not a.fused:   # forked workers: before anything touches the GPU
        cpu = cpu_baseline(x)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v, g, beta = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta))
    o = torch.empty(B, L, Hv, Dv, device=dev, dtype=v.dtype)
    s_final = torch.empty(B, Hv, Dk, Dv, device=dev, dtype=torch.float32)
    desc = gdr.make_desc(B, L, Hk, Hv, 0, True, a.fused)
    ws = torch.empty(gdr.workspace_size(desc), device=dev, dtype=torch.uint8)
    fused = {}
    if a.fused:   # raw bf16 gate projections in place of g and beta, and the gate z of the norm
        from workloads import draw_layer
        y = draw_layer(B, L, 1, Hv, 1, 5252, torch.bfloat16, D=Dv)
        fused = {"gates": tuple(t.to(dev) for t in (y.b_raw, y.a_raw, y.A_log, y.dt_bias)),
                 "norm": (y.x.to(dev), y.norm_w.to(dev), 1e-6)}
        g = beta = None

    def step():
        gdr.prefill(q, k, v, g, beta, out=o, s_final=s_final, workspace=ws, **fused)

    settle(step, a.settle)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ms, kern = run_timed(step, a.steps)
    # (row, head) pairs the last call recomputed without truncation (the status word), then the same
    # call with truncated segment starts switched off (the exact composition), for context
    off = gdr.status_offset(desc)
    reruns = int(ws[off:off + 4].view(torch.int32).item()) if off is not None else None
    ms_exact = None
    if not a.no_exact:
        gdr.set_truncation(False)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        ms_exact, _ = run_timed(step, max(10, a.steps // 2))
        gdr.set_truncation(True)

    units, nbytes, flops = algorithmic(B, L, Hk, Hv, 2, 0, True)
    if a.fused:   # raw bf16 projections instead of fp32 g, beta; plus the gate z
        nbytes += -2 * B * L * Hv * 4 + 2 * B * L * Hv * 2 + B * L * Hv * Dv * 2
    P = seg_plan(B, Hv, (L + CHUNK - 1) // CHUNK)
    per_kernel = {n: (t / max(c, 1), c) for n, (t, c) in kern.items() if c > 0}
    dominant = max(per_kernel, key=lambda n: per_kernel[n][0])
    k_ms = per_kernel[dominant][0]
    k_bytes = kernel_bytes(dominant, B, L, Hk, Hv, 2, P, fused=a.fused)
    # roofline of the whole call (every kernel of the path, back to back): the path's algorithmic bytes
    # (per unit, one token x one value head, times the units of the call) over the measured step time.
    # The dominant kernel's own figures sit under "dominant_kernel": the same algorithmic bytes over
    # its average launch time (the bound it would reach if the other kernels cost nothing), and its
    # interface bytes (what it reads and writes itself, intermediates included) over that time.
    achieved = nbytes / (ms * 1e-3) / 1e9
    traffic = None
    prof = os.path.join(ROOT, "profiles", "traffic_l16384_bf16.json")
    if os.path.exists(prof) and not a.fused:
        with open(prof) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash():   # counters of these very kernels only
            traffic = sum(k.get("hbm_bytes", 0) for k in tr.get("kernels", {}).values()) or None
    line = {
        "metric": METRIC if not a.fused else METRIC + ", gate prologue and gated RMSNorm fused",
        "value": units / (ms * 1e-3),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, beta~U(0.2,0.9), g~-U(0,0.5))",
        "config": {"workload": ("long prefill B=1 L=16384 Hk=16 Hv=32 Dk=Dv=128 bf16 q/k/v fp32 g/beta/state, "
                                "zero initial state, final state returned") if not a.fused else
                               ("long prefill B=1 L=16384 Hk=16 Hv=32 Dk=Dv=128 bf16 q/k/v, gate prologue from raw "
                                "bf16 projections and gated RMSNorm fused, fp32 state, final state returned"),
                   "B": B, "L": L, "Hk": Hk, "Hv": Hv, "D": Dk, "global_batch": B, "seq_len": L,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "scope": "whole gdr_prefill call (all kernels), algorithmic bytes / step time",
                     "alg_bytes_per_unit": nbytes / units, "units": units, "alg_bytes": nbytes,
                     "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "tflops": flops / (ms * 1e-3) / 1e12,
                     "dominant_kernel": {"name": dominant, "ms": k_ms,
                                         "frac_alg_bytes": nbytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                         "interface_bytes": k_bytes,
                                         "interface_GBs": k_bytes / (k_ms * 1e-3) / 1e9}},
        "path": {"ms": ms, "kernel_ms": {n: t for n, (t, c) in per_kernel.items()}, "segments": P,
                 "reruns": reruns, "exact_ms": ms_exact, "source_hash": source_hash()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

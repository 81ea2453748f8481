"""Seeded synthetic inputs for the chunked gated delta rule.

This module only draws random tensors. It holds none of the method's arithmetic (no
normalisation, no decay, no recurrence), so both the float64 oracle and the HIP path can
be fed from it without sharing any computation.

The regimes are the numerical situations of the kernel-test page (``r15_kernel_test.py``,
its input regimes), each a row of ``REGIME_TABLE`` read by one sampler:

* ``R1``: random keys, strong decay: beta ~ U(0.2, 0.9), g ~ -U(0.05, 3.0)
* ``R2``: random keys, weak decay:   beta ~ U(0.2, 0.9), g ~ -0.02 U(0, 1)
* ``R3``: correlated keys k = u sqrt(D)/|u| + 0.3 N(0,1), one u per key head,
          beta ~ U(0.3, 1.0), g ~ -0.02 U(0, 1)
* ``R4``: one key per head for every token, beta = 0.5, g = 0
* ``LONG``: random keys, beta ~ U(0.2, 0.9), g ~ -U(0.0, 0.5)  (the long-prefill case)

Draws are made in float32 with ``torch.Generator('cpu').manual_seed(seed)`` in the order
q, k, v, beta, g, s0 (``R3`` draws its direction u between q and the key noise; constant gates
draw nothing), then q, k and v are cast to the requested dtype. Right pads (positions at or past a
row's length) get beta = g = 0 in the tensors as well, as the page on the fork model
(``model.py``, class ``State`` docstring and ``_dn_gates``) makes pads exact no-ops.

The five named workloads are ``CONFIGS[1..5]``; ``config(i)`` returns their tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = ["Inputs", "draw", "config", "CONFIGS", "ConfigSpec", "LayerInputs", "draw_layer", "REGIME_TABLE",
           "Regime"]

@dataclass(frozen=True)
class Regime:
    """How one regime draws its keys and gates.

    keys: "random" (k ~ N(0,1)), "direction" (k = u sqrt(D)/|u| + 0.3 N(0,1), one unit direction u per
    (row, key head), drawn before the key noise) or "single" (one N(0,1) key per (row, key head),
    repeated at every token). beta and decay: (base, width) for base + width U(0,1) (beta) and
    -(base + width U(0,1)) (g), or a plain number for a constant.
    """

    keys: str
    beta: object
    decay: object


REGIME_TABLE = {
    "R1": Regime("random", (0.2, 0.7), (0.05, 2.95)),     # strong decay
    "R2": Regime("random", (0.2, 0.7), (0.0, 0.02)),      # weak decay
    "R3": Regime("direction", (0.3, 0.7), (0.0, 0.02)),   # correlated keys, weak decay
    "R4": Regime("single", 0.5, 0.0),                     # one key, no decay
    "LONG": Regime("random", (0.2, 0.7), (0.0, 0.5)),     # the long-prefill case
}
REGIMES = tuple(REGIME_TABLE)


def _uniform(spec, shape, gen):
    """base + width U(0, 1) for a (base, width) pair, else the constant."""
    if isinstance(spec, tuple):
        base, width = spec
        return base + width * torch.rand(*shape, generator=gen)
    return torch.full(shape, float(spec))


def _keys(mode, B, L, Hk, D, gen):
    if mode == "random":
        return torch.randn(B, L, Hk, D, generator=gen)
    if mode == "direction":
        u = torch.randn(B, 1, Hk, D, generator=gen)
        u = u / u.norm(dim=-1, keepdim=True) * D ** 0.5   # unit direction, length sqrt(D)
        return u + 0.3 * torch.randn(B, L, Hk, D, generator=gen)
    return torch.randn(B, 1, Hk, D, generator=gen).expand(B, L, Hk, D).contiguous()   # "single"


@dataclass
class Inputs:
    """One call's worth of inputs (CPU tensors, contiguous).

    q, k: [B, L, Hk, D] (dtype); v: [B, L, Hv, Dv] (dtype); g, beta: [B, L, Hv] float32;
    lengths: [B] int32 or None (all L valid); s0: [n_s0, Hv, D, Dv] float32 or None;
    s0_row: [B] int32 or None (identity).
    """

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    lengths: torch.Tensor | None
    s0: torch.Tensor | None
    s0_row: torch.Tensor | None

    @property
    def shape(self):
        B, L, Hk, D = self.q.shape
        return B, L, Hk, self.v.shape[2], D, self.v.shape[3]


def _row_lengths(lengths, B, L, gen):
    """(lengths [B] int64 or None, L): an int, a sequence, or "random:lo:hi" (drawn first; with L <= 0
    the rows are padded to a whole number of 64-token chunks)."""
    if lengths is None:
        return None, L
    if isinstance(lengths, str):
        _, lo, hi = lengths.split(":")
        lens = torch.randint(int(lo), int(hi) + 1, (B,), generator=gen, dtype=torch.int64)
        if L <= 0:
            L = 64 * math.ceil(int(lens.max()) / 64)
        return lens, L
    if isinstance(lengths, int):
        return torch.full((B,), lengths, dtype=torch.int64), L
    lens = torch.as_tensor(list(lengths), dtype=torch.int64)
    if lens.shape != (B,):
        raise ValueError("lengths must have B entries")
    return lens, L


def draw(B: int, L: int, Hk: int, Hv: int, D: int, regime: str, seed: int,
         dtype: torch.dtype = torch.float32, lengths=None, s0_rows: int = 0,
         s0_row=None, Dv: int | None = None, zero_pads: bool = True) -> Inputs:
    """Draw one seeded input set.

    lengths: None (all valid), an int (same for every row), a sequence of B ints, or the
    string "random:lo:hi" (one length per row, uniform integers in [lo, hi], drawn first).
    s0_rows: 0 for no initial state, else the number of state rows to draw
    (0.1 N(0,1) each). s0_row: None or a sequence of B row indices into those rows.
    """
    spec = REGIME_TABLE.get(regime)
    if spec is None:
        raise ValueError(f"unknown regime {regime!r}")
    if Hv % Hk:
        raise ValueError("Hv must be a multiple of Hk")
    Dv = D if Dv is None else Dv
    gen = torch.Generator().manual_seed(seed)
    lens, L = _row_lengths(lengths, B, L, gen)
    q = torch.randn(B, L, Hk, D, generator=gen)
    k = _keys(spec.keys, B, L, Hk, D, gen)
    v = torch.randn(B, L, Hv, Dv, generator=gen)
    beta = _uniform(spec.beta, (B, L, Hv), gen)
    g = -_uniform(spec.decay, (B, L, Hv), gen) if isinstance(spec.decay, tuple) else \
        torch.full((B, L, Hv), -float(spec.decay) + 0.0)
    s0 = torch.randn(s0_rows, Hv, D, Dv, generator=gen) * 0.1 if s0_rows else None
    if lens is not None and zero_pads:
        pad = (torch.arange(L)[None, :] >= lens[:, None])[..., None]  # [B, L, 1]
        beta = beta.masked_fill(pad, 0.0)
        g = g.masked_fill(pad, 0.0)
    rows = None if s0_row is None else torch.as_tensor(list(s0_row), dtype=torch.int32)
    return Inputs(q=q.to(dtype).contiguous(), k=k.to(dtype).contiguous(), v=v.to(dtype).contiguous(),
                  g=g.contiguous(), beta=beta.contiguous(),
                  lengths=None if lens is None else lens.to(torch.int32),
                  s0=s0, s0_row=rows)


@dataclass(frozen=True)
class ConfigSpec:
    name: str
    B: int
    L: int          # 0 = derived from the drawn lengths (64-token multiple of the longest)
    Hk: int
    Hv: int
    D: int
    dtype: torch.dtype
    regime: str
    seed: int
    lengths: object
    s0_rows: int
    s0_row: object

    def draw(self) -> Inputs:
        return draw(self.B, self.L, self.Hk, self.Hv, self.D, self.regime, self.seed, self.dtype,
                    lengths=self.lengths, s0_rows=self.s0_rows, s0_row=self.s0_row)


CONFIGS = {
    # 16 heads, no sharing, L = 64, fp32, strong decay, zero state, all valid.
    1: ConfigSpec("h16_l64_f32", 1, 64, 16, 16, 128, torch.float32, "R1", 11, None, 0, None),
    # 16 key / 32 value heads, L = 256 with 130 valid, weak decay, initial state 0.1 N(0,1).
    2: ConfigSpec("h16x32_l256_len130_s0_f32", 1, 256, 16, 32, 128, torch.float32, "R2", 21, 130, 1, None),
    # 16 / 32 heads, L = 4096, correlated keys, weak decay, zero state.
    3: ConfigSpec("h16x32_l4096_corr_f32", 1, 4096, 16, 32, 128, torch.float32, "R3", 31, None, 0, None),
    # 64 fork rows, lengths U{32..1024} padded to a 64 multiple, bf16, one shared initial state.
    4: ConfigSpec("forks_b64_h16x32_ragged_bf16", 64, 0, 16, 32, 128, torch.bfloat16, "R1", 41,
                  "random:32:1024", 1, tuple([0] * 64)),
    # Long prefill: L = 16384, bf16 q/k/v, fp32 g/beta/state, zero state.
    5: ConfigSpec("h16x32_l16384_bf16", 1, 16384, 16, 32, 128, torch.bfloat16, "LONG", 51, None, 0, None),
}


def config(i: int) -> Inputs:
    return CONFIGS[i].draw()


@dataclass
class LayerInputs:
    """Inputs of the layer steps around the delta rule (CPU tensors, contiguous).

    Gate prologue: b_raw, a_raw [B, L, Hv] (dtype) ~ N(0, 1); A_log [Hv] = log U(1, 16);
    dt_bias [Hv] ~ -2 + 0.5 N(0, 1) (float32).
    Conv: mixed [B, L, (2 Hk + Hv) D] (dtype) ~ N(0, 1); tail [B, K-1, Cm] (dtype) ~ N(0, 1);
    conv_w [Cm, K] ~ U(-1, 1) / sqrt(K) (float32).
    Norm: x, z [B, L, Hv, D] (dtype) ~ N(0, 1); norm_w [D] ~ 1 + 0.1 N(0, 1) (float32).
    lengths [B] int32 or None.
    """

    b_raw: torch.Tensor
    a_raw: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    mixed: torch.Tensor
    tail: torch.Tensor
    conv_w: torch.Tensor
    x: torch.Tensor
    z: torch.Tensor
    norm_w: torch.Tensor
    lengths: torch.Tensor | None


def draw_layer(B: int, L: int, Hk: int, Hv: int, K: int, seed: int, dtype: torch.dtype = torch.float32,
               lengths=None, D: int = 128) -> LayerInputs:
    """Seeded draws (float32, then cast) in the order b, a, A_log, dt_bias, mixed, tail, conv_w, x, z,
    norm_w. ``lengths``: None or a list of B ints."""
    gen = torch.Generator("cpu").manual_seed(seed)
    Cm = (2 * Hk + Hv) * D
    b_raw = torch.randn(B, L, Hv, generator=gen)
    a_raw = torch.randn(B, L, Hv, generator=gen)
    A_log = torch.log(1.0 + 15.0 * torch.rand(Hv, generator=gen))
    dt_bias = -2.0 + 0.5 * torch.randn(Hv, generator=gen)
    mixed = torch.randn(B, L, Cm, generator=gen)
    tail = torch.randn(B, K - 1, Cm, generator=gen)
    conv_w = (2.0 * torch.rand(Cm, K, generator=gen) - 1.0) / math.sqrt(K)
    x = torch.randn(B, L, Hv, D, generator=gen)
    z = torch.randn(B, L, Hv, D, generator=gen)
    norm_w = 1.0 + 0.1 * torch.randn(D, generator=gen)
    lens = None if lengths is None else torch.as_tensor(list(lengths), dtype=torch.int32)
    c = lambda t: t.to(dtype).contiguous()
    return LayerInputs(b_raw=c(b_raw), a_raw=c(a_raw), A_log=A_log, dt_bias=dt_bias, mixed=c(mixed), tail=c(tail),
                       conv_w=conv_w.contiguous(), x=c(x), z=c(z), norm_w=norm_w, lengths=lens)

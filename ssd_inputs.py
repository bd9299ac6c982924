"""Seeded synthetic inputs for the SSD (Mamba-2 state space dual) layer.

This module only draws random tensors: it holds none of the method's
arithmetic, and both the HIP path and the CPU oracle consume what it returns.
Everything is drawn in float32 on the CPU from a seeded ``torch.Generator``
and then rounded (round-to-nearest-even) to the working dtype, so the oracle
sees exactly the values the GPU sees.

Distributions (the five standard workloads):

* x ~ N(0, 1)                         layout [b, L, H, P]
* B, C ~ N(0, 1) / sqrt(N)            layout [b, L, G, N]
* dt = exp(U(ln 1e-3, ln 1e-1))       layout [b, L, H]   (log-uniform)
* A_h = -U(1, 16)                     layout [H], float32
* D_h = 0 or N(0, 1)                  layout [H], float32
* init state 0 or N(0, 1)             layout [b, H, P, N], float32
* "split" dt (long workload): dt = c * U(0.8, 1.2) with c = 1e-4 on heads
  [0, H/2) (decay ~1, long memory) and c = 0.5 on heads [H/2, H).

Draw order: A, D, x, B, C, dt, init.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int = 1
    chunk: int = 256
    dtype: str = "bf16"          # dtype of x, dt, B, C and y
    d_mode: str = "normal"       # "zero" | "normal"
    init_mode: str = "zero"      # "zero" (passed as NULL) | "normal"
    dt_mode: str = "loguniform"  # "loguniform" | "split"
    seed: int = 0
    steps: int = 0               # decode workloads: number of single-token steps

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five standard workloads (seed = 1000 + index).
WORKLOADS = {
    0: Workload("tiny-fp32", 1, 256, 4, 16, 16, 1, 64, "f32", "zero", "zero", seed=1000),
    1: Workload("370M-layer-bf16", 8, 2048, 32, 64, 128, 1, 256, "bf16", "normal", "zero", seed=1001),
    2: Workload("2.7B-layer-bf16", 4, 4096, 80, 64, 128, 1, 256, "bf16", "normal", "zero", seed=1002),
    3: Workload("long-carried-fp32", 1, 65536, 32, 64, 128, 1, 256, "f32", "normal", "normal",
                dt_mode="split", seed=1003),
    4: Workload("decode-bf16", 256, 1, 80, 64, 128, 1, 256, "bf16", "normal", "normal",
                seed=1004, steps=512),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _uniform(shape, lo, hi, g):
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def draw_A_D(w: Workload, g: torch.Generator):
    A = -_uniform((w.nheads,), 1.0, 16.0, g)
    if w.d_mode == "zero":
        D = torch.zeros(w.nheads, dtype=torch.float32)
    else:
        D = torch.randn(w.nheads, generator=g, dtype=torch.float32)
    return A, D


def draw_dt(w: Workload, shape, g: torch.Generator) -> torch.Tensor:
    """dt of the given shape whose last axis is the head axis."""
    if w.dt_mode == "loguniform":
        return torch.exp(_uniform(shape, math.log(1e-3), math.log(1e-1), g))
    if w.dt_mode == "split":
        H = shape[-1]
        c = torch.full((H,), 0.5, dtype=torch.float32)
        c[: H // 2] = 1e-4
        return _uniform(shape, 0.8, 1.2, g) * c
    raise ValueError(w.dt_mode)


def make_forward_inputs(w: Workload, seed: int | None = None) -> dict:
    """Inputs of one forward call, as CPU tensors in the workload's dtype.

    Returns a dict with x, dt, A, B, C, D (None when d_mode == "zero"),
    init (None when init_mode == "zero") and the Workload itself.
    """
    g = _gen(w.seed if seed is None else seed)
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    dt_ = DTYPES[w.dtype]
    A, D = draw_A_D(w, g)
    x = torch.randn((b, L, H, P), generator=g, dtype=torch.float32)
    B = torch.randn((b, L, G, N), generator=g, dtype=torch.float32) / math.sqrt(N)
    C = torch.randn((b, L, G, N), generator=g, dtype=torch.float32) / math.sqrt(N)
    dt = draw_dt(w, (b, L, H), g)
    init = None
    if w.init_mode == "normal":
        init = torch.randn((b, H, P, N), generator=g, dtype=torch.float32)
    return {
        "x": x.to(dt_).contiguous(),
        "dt": dt.to(dt_).contiguous(),
        "A": A.contiguous(),
        "B": B.to(dt_).contiguous(),
        "C": C.to(dt_).contiguous(),
        "D": None if w.d_mode == "zero" else D.contiguous(),
        "init": init,
        "workload": w,
    }


def make_output_grads(w: Workload, seed: int | None = None, with_final: bool = True) -> dict:
    """Seeded output gradients for a backward call: dy ~ N(0, 1) [b, L, H, P]
    in the workload's dtype and dfinal ~ N(0, 1) [b, H, P, N] float32 (None
    when with_final is False).  Seeded by seed (default w.seed + 500000)."""
    g = _gen(w.seed + 500000 if seed is None else seed)
    b, L, H, P, N = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate
    dy = torch.randn((b, L, H, P), generator=g, dtype=torch.float32)
    dfinal = torch.randn((b, H, P, N), generator=g, dtype=torch.float32) if with_final else None
    return {"dy": dy.to(DTYPES[w.dtype]).contiguous(), "dfinal": dfinal}


def make_decode_params(w: Workload) -> dict:
    """A, D and the initial state of a decode run (seeded by w.seed)."""
    g = _gen(w.seed)
    A, D = draw_A_D(w, g)
    state = torch.randn((w.batch, w.nheads, w.headdim, w.dstate), generator=g, dtype=torch.float32)
    return {"A": A, "D": None if w.d_mode == "zero" else D, "state": state}


def make_decode_step_inputs(w: Workload, step: int) -> dict:
    """Per-token inputs of decode step ``step`` (seed = w.seed * 10**6 + step)."""
    g = _gen(w.seed * 10**6 + step)
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    dt_ = DTYPES[w.dtype]
    x = torch.randn((b, H, P), generator=g, dtype=torch.float32)
    B = torch.randn((b, G, N), generator=g, dtype=torch.float32) / math.sqrt(N)
    C = torch.randn((b, G, N), generator=g, dtype=torch.float32) / math.sqrt(N)
    dt = draw_dt(w, (b, H), g)
    return {"x": x.to(dt_), "dt": dt.to(dt_), "B": B.to(dt_), "C": C.to(dt_)}


def to_f64(t):
    """Exact widening of a (bf16 / f32) tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()

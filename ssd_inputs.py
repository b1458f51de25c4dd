"""Seeded synthetic inputs for the chunked SSD scan.

This module only draws random tensors in a fixed order; it holds none of the
scan's arithmetic. Both the float64 oracle (``oracle/``) and the HIP path
(``chunked_ssd_scan_amd``) consume exactly the bytes produced here, so the two
sides see identical inputs (bf16 values are decoded exactly by the oracle).

Recipe (synthetic Mamba-2 / Mamba-3 layer-shaped data, no dataset, no weights):
  1. u ~ U(0, ln 16) [H],           A = -exp(u)             (per-head decay rate)
  2. z ~ N(0,1) [b,T,H],            dt = softplus(z - shift) (shift 2, or 4 for slow decay)
                                    da = dt * A              (float32 log-decay, <= 0)
  3. x ~ N(0,1) [b,T,R,H,P]
  4. B ~ N(0,1) [b,T,R,G,N]
  5. C ~ N(0,1) [b,T,R,G,N]        (x, B, C cast to the input dtype, bf16 by RNE)
  6. D ~ N(0,1) [H]                 (or zeros, or absent)
  7. theta ~ U(0, 0.1) [b,T,H,N/2]  (only when rotation is on)
  8. init = 0.1 * N(0,1) [b,H,P,N]  (only when an initial state is given)
All draws use one CPU ``torch.Generator`` seeded with ``seed`` (default 0).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass(frozen=True)
class Shape:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int = 1
    mimo_rank: int = 1
    chunk_len: int = 256
    dtype: str = "bf16"          # "bf16" or "f32": dtype of x, B, C
    skip: str = "randn"          # "randn" | "zeros" | "none"
    rotation: bool = False
    init_state: bool = False
    dt_shift: float = 2.0
    name: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five workloads: a tiny fp32 case, the Mamba-2 130M and 2.7B layer shapes,
# a Mamba-3 MIMO rank-4 layer with rotation, and a long-context slow-decay case.
CONFIGS = {
    0: Shape(1, 256, 4, 16, 16, 1, 1, 64, "f32", "zeros", False, False, 2.0,
             "tiny SISO fp32 b1 T256 H4 P16 N16 l64"),
    1: Shape(4, 4096, 24, 64, 128, 1, 1, 256, "bf16", "randn", False, False, 2.0,
             "mamba2-130m layer b4 T4096 H24 P64 N128 l256"),
    2: Shape(8, 8192, 80, 64, 128, 1, 1, 256, "bf16", "randn", False, False, 2.0,
             "mamba2-2.7b layer b8 T8192 H80 P64 N128 l256"),
    3: Shape(4, 4096, 32, 64, 128, 1, 4, 64, "bf16", "none", True, True, 2.0,
             "mamba3 mimo R4 rotation b4 T4096 H32 P64 N128 l64"),
    4: Shape(1, 131072, 64, 64, 128, 1, 1, 256, "bf16", "none", False, False, 4.0,
             "long context b1 T131072 H64 P64 N128 l256"),
}


@dataclass
class Inputs:
    shape: Shape
    x: torch.Tensor                  # [b,T,R,H,P]  bf16 or f32
    da: torch.Tensor                 # [b,T,H]      f32
    B: torch.Tensor                  # [b,T,R,G,N]  bf16 or f32
    C: torch.Tensor                  # [b,T,R,G,N]  bf16 or f32
    D: Optional[torch.Tensor]        # [H]          f32
    theta: Optional[torch.Tensor]    # [b,T,H,N/2]  f32
    init_state: Optional[torch.Tensor]  # [b,H,P,N] f32
    extra: dict = field(default_factory=dict)

    def to(self, device) -> "Inputs":
        mv = lambda t: None if t is None else t.to(device)
        return Inputs(self.shape, mv(self.x), mv(self.da), mv(self.B), mv(self.C),
                      mv(self.D), mv(self.theta), mv(self.init_state), dict(self.extra))


def _torch_dtype(name: str) -> torch.dtype:
    if name == "bf16":
        return torch.bfloat16
    if name == "f32":
        return torch.float32
    raise ValueError(f"unknown input dtype {name!r}")


def make_inputs(shape: Shape, seed: int = 0) -> Inputs:
    """Draw one seeded input set for ``shape`` on the CPU (fixed draw order)."""
    b, T, H, P, N = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate
    G, R = shape.ngroups, shape.mimo_rank
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt_in = _torch_dtype(shape.dtype)

    u = torch.rand(H, generator=g, dtype=torch.float32) * math.log(16.0)
    A = -torch.exp(u)
    z = torch.randn(b, T, H, generator=g, dtype=torch.float32)
    dt = torch.nn.functional.softplus(z - shape.dt_shift)
    da = (dt * A).contiguous()
    del z, dt
    x = torch.randn(b, T, R, H, P, generator=g, dtype=torch.float32).to(dt_in)
    Bm = torch.randn(b, T, R, G, N, generator=g, dtype=torch.float32).to(dt_in)
    Cm = torch.randn(b, T, R, G, N, generator=g, dtype=torch.float32).to(dt_in)
    if shape.skip == "randn":
        D = torch.randn(H, generator=g, dtype=torch.float32)
    elif shape.skip == "zeros":
        D = torch.zeros(H, dtype=torch.float32)
    elif shape.skip == "none":
        D = None
    else:
        raise ValueError(f"unknown skip mode {shape.skip!r}")
    theta = None
    if shape.rotation:
        if N % 2:
            raise ValueError("rotation needs an even state size")
        theta = torch.rand(b, T, H, N // 2, generator=g, dtype=torch.float32) * 0.1
    init = None
    if shape.init_state:
        init = 0.1 * torch.randn(b, H, P, N, generator=g, dtype=torch.float32)
    return Inputs(shape, x.contiguous(), da, Bm.contiguous(), Cm.contiguous(), D, theta, init)


def make_cotangents(shape: Shape, seed: int = 0, dfinal: bool = True):
    """Seeded cotangents for the backward: (dy, dfinal or None), float32.

    Their own CPU generator seeded with ``seed + 1000``, in this order:
    dy ~ N(0,1) [b,T,R,H,P], then dfinal ~ N(0,1) [b,H,P,N].
    """
    b, T, H, P, N = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 1000)
    dy = torch.randn((b, T, shape.mimo_rank, H, P), generator=g, dtype=torch.float32)
    df = torch.randn((b, H, P, N), generator=g, dtype=torch.float32) if dfinal else None
    return dy, df


def small_shape(**kw) -> Shape:
    """A Shape with defaults suited to quick oracle/parity cases."""
    base = dict(batch=2, seqlen=37, nheads=3, headdim=16, dstate=32, ngroups=1,
                mimo_rank=1, chunk_len=16, dtype="f32", skip="randn",
                rotation=False, init_state=False, dt_shift=2.0, name="small")
    base.update(kw)
    return Shape(**base)


# ---------------------------------------------------------------------------
# Mamba-1 selective scan (per-(channel, state) decay): seeded inputs.
# Recipe, one CPU generator seeded with ``seed``, in this order:
#   1. u ~ N(0,1) [b,T,D]
#   2. z ~ N(0,1) [b,T,D],  delta = softplus(z - shift)   (> 0; shift 2)
#   3. r ~ U(0, ln 16) [D,N], A = -exp(r)                  (< 0)
#   4. B ~ N(0,1) [b,T,N]
#   5. C ~ N(0,1) [b,T,N]
#   6. skip ~ N(0,1) [D]
# all float32. The workload is the LeetGPU performance-test shape.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class ScanShape:
    batch: int
    seqlen: int
    d_model: int
    d_state: int
    dt_shift: float = 2.0
    name: str = ""


SCAN_CONFIGS = {
    0: ScanShape(1, 64, 8, 4, 2.0, "tiny b1 T64 D8 N4"),
    1: ScanShape(4, 4096, 512, 16, 2.0, "selective scan b4 T4096 D512 N16"),
}


@dataclass
class ScanInputs:
    shape: ScanShape
    u: torch.Tensor        # [b,T,D]
    delta: torch.Tensor    # [b,T,D]
    A: torch.Tensor        # [D,N]
    B: torch.Tensor        # [b,T,N]
    C: torch.Tensor        # [b,T,N]
    skip: torch.Tensor     # [D]

    def to(self, device) -> "ScanInputs":
        return ScanInputs(self.shape, *(t.to(device) for t in (self.u, self.delta, self.A, self.B,
                                                                 self.C, self.skip)))


def make_scan_inputs(shape: ScanShape, seed: int = 0) -> ScanInputs:
    """Draw one seeded selective-scan input set on the CPU (fixed draw order)."""
    b, T, Dm, N = shape.batch, shape.seqlen, shape.d_model, shape.d_state
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    u = torch.randn(b, T, Dm, generator=g, dtype=torch.float32)
    z = torch.randn(b, T, Dm, generator=g, dtype=torch.float32)
    delta = torch.nn.functional.softplus(z - shape.dt_shift).contiguous()
    A = (-torch.exp(torch.rand(Dm, N, generator=g, dtype=torch.float32) * math.log(16.0))).contiguous()
    Bm = torch.randn(b, T, N, generator=g, dtype=torch.float32)
    Cm = torch.randn(b, T, N, generator=g, dtype=torch.float32)
    skip = torch.randn(Dm, generator=g, dtype=torch.float32)
    return ScanInputs(shape, u, delta, A, Bm, Cm, skip)


# ---------------------------------------------------------------------------
# Mamba-3 trapezoid (two-write) inputs: an SSD input set plus the trapezoid
# weights and the previous-token entries.
# ---------------------------------------------------------------------------

@dataclass
class TrapInputs:
    base: Inputs             # x, da, B, C, theta, init_state (D is not used)
    beta: torch.Tensor       # [b,T,H] fp32, weight of the previous step's write
    gamma: torch.Tensor      # [b,T,H] fp32, weight of this step's write
    prev_x: Optional[torch.Tensor]   # [b,R,H,P], x's dtype
    prev_B: Optional[torch.Tensor]   # [b,R,G,N], x's dtype

    def to(self, device) -> "TrapInputs":
        mv = lambda t: None if t is None else t.to(device)
        return TrapInputs(self.base.to(device), mv(self.beta), mv(self.gamma), mv(self.prev_x),
                          mv(self.prev_B))


def make_trapezoid_inputs(shape: Shape, seed: int = 0, prev: bool = True) -> TrapInputs:
    """Seeded trapezoid inputs on the CPU.

    The SSD inputs come from make_inputs(shape, seed). A second generator,
    seeded with seed + 7919, then draws in this order: lam ~ U(0, 1) [b,T,H],
    gamma = lam, beta = (1 - lam) * exp(da) (the trapezoid rule's weights with
    the step size already in x); prev_x ~ N(0, 1) [b,R,H,P] and
    prev_B ~ N(0, 1) [b,R,G,N], cast to x's dtype (when ``prev``).
    """
    base = make_inputs(shape, seed)
    b, T, H, P, N, G, R = (shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate,
                           shape.ngroups, shape.mimo_rank)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 7919)
    lam = torch.rand(b, T, H, generator=g, dtype=torch.float32)
    gamma = lam.contiguous()
    beta = ((1.0 - lam) * torch.exp(base.da)).contiguous()
    prev_x = prev_B = None
    if prev:
        dt = base.x.dtype
        prev_x = torch.randn(b, R, H, P, generator=g, dtype=torch.float32).to(dt).contiguous()
        prev_B = torch.randn(b, R, G, N, generator=g, dtype=torch.float32).to(dt).contiguous()
    return TrapInputs(base, beta, gamma, prev_x, prev_B)

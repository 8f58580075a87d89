"""Seeded synthetic inputs for the GDN verify step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through the tests and the benchmark)
and the CPU oracle take their inputs from here.

Workloads (sizes and value distributions; N(0, s) means standard deviation s):
  x ~ N(0, 1), conv taps ~ N(0, 0.5), conv history ~ N(0, 1),
  raw beta ~ N(0, 1), alpha ~ N(0, 1), dt_bias ~ U(-1, 1), A_log ~ U(0, ln 16),
  initial state ~ N(0, 0.1), accept lengths ~ U{0..K}.
Draw order from one torch CPU generator seeded once: x, w, hist, beta_raw,
alpha, dt_bias, A_log, S_in, accept.  bf16 tensors are rounded from the float32
draw by torch (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int          # verify window K, or prompt length for prefill
    Hk: int
    Hv: int
    dk: int
    dv: int
    W: int = 4
    bf16: bool = True
    chunk: int = 0  # > 0 for chunked prefill
    capture: bool = True

    @property
    def C(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv

    def as_dict(self):
        d = asdict(self)
        d["C"] = self.C
        return d


WORKLOADS = {
    # B=1, 2 heads, d=32, K=4 verify tokens, conv over 192 channels, fp32 everywhere
    "tiny": Workload("tiny", B=1, T=4, Hk=2, Hv=2, dk=32, dv=32, bf16=False),
    # decode step K=1: 16 key heads, 48 value heads (3:1), d=128, C=10240
    "decode": Workload("decode", B=1, T=1, Hk=16, Hv=48, dk=128, dv=128, capture=False),
    # speculative verify K=16 with intermediate-state capture
    "verify16": Workload("verify16", B=1, T=16, Hk=16, Hv=48, dk=128, dv=128),
    # batched verify: 32 sequences, K=8
    "batched": Workload("batched", B=32, T=8, Hk=16, Hv=48, dk=128, dv=128),
    # chunked prefill: 4 sequences x 4096 tokens, chunk 64, final state only
    "prefill": Workload("prefill", B=4, T=4096, Hk=16, Hv=48, dk=128, dv=128, chunk=64, capture=False),
}


def make_inputs(wl: Workload, seed: int = 0, weak_decay: bool = False, accept=None):
    """Draw the inputs of one workload on the CPU.

    Returns a dict of CPU tensors:
      x [B][T][C], w [C][W] f32, hist [B][W-1][C], beta_raw [B][T][Hv],
      alpha [B][T][Hv], dt_bias [Hv] f32, A_log [Hv] f32,
      S_in [B][Hv][dv][dk] f32, accept [B] int32.
    x, hist, beta_raw and alpha are bf16 for bf16 workloads, else f32.
    weak_decay draws A_log ~ U(-6, -2) instead (a test variant in which the
    initial state still matters after a long window).
    """
    g = torch.Generator().manual_seed(seed)
    io = torch.bfloat16 if wl.bf16 else torch.float32
    B, T, C, W, Hv = wl.B, wl.T, wl.C, wl.W, wl.Hv
    x = torch.randn(B, T, C, generator=g).to(io)
    w = (torch.randn(C, W, generator=g) * 0.5).float()
    hist = torch.randn(B, W - 1, C, generator=g).to(io)
    beta_raw = torch.randn(B, T, Hv, generator=g).to(io)
    alpha = torch.randn(B, T, Hv, generator=g).to(io)
    dt_bias = (torch.rand(Hv, generator=g) * 2.0 - 1.0).float()
    u = torch.rand(Hv, generator=g)
    if weak_decay:
        A_log = (u * 4.0 - 6.0).float()
    else:
        A_log = (u * math.log(16.0)).float()
    S_in = (torch.randn(B, Hv, wl.dv, wl.dk, generator=g) * 0.1).float()
    if accept is None:
        acc = torch.randint(0, T + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        acc = torch.as_tensor(accept, dtype=torch.int32).reshape(B)
    return dict(x=x, w=w, hist=hist, beta_raw=beta_raw, alpha=alpha,
                dt_bias=dt_bias, A_log=A_log, S_in=S_in, accept=acc)


def make_qkv(wl: Workload, seed: int = 0):
    """A q|k|v slab [B][T][C] ~ N(0, 1) drawn directly (for verify-only tests)."""
    g = torch.Generator().manual_seed(seed + 7919)
    io = torch.bfloat16 if wl.bf16 else torch.float32
    return torch.randn(wl.B, wl.T, wl.C, generator=g).to(io)


def small(name: str, **over) -> Workload:
    """A copy of a named workload with some sizes replaced (for tests)."""
    base = asdict(WORKLOADS[name])
    base.update(over)
    return Workload(**base)


def make_tree(B: int, N: int, seed: int = 0, shape: str = "random", fan: int = 4):
    """Parent indices [B][N] int32 of a draft tree, numbered parents first.

    chain:  parent[i] = i - 1 (node 0 a root) -- the plain verify window;
    star:   every node a root (N one-token continuations of the committed state);
    random: node 0 a root, node i >= 1 picks its parent uniformly among the
            `fan` nodes before it (depth about N / (fan/2 + 1));
    forest: like random, with the committed state (-1) as one more choice;
    binary: a complete binary tree numbered breadth first (parent (i-1)/2), the
            numbering of a level-by-level top-2 expansion: parents lie far back.
    """
    g = torch.Generator().manual_seed(seed + 104729)
    par = torch.empty(B, N, dtype=torch.int32)
    for b in range(B):
        for i in range(N):
            if shape == "chain":
                p = i - 1
            elif shape == "star":
                p = -1
            elif shape == "binary":
                p = (i - 1) // 2 if i > 0 else -1
            elif shape in ("random", "forest"):
                lo = max(0, i - fan)
                choices = list(range(lo, i)) + ([-1] if (shape == "forest" or i == 0) else [])
                p = choices[int(torch.randint(0, len(choices), (1,), generator=g))]
            else:
                raise ValueError("unknown tree shape %r" % shape)
            par[b, i] = p
    return par


def make_tree_accept(B: int, N: int, seed: int = 0):
    """The accepted node per sequence [B] int32, uniform over {-1 (none), 0..N-1}."""
    g = torch.Generator().manual_seed(seed + 15485863)
    return torch.randint(-1, N, (B,), generator=g, dtype=torch.int64).to(torch.int32)

"""Seeded synthetic inputs for the Longformer sparse-attention forward.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic.  Both the HIP path and the fp64 oracle are fed
from it, so the two sides always see bit-identical inputs.

Recipe (one per workload):

* ``torch.Generator('cpu').manual_seed(seed)``; q, k, v are drawn in that
  order as float32 ``randn`` of shape [B, H, T, d], multiplied by ``scale``
  and then cast to the working dtype (``.to(torch.bfloat16)`` rounds to
  nearest-even).
* integer draws (valid lengths, random global positions) come from
  ``numpy.random.default_rng(seed + 1)``: lengths first, then globals.

The shapes follow the Longformer-base attention geometry (12 heads of 64,
window 513) that the pages use as their running example (Longformer,
eightmm.github.io, "Sliding-Window Attention"; ciallo.wiki Longformer §6.1
names the base-4096 model).  No dataset is read: the long-document QA and
classification suites the pages evaluate on are stood in for by these
tensors (their statistics, not their contents, matter to the kernel).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    T: int
    d: int
    r: int
    dtype: str                      # "f32" or "bf16"
    scale: float = 1.0              # std of the N(0, scale^2) draw
    dilation: Optional[tuple] = None  # per-head stride, None = all 1
    # global pattern: list of fixed positions plus n_random random ones
    fixed_globals: tuple = ()
    n_random_globals: int = 0
    random_global_lo: int = 0       # random globals drawn from [lo, hi)
    random_global_hi_from_min_len: bool = False
    # right padding: valid length per sequence drawn uniformly from
    # [len_lo, len_hi] inclusive; None = no padding
    len_lo: Optional[int] = None
    len_hi: Optional[int] = None
    description: str = ""
    radius: Optional[tuple] = None  # one radius per head (replaces r), None = r for all
    one_sided: bool = False         # window keeps only the keys at or before the query
    n_rand: int = 0                 # random key blocks of 64 per query block of 64 (drawn last)


WORKLOADS: List[Workload] = [
    Workload("fp32-b1h2t1024-r64-g1", 1001, 1, 2, 1024, 64, 64, "f32",
             fixed_globals=(0,),
             description="B=1 H=2 T=1024 d=64 r=64 (w=129), one global at 0, fp32 N(0,1)"),
    Workload("bf16-b1h12t4096-r256-g1", 1002, 1, 12, 4096, 64, 256, "bf16",
             fixed_globals=(0,),
             description="Longformer-base shape: B=1 H=12 T=4096 d=64 r=256 (w=513), global at 0, bf16 N(0,1)"),
    Workload("bf16-b1h12t4096-r128-dil", 1003, 1, 12, 4096, 64, 128, "bf16",
             dilation=(1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 4, 4),
             description="dilated heads [1,1,2,2,2,2,3,3,3,3,4,4], r=128, no globals, bf16 N(0,1)"),
    Workload("bf16-b2h12t4096-r256-g68", 1004, 2, 12, 4096, 64, 256, "bf16",
             fixed_globals=tuple(range(64)), n_random_globals=4, random_global_lo=64,
             description="QA-style globals: 0..63 plus 4 random in [64,4096), B=2 H=12 T=4096 r=256, bf16 N(0,1)"),
    Workload("bf16-b4h16t16384-r512-g8-pad", 1005, 4, 16, 16384, 64, 512, "bf16", scale=0.5,
             n_random_globals=8, random_global_hi_from_min_len=True, len_lo=8192, len_hi=16384,
             description="B=4 H=16 T=16384 r=512, 8 random globals, valid lengths U{8192..16384} with right padding, bf16 0.5*N(0,1)"),
    # the two window forms beyond the five configurations: one-sided windows and one
    # radius per head (the per-layer window list applied per head)
    Workload("bf16-b1h12t4096-r256-g1-onesided", 1006, 1, 12, 4096, 64, 256, "bf16",
             fixed_globals=(0,), one_sided=True,
             description="the headline shape with one-sided windows (the query and the 256 keys before it), global at 0"),
    Workload("bf16-b1h12t4096-rhead-g1", 1007, 1, 12, 4096, 64, 512, "bf16",
             fixed_globals=(0,), radius=(32, 32, 64, 64, 128, 128, 256, 256, 384, 384, 512, 512),
             description="one radius per head, 32..512 in pairs, global at 0, bf16 N(0,1)"),
    # BigBird-style: window of about three blocks, the first and last token global,
    # three random key blocks of 64 per query block of 64
    Workload("bf16-b1h12t4096-r96-g2-rand3", 1008, 1, 12, 4096, 64, 96, "bf16",
             fixed_globals=(0, 4095), n_rand=3,
             description="r=96, globals 0 and T-1, 3 random key blocks of 64 per query block (per head), bf16 N(0,1)"),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    r: int
    dilation: Optional[List[int]]
    global_idx: List[int]
    lengths: Optional[List[int]]
    key_padding_mask: Optional[torch.Tensor]  # uint8 [B][T], nonzero = padded
    extra: dict = field(default_factory=dict)
    one_sided: bool = False                   # r: one radius, or a list with one per head
    random_blocks: Optional[np.ndarray] = None  # int32 [H][ceil(T/64)][n_rand] key-block indices


def _draw_qkv(seed, B, H, T, d, scale, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    out = []
    for _ in range(3):
        x = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
        if scale != 1.0:
            x = x * scale
        out.append(x.to(dtype).contiguous())
    return out


def make_inputs(w: Workload, dtype: Optional[str] = None, T: Optional[int] = None,
                B: Optional[int] = None, H: Optional[int] = None) -> Inputs:
    """Materialise a workload on the CPU.

    ``dtype`` overrides the workload's dtype (used to run every shape in
    fp32 as well); ``T``/``B``/``H`` shrink the shape for quick tests while
    keeping the rest of the recipe (fixed globals beyond the new T are
    dropped, random ones are drawn in the new range).
    """
    dt = dtype or w.dtype
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dt]
    B_ = B or w.B
    H_ = H or w.H
    T_ = T or w.T
    q, k, v = _draw_qkv(w.seed, B_, H_, T_, w.d, w.scale, tdt)
    rng = np.random.default_rng(w.seed + 1)
    lengths = None
    kpm = None
    if w.len_lo is not None:
        # a shrunk sequence keeps the same fraction of padding
        lo = max(1, (w.len_lo * T_) // w.T)
        hi = max(lo, (w.len_hi * T_) // w.T)
        lengths = [int(x) for x in rng.integers(lo, hi + 1, size=B_)]
        pos = torch.arange(T_).unsqueeze(0)
        kpm = (pos >= torch.tensor(lengths).unsqueeze(1)).to(torch.uint8).contiguous()
    glob = [g for g in w.fixed_globals if g < T_]
    if w.n_random_globals:
        if w.random_global_hi_from_min_len:
            hi = min(lengths) if lengths else T_
        else:
            hi = T_
        lo = min(w.random_global_lo, hi)
        pool = hi - lo
        n = min(w.n_random_globals, pool)
        if n > 0:
            glob += [int(x) + lo for x in rng.choice(pool, size=n, replace=False)]
    dil = list(w.dilation)[:H_] if w.dilation else None
    if dil is not None and len(dil) < H_:
        dil = dil + [1] * (H_ - len(dil))
    r = list(w.radius)[:H_] if w.radius else w.r
    rb = None
    if w.n_rand:
        # per head and query block: n_rand distinct key blocks, uniform
        nqb = (T_ + 63) // 64
        rb = np.stack([np.stack([rng.choice(nqb, size=min(w.n_rand, nqb), replace=False) for _ in range(nqb)])
                       for _ in range(H_)]).astype(np.int32)
    return Inputs(q, k, v, r, dil, glob, lengths, kpm, one_sided=w.one_sided, random_blocks=rb)


def random_case(seed: int, B: int, H: int, T: int, d: int = 64, dtype: str = "f32",
                r: Optional[int] = None, max_dil: int = 4, n_global: Optional[int] = None,
                pad: str = "random", n_rand: int = 0) -> Inputs:
    """A small random case for edge-case sweeps.

    pad: "none", "right" (random valid length per sequence, possibly 0) or
    "random" (an arbitrary per-key pattern).
    """
    rng = np.random.default_rng(seed)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    q, k, v = _draw_qkv(seed, B, H, T, d, 1.0, tdt)
    if r is None:
        r = int(rng.integers(0, T + 3))
    dil = [int(x) for x in rng.integers(1, max_dil + 1, size=H)]
    if n_global is None:
        n_global = int(rng.integers(0, min(T, 6) + 1))
    glob = [int(x) for x in rng.integers(0, T, size=n_global)]  # duplicates allowed
    lengths = None
    kpm = None
    if pad == "right":
        lengths = [int(x) for x in rng.integers(0, T + 1, size=B)]
        pos = torch.arange(T).unsqueeze(0)
        kpm = (pos >= torch.tensor(lengths).unsqueeze(1)).to(torch.uint8).contiguous()
    elif pad == "random":
        kpm = torch.from_numpy((rng.random((B, T)) < 0.2).astype(np.uint8)).contiguous()
    rb = None
    if n_rand:
        # random key blocks need undilated heads; blocks may repeat (they count once)
        dil = [1] * H
        nqb = (T + 63) // 64
        rb = rng.integers(0, nqb, size=(H, nqb, n_rand)).astype(np.int32)
    return Inputs(q, k, v, r, dil, glob, lengths, kpm, random_blocks=rb)


def make_grad(inp: Inputs, seed: int) -> torch.Tensor:
    """An upstream gradient dy like q: float32 ``randn`` from a generator
    seeded with ``seed``, cast (round to nearest even) to q's dtype."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    return torch.randn(tuple(inp.q.shape), generator=g, dtype=torch.float32).to(inp.q.dtype)

"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This module only draws numbers and describes input structure (shapes, packed
sequence lengths).  It holds none of the attention arithmetic and none of the
token-to-device layout logic: the oracle and the HIP library each apply their
own layout to the global tensors drawn here.

Recipes:
* Q, K, V, dO ~ N(0, 1), drawn in float32 by torch's counter-based generator
  (``torch.Generator`` on the requested device, seeded), then rounded to the
  working dtype (bf16 by round-to-nearest-even).  The draw order is Q, K, V,
  dO from one generator.
* Packed sequence lengths: log-uniform in [lo, hi] from numpy's
  ``default_rng(seed)``; lengths are appended until their sum reaches the
  total and the last one is cut so that the sum equals the total exactly.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def draw_normal(shapes: Sequence[Tuple[int, ...]], dtype, seed: int, device="cpu"):
    """Tensors ~ N(0, 1) of the given shapes, drawn in order from one generator."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    outs = []
    for shp in shapes:
        x = torch.randn(tuple(shp), generator=gen, device=device, dtype=torch.float32)
        outs.append(x.to(dtype))
    return outs


def qkv(seq_len: int, heads: int, head_dim: int, dtype, seed: int, device="cpu",
        batch: int = 1, with_dout: bool = False):
    """Global token-major [batch, seq_len, heads, head_dim] Q, K, V (and dO)."""
    shp = (batch, seq_len, heads, head_dim)
    n = 4 if with_dout else 3
    return draw_normal([shp] * n, dtype, seed, device)


def loguniform_lengths(total: int, lo: int, hi: int, seed: int) -> List[int]:
    """Packed sequence lengths, log-uniform in [lo, hi], summing to ``total``."""
    rng = np.random.default_rng(int(seed))
    out: List[int] = []
    acc = 0
    while acc < total:
        n = int(math.exp(rng.uniform(math.log(lo), math.log(hi))))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out


def cu_seqlens(lengths: Sequence[int]) -> np.ndarray:
    """int32 offsets [0, l0, l0+l1, ...] of packed sequences."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def round_lengths(lengths, unit: int):
    """Round packed sequence lengths down to multiples of ``unit`` (at least one
    unit each), giving what that removes to the last sequence, so the total is
    unchanged (it must itself be a multiple of ``unit``)."""
    total = int(sum(lengths))
    if total % unit:
        raise ValueError("total length must be a multiple of unit")
    out = [max(unit, (int(n) // unit) * unit) for n in lengths]
    out[-1] += total - sum(out)
    if out[-1] <= 0:
        raise ValueError("lengths too short to round")
    return out

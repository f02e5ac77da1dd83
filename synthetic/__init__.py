"""Seeded synthetic inputs shaped like the workloads of the W4A16 group-wise INT4 pages.

This module only draws random tensors; it holds none of the quantization arithmetic.
Both the CPU oracle tests and the GPU path take their inputs from here, so the two sides
see identical bytes.

Distribution recipe (stated once, used everywhere):

* Weights: ``randn`` in fp32 times ``sigma``.  A set of "outlier" input channels
  (columns of W) is multiplied by a factor in fp32, then the tensor is cast once to the
  target dtype (round-to-nearest-even for bf16/fp16).  The outlier fraction is about 0.1%
  of the input channels, the share the page "Quantization Algorithms 단권화" gives for
  emergent outlier channels (LLM.int8() chapter, "problem: emergent outlier").
* Activations: ``randn`` in fp32 (standard normal), optionally with the same outlier
  channels scaled, then cast once to the activation dtype.
* Outlier channel set: ``randperm(K)[:round(0.001*K)]`` from the weight's own generator,
  so weight and activation outliers sit on the same channels.
* KV-cache tokens (the KV-cache chapter of "Quantization Algorithms 단권화" describes K as
  centred near zero with a mild per-channel skew and V as asymmetric with magnitudes that
  vary from token to token): K[t, h, i] = N(0, 1) + b[h, i] with a per-channel offset
  b ~ N(0, 0.5); V[t, h, i] = N(0, 1) * m[t, h] + 0.25 with a per-token magnitude
  m = exp(N(0, 0.5)); queries q[h, i] ~ N(0, 1).  Drawn in fp32, cast once.

Every generator is a ``torch.Generator`` seeded with the stated seed.  Host (CPU)
generation is the default.  ``device="cuda"`` uses a seeded device generator (a
different stream of numbers than the CPU one, still deterministic); it serves the
multi-gigabyte checkpoint sweep, whose parity is checked on rows copied back to the host.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import torch

__all__ = [
    "outlier_channels",
    "weight",
    "activations",
    "Matrix",
    "TINY",
    "DECODE_7B",
    "MLP_SWEEP",
    "PREFILL_70B",
    "checkpoint_7b",
    "kv_tokens",
    "query",
    "KV_7B",
    "sparse_groups",
]


def outlier_channels(k: int, seed: int, fraction: float = 0.001) -> torch.Tensor:
    """Indices of the outlier input channels for a K-wide matrix (int64, sorted)."""
    n_out = int(round(fraction * k))
    g = torch.Generator().manual_seed(int(seed) * 7919 + 17)
    idx = torch.randperm(k, generator=g)[:n_out]
    return torch.sort(idx).values


def weight(n: int, k: int, sigma: float, seed: int, dtype=torch.bfloat16,
           outlier_factor: float = 0.0, device: str = "cpu") -> torch.Tensor:
    """W [n, k] ~ N(0, sigma^2), optional outlier input channels times ``outlier_factor``."""
    if device == "cpu":
        g = torch.Generator().manual_seed(int(seed))
    else:
        g = torch.Generator(device=device).manual_seed(int(seed))
    w = torch.randn(n, k, generator=g, dtype=torch.float32, device=device)
    w.mul_(sigma)
    if outlier_factor:
        cols = outlier_channels(k, seed).to(device)
        w[:, cols] *= outlier_factor
    return w.to(dtype)


def activations(m: int, k: int, seed: int, dtype=torch.bfloat16,
                outlier_seed: Optional[int] = None, outlier_factor: float = 0.0,
                device: str = "cpu") -> torch.Tensor:
    """x [m, k] ~ N(0, 1); channels of ``outlier_channels(k, outlier_seed)`` times a factor."""
    if device == "cpu":
        g = torch.Generator().manual_seed(int(seed))
    else:
        g = torch.Generator(device=device).manual_seed(int(seed))
    x = torch.randn(m, k, generator=g, dtype=torch.float32, device=device)
    if outlier_factor and outlier_seed is not None:
        cols = outlier_channels(k, outlier_seed).to(device)
        x[:, cols] *= outlier_factor
    return x.to(dtype)


@dataclasses.dataclass(frozen=True)
class Matrix:
    """One projection-shaped weight matrix of a workload."""
    name: str
    n: int            # output features (rows of W)
    k: int            # input features (columns of W, the group axis)
    sigma: float
    seed: int
    outlier_factor: float = 0.0
    dtype: torch.dtype = torch.bfloat16

    def make(self, device: str = "cpu") -> torch.Tensor:
        return weight(self.n, self.k, self.sigma, self.seed, self.dtype,
                      self.outlier_factor, device)


# Tiny reference: W fp32 [256 x 512] ~ N(0, 0.02), x bf16 [1 x 512] ~ N(0, 1), group 128.
TINY = dict(
    w=Matrix("tiny", 256, 512, 0.02, seed=0, dtype=torch.float32),
    x_seed=1, m=1, group_size=128,
)

# 7B-like decode projections, M = 1, group 128, asymmetric; 0.1% outlier columns x20.
DECODE_7B = dict(
    mats=[Matrix("attn_4096x4096", 4096, 4096, 0.02, seed=2, outlier_factor=20.0),
          Matrix("mlp_11008x4096", 11008, 4096, 0.02, seed=3, outlier_factor=20.0)],
    x_seed=4, m=1, group_size=128, symmetric=False,
)

# 7B-like MLP batch sweep: both MLP orientations, g in {32, 64, 128}, sym and asym,
# M in {1, 2, 4, 8, 16} (first M rows of one x per K).
MLP_SWEEP = dict(
    mats=[Matrix("up_11008x4096", 11008, 4096, 0.02, seed=5),
          Matrix("down_4096x11008", 4096, 11008, 0.02, seed=6)],
    x_seed=7, ms=(1, 2, 4, 8, 16), group_sizes=(32, 64, 128), symmetric=(False, True),
)

# 70B-like prefill: W [28672 x 8192] ~ N(0, 0.015) with 0.1% outlier channels x20,
# x [2048 x 8192] ~ N(0, 1) with the same channels x10; group 128 asymmetric.
PREFILL_70B = dict(
    w=Matrix("mlp_28672x8192", 28672, 8192, 0.015, seed=8, outlier_factor=20.0),
    x_seed=9, m=2048, x_outlier_factor=10.0, group_size=128, symmetric=False,
)


def checkpoint_7b(layers: int = 32) -> List[Matrix]:
    """The 32-layer 7B-like checkpoint: per layer q, k, v, o [4096x4096], gate, up
    [11008x4096], down [4096x11008], bf16 ~ N(0, 0.02); seed 100 + 7*layer + index."""
    shapes = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
              ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
    out = []
    for layer in range(layers):
        for idx, (nm, n, k) in enumerate(shapes):
            out.append(Matrix(f"L{layer}.{nm}", n, k, 0.02, seed=100 + 7 * layer + idx))
    return out


def sample_rows(n: int, count: int, seed: int) -> torch.Tensor:
    """A seeded, sorted sample of ``count`` distinct row indices in [0, n), always
    including the first and the last row (edges of the tiling)."""
    count = min(count, n)
    g = torch.Generator().manual_seed(int(seed))
    idx = torch.randperm(n, generator=g)[:count]
    idx = torch.unique(torch.cat([idx, torch.tensor([0, n - 1])]))
    return idx[:max(count, 2)] if idx.numel() > count + 2 else idx


def as_u16(t: torch.Tensor):
    """Raw 16-bit patterns of a bf16/fp16 tensor as a numpy uint16 array (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def kv_tokens(t: int, heads: int, head_dim: int, seed: int, kind: str,
              dtype=torch.bfloat16) -> torch.Tensor:
    """New KV-cache entries [t, heads, head_dim] of the K ("k") or V ("v") recipe."""
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn((t, heads, head_dim), generator=g, dtype=torch.float32)
    if kind == "k":
        b = torch.randn((1, heads, head_dim), generator=g, dtype=torch.float32) * 0.5
        x = x + b
    elif kind == "v":
        m = torch.exp(torch.randn((t, heads, 1), generator=g, dtype=torch.float32) * 0.5)
        x = x * m + 0.25
    else:
        raise ValueError("kind must be 'k' or 'v'")
    return x.to(dtype)


def query(heads: int, head_dim: int, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    """One decode step's queries q [heads, head_dim] ~ N(0, 1)."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn((heads, head_dim), generator=g, dtype=torch.float32).to(dtype)


# 7B-shaped decode attention over an INT4 cache: 32 heads of 128 dimensions, groups of 32
# along the head dimension, asymmetric (the pages' KV scheme), a 4096-token context.
KV_7B = dict(heads=32, head_dim=128, group_size=32, symmetric=False, t=4096, t_cap=4096,
             k_seed=200, v_seed=201, q_seed=202)


def sparse_groups(n: int, k: int, g: int, m: int, dtype=torch.bfloat16):
    """A decode input built so that almost every code of a group equals its zero point
    while those columns carry large activations: W [n, k] fp32 is zero except one weight
    per group of g columns, at column (7j + 3) mod g of group j (the same columns in every
    row), of magnitude (1 + r mod 7)/8 and sign (-1)^r in row r; x [m, k] is
    64 * (1 + i/16) on the zero columns of row i, negated where k mod 3 == 0 in the odd
    rows, and 2^-7 * (1 + i/8) on the weighted ones.  A dot product of such a row is small
    while sum |x| over each group is about 64 g.  No randomness."""
    cols = torch.tensor([j * g + (7 * j + 3) % g for j in range(k // g)], dtype=torch.int64)
    w = torch.zeros(n, k, dtype=torch.float32)
    r = torch.arange(n, dtype=torch.float32)
    mag = (1.0 + torch.remainder(r, 7)) / 8.0
    sign = 1.0 - 2.0 * torch.remainder(r, 2)
    w[:, cols] = (mag * sign)[:, None]
    i = torch.arange(m, dtype=torch.float32)[:, None]
    kk = torch.arange(k)
    neg = (kk % 3 == 0)[None, :] & (torch.arange(m) % 2 == 1)[:, None]
    x = 64.0 * (1.0 + i / 16.0) * torch.where(neg, -1.0, 1.0)
    x[:, cols] = (2.0 ** -7) * (1.0 + i / 8.0)
    return w, x.to(dtype)

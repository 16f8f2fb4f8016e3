"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module only describes shapes and draws random numbers; it holds none of
the attention arithmetic, so both the HIP path and the fp64 oracle can be fed
from it without sharing any of the method.

The five workloads stand in for the data the Sparse Transformer pages model
(no dataset is read or reproduced; only the shapes are taken):

* ``tiny``   -- a 256-long strided A/B pair, fp32, block 16: small enough for
  the oracle and a dense brute force to cover completely.
* ``img32``  -- CIFAR-10-shaped images, 32x32x3 = 3072 positions, strided
  l=128, head dim 128 ("OpenAI Sparse Transformer", "Experimental Results
  and Performance").
* ``text``   -- Enwik8-shaped byte text, 12288 positions, fixed pattern
  l=128, c=32 (the fixed pattern is the one the pages recommend for text,
  "Factorized Attention Patterns").
* ``img64``  -- ImageNet 64x64x3 = 12288 positions, strided l=128; the same
  shape as the 154 GB example of "Reducing Memory Constraints with Deep
  Attention", and also run with dense causal attention for comparison.
* ``audio``  -- raw-audio-shaped, 65536 positions (the pages quote about
  65,000 samples, "Raw Audio Generation"), strided l=256.

Heads alternate between the two halves of a factorized pattern: even heads
use part A, odd heads part B.  Q, K and V are iid N(0,1)/sqrt(d) drawn in
fp32 on the CPU from ``torch.Generator().manual_seed(20190423 + index)`` and
cast to the workload dtype; dO is iid N(0,1) from seed + 1000.  The kernels
and the oracle receive the same (cast) values; the oracle upcasts them
exactly to fp64.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

import numpy as np
import torch

SEED_BASE = 20190423


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the list below (seed offset)
    batch: int
    heads: int
    n: int
    d: int
    block: int
    dtype: str            # "f32" or "bf16"
    pattern: str          # "strided" or "fixed"
    l: int
    c: int
    backward: bool
    dense_comparison: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def head_patterns(self, dense: bool = False) -> List[Tuple[str, int, int]]:
        """(pattern name, l, c) per head: even heads A, odd heads B."""
        if dense:
            return [("dense", 1, 1)] * self.heads
        a, b = ("strided_a", "strided_b") if self.pattern == "strided" else ("fixed_a", "fixed_b")
        return [(a if h % 2 == 0 else b, self.l, self.c) for h in range(self.heads)]

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.batch, self.heads, self.n, self.d)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 0, 1, 2, 256, 64, 16, "f32", "strided", 16, 1, backward=False),
        Workload("img32", 1, 8, 2, 3072, 128, 64, "bf16", "strided", 128, 1, backward=True),
        Workload("text", 2, 4, 8, 12288, 64, 64, "bf16", "fixed", 128, 32, backward=True),
        Workload("img64", 3, 2, 16, 12288, 64, 64, "bf16", "strided", 128, 1, backward=True,
                 dense_comparison=True),
        Workload("audio", 4, 1, 4, 65536, 64, 64, "bf16", "strided", 256, 1, backward=True),
    ]
}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def draw(shape, seed: int, std: float, dtype: torch.dtype) -> torch.Tensor:
    """iid N(0, std^2) drawn in fp32 on the CPU, then cast to ``dtype``."""
    x = torch.randn(shape, generator=generator(seed), dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def make_inputs(w: Workload, shape=None, seed_offset: int = 0, std: float = None,
                with_dout: bool = True) -> Dict[str, torch.Tensor]:
    """Q, K, V (and dO) on the CPU for workload ``w`` (or a custom shape with the
    same recipe).  ``std`` defaults to 1/sqrt(d); the "sharp" variant passes 1."""
    shape = shape or w.shape
    d = shape[-1]
    s = 1.0 / math.sqrt(d) if std is None else std
    seed = SEED_BASE + w.index + seed_offset
    out = {
        "q": draw(shape, seed * 4 + 0, s, w.torch_dtype),
        "k": draw(shape, seed * 4 + 1, s, w.torch_dtype),
        "v": draw(shape, seed * 4 + 2, s, w.torch_dtype),
    }
    if with_dout:
        out["do"] = draw(shape, (seed + 1000) * 4 + 3, 1.0, w.torch_dtype)
    return out


def custom_inputs(shape, dtype: torch.dtype, seed: int, std: float = None,
                  with_dout: bool = True) -> Dict[str, torch.Tensor]:
    """Same recipe for an arbitrary shape/dtype (edge-case tests)."""
    d = shape[-1]
    s = 1.0 / math.sqrt(d) if std is None else std
    out = {
        "q": draw(shape, seed * 4 + 0, s, dtype),
        "k": draw(shape, seed * 4 + 1, s, dtype),
        "v": draw(shape, seed * 4 + 2, s, dtype),
    }
    if with_dout:
        out["do"] = draw(shape, (seed + 1000) * 4 + 3, 1.0, dtype)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16/fp32 tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float32).to(torch.float64).numpy()

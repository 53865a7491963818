"""Seeded synthetic tensor-parallel tensors for tests and benchmarks.

This module only draws random numbers and casts them to bf16; it holds none of
the compression method's arithmetic, so both the HIP path and the CPU oracle can
consume its output.

The pages describe TP intermediate tensors as dense and concentrated near zero
with a long tail [TACO pt-summary, section 1 (data distribution) and 2.A].  No
dataset or weights are available, so each workload below stands in for the
activations or gradients of a model of the named shape:

* activation mix: with probability 0.99 a Laplace(0, b=0.01) draw, otherwise a
  Student-t(nu=2) draw (the long tail);
* gradient mix: with probability 0.99 a Gaussian(0, sigma=1e-4) draw, otherwise
  1e-2 * Student-t(nu=3);
* outlier columns: round(0.5% * hidden) distinct columns multiplied by a factor;
* per-row magnitudes (Qwen-shaped): every row multiplied by LogNormal(0, 1.5).

Draw order for one tensor from ``numpy.random.default_rng(seed)``: mixture
selector, body, tail, outlier columns, row magnitudes.  The float64 draws are
cast to float32 and then to bfloat16 (round to nearest even) with torch; the
resulting bf16 tensor is the ground truth fed to every implementation.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    block: int
    mix: str                 # "act" or "grad"
    outlier_factor: float    # 0 = no outlier columns
    row_lognormal: bool = False
    description: str = ""

    @property
    def numel(self) -> int:
        return self.tokens * self.hidden


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 256, 1024, 64, "act", 0.0,
                 description="tiny bf16 [256, 1024], block 64, activation mix"),
        Workload("gpt2_1p5b", 4096, 1600, 64, "act", 20.0,
                 description="GPT-2-1.5B-shaped TP activation bf16 [4096, 1600], block 64, "
                             "0.5% outlier columns x20"),
        Workload("gpt3_6p7b_act", 4096, 4096, 128, "act", 20.0,
                 description="GPT-3-6.7B-shaped TP forward activation bf16 [4096, 4096], "
                             "block 128, 0.5% outlier columns x20"),
        Workload("gpt3_6p7b_grad", 4096, 4096, 128, "grad", 0.0,
                 description="GPT-3-6.7B-shaped TP backward gradient bf16 [4096, 4096], "
                             "block 128, Gaussian body with Student-t(3) tail"),
        Workload("qwen_7b", 8192, 3584, 128, "act", 50.0, row_lognormal=True,
                 description="Qwen-7B-shaped TP activation bf16 [8192, 3584], block 128, "
                             "LogNormal(0,1.5) row magnitudes, 0.5% outlier columns x50"),
        Workload("dsum_part", 4096, 4096, 256, "act", 20.0,
                 description="one partial-sum part for decompress-and-sum, bf16 "
                             "[4096, 4096], block 256, GPT-3 activation mix"),
    ]
}


def draw_f64(tokens: int, hidden: int, mix: str, outlier_factor: float,
             row_lognormal: bool, seed: int) -> np.ndarray:
    """float64 draws in the documented order (see module docstring)."""
    rng = np.random.default_rng(seed)
    shape = (tokens, hidden)
    u = rng.random(shape)
    if mix == "act":
        body = rng.laplace(0.0, 0.01, shape)
        tail = rng.standard_t(2.0, shape)
    elif mix == "grad":
        body = rng.normal(0.0, 1e-4, shape)
        tail = 1e-2 * rng.standard_t(3.0, shape)
    else:
        raise ValueError(f"unknown mix {mix!r}")
    x = np.where(u < 0.01, tail, body)
    del u, body, tail
    if outlier_factor:
        n_out = int(round(0.005 * hidden))
        cols = rng.choice(hidden, n_out, replace=False)
        x[:, cols] *= outlier_factor
    if row_lognormal:
        x *= rng.lognormal(0.0, 1.5, tokens)[:, None]
    return x


def make(name: str, seed: int = 0, tokens: int | None = None) -> torch.Tensor:
    """bf16 CPU tensor of workload ``name`` (optionally only the first ``tokens`` rows
    of a shorter draw with the same recipe)."""
    w = WORKLOADS[name]
    t = w.tokens if tokens is None else tokens
    x = draw_f64(t, w.hidden, w.mix, w.outlier_factor, w.row_lognormal, seed)
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (on CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(bits: np.ndarray) -> torch.Tensor:
    """bf16 tensor from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)

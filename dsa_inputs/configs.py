"""Workload table for the DSV-style block-sparse attention path.

Each entry is a synthetic stand-in for one attention layer of a video diffusion
transformer (DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video DiT
Training, gist.science/ar/paper/2502.07590).  The page gives no dataset and no
shapes; the shapes, tilings, predictor rank, keep fractions and feature
amplitudes below are the five workloads this library is specified against:

* ``tiny_fp32``    -- 256 tokens, fp32, 16 blocks; the oracle's exact-check size.
* ``layer_32k``    -- one bf16 layer, 32,768 tokens, 512 blocks, 10 % kept
                      (the page's "attend to about a tenth", section 3a).
* ``long_524k``    -- 524,288 tokens, 8,192 blocks, 5 % kept (the page's
                      ~520K-token videos, Result section; "95 % wasted", section 1).
* ``train_32k``    -- ``layer_32k`` plus an upstream gradient: a training step.
* ``dynamic_55k``  -- 55,296 tokens, per-head keep fraction and per-sample
                      feature amplitude, so patterns differ across heads and
                      samples (the page's "dynamic, near and far", section 2).

This module holds no arithmetic of the method; it only names sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    d: int
    latent: Tuple[int, int, int]      # (Lt, Lh, Lw); tokens row-major over (t, y, x)
    tile: Tuple[int, int, int]        # (tt, th, tw); query tile == key block
    r: int                            # predictor rank
    keep_percent: Tuple[int, ...]     # one entry (all heads) or one per head
    amplitude: Tuple[float, ...]      # one entry (all samples) or one per sample
    dtype: str                        # "fp32" or "bf16"
    backward: bool = False
    shuffle_keep: bool = False        # keep_percent is a pool shuffled over heads
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        Lt, Lh, Lw = self.latent
        return Lt * Lh * Lw

    @property
    def T(self) -> int:
        tt, th, tw = self.tile
        return tt * th * tw

    @property
    def NB(self) -> int:
        return self.N // self.T


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 0, 1, 2, 64, (4, 8, 8), (1, 4, 4), 16, (25,), (0.5,), "fp32",
                          backward=True),
    "layer_32k": Workload("layer_32k", 1, 1, 24, 128, (16, 32, 64), (1, 8, 8), 16, (10,), (0.5,), "bf16"),
    "long_524k": Workload("long_524k", 2, 1, 24, 128, (32, 128, 128), (1, 8, 8), 16, (5,), (1.0,), "bf16"),
    # same inputs and mask as layer_32k (seed 1), plus dO
    "train_32k": Workload("train_32k", 1, 1, 24, 128, (16, 32, 64), (1, 8, 8), 16, (10,), (0.5,), "bf16",
                          backward=True),
    "dynamic_55k": Workload("dynamic_55k", 4, 2, 16, 128, (24, 48, 48), (2, 4, 8), 16, (2, 5, 10, 25),
                            (0.2, 1.5), "bf16", backward=True, shuffle_keep=True),
}


def keep_to_k(percent: int, NB: int) -> int:
    """Blocks kept per query tile for a keep fraction given in percent.

    ceil(percent * NB / 100) in integer arithmetic, so 10 % of 512 is 52 and
    5 % of 8192 is 410 without any floating-point rounding question.
    """
    if percent <= 0 or percent > 100:
        raise ValueError("keep percent must be in (0, 100]")
    return max(1, min(NB, (percent * NB + 99) // 100))

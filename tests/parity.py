"""Helpers shared by the GPU parity tests: running the fp64 oracle on the same
bytes the GPU consumed, and the comparison rules.

Comparison rules (the library's specification):
* block indices: bit-exact per row, except where the oracle's fp64 scores of the
  last kept and first dropped non-own blocks differ by less than 1e-5 relative;
  in such a row every block in the symmetric difference must itself lie within
  1e-5 relative of that cut (a near-tie), and the structure must still hold;
* attention outputs and gradients: max-abs <= 1e-2 and relative Frobenius
  <= 5e-3 for bf16 inputs; both <= 1e-5 for fp32 inputs.  Outputs are compared
  in the kernels' fp32 store mode; the bf16 store must equal round-to-nearest-
  even of the fp32 store bit for bit.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle
from oracle import Geometry

BF16_MAX_ABS, BF16_REL_FRO = 1e-2, 5e-3
F32_MAX_ABS, F32_REL_FRO = 1e-5, 1e-5
TIE_REL = 1e-5


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def bounds(dtype: str) -> Tuple[float, float]:
    return (F32_MAX_ABS, F32_REL_FRO) if dtype == "fp32" else (BF16_MAX_ABS, BF16_REL_FRO)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> Dict[str, float]:
    max_abs_tol, rel_tol = bounds(dtype)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    assert max_abs <= max_abs_tol, f"{what}: max-abs {max_abs:.3e} > {max_abs_tol:.0e} (rel-fro {rel:.3e})"
    assert rel <= rel_tol, f"{what}: rel-frobenius {rel:.3e} > {rel_tol:.0e} (max-abs {max_abs:.3e})"
    return {"max_abs": max_abs, "rel_fro": rel}


def rne_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even to bf16 (torch's conversion), as raw int16 bits."""
    return x.to(torch.bfloat16).view(torch.int16)


def check_index_row(got: np.ndarray, scores: np.ndarray, tau: int, k: int, kmax: int) -> str:
    """'exact', 'exempt' or raises.  scores: the oracle's fp64 row."""
    NB = scores.shape[0]
    got = np.asarray(got)
    assert got.shape == (kmax,)
    sel = got[:k]
    assert (got[k:] == -1).all(), f"row {tau}: padding is not -1"
    assert (sel >= 0).all() and (sel < NB).all(), f"row {tau}: index out of range"
    assert (np.diff(sel) > 0).all(), f"row {tau}: not strictly ascending"
    assert tau in sel, f"row {tau}: own block missing"
    want = oracle.select_row(scores, tau, k)
    if np.array_equal(sel, want):
        return "exact"
    assert 1 < k < NB, f"row {tau}: k={k} has a unique answer but GPU {sel} != oracle {want}"
    others = np.array([j for j in range(NB) if j != tau])
    order = others[np.lexsort((others, -scores[others]))]
    s_in, s_out = scores[order[k - 2]], scores[order[k - 1]]
    band = TIE_REL * max(abs(s_in), abs(s_out))
    assert abs(s_in - s_out) < band, f"row {tau}: GPU {sel} != oracle {want} outside the tie band"
    for j in np.setxor1d(sel, want):
        assert abs(scores[j] - s_in) < TIE_REL * max(abs(scores[j]), abs(s_in)), \
            f"row {tau}: block {j} differs but is not a near-tie"
    return "exempt"


def layout_of(wl):
    from dynamic_sparse_attention_lowrank_amd import Layout
    return Layout(tuple(wl.latent), tuple(wl.tile))


def geom_of(wl) -> Geometry:
    return Geometry(*wl.latent, *wl.tile)


def sample_tiles(NB: int, n: int, seed: int) -> List[int]:
    """Deterministic sample of query tiles: always the first and last, then spread."""
    if n >= NB:
        return list(range(NB))
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, NB - 1), size=n - 2, replace=False)
    return sorted({0, NB - 1, *map(int, rest)})

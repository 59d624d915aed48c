"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

Nothing here computes any step of the attention method: it only draws numbers.

Random numbers
--------------
* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014), used counter-style: stream ``(seed, tag)`` starts at
  state ``s0 = mix(seed ^ mix(tag))`` and element ``i`` is ``mix(s0 + (i+1)*G)``
  with ``G = 0x9E3779B97F4A7C15`` -- exactly the i-th output of a SplitMix64
  generator started at ``s0``.  Any element can be computed independently.
* Uniforms take the top 53 bits: ``(x >> 11) * 2**-53``.
* Normals by Box & Muller (1958) on element pairs ``(2p, 2p+1)``:
  ``R = sqrt(-2 ln(1-u1))``, ``z0 = R cos(2 pi u2)``, ``z1 = R sin(2 pi u2)``.

Video-token structure
---------------------
The DSV page (gist.science/ar/paper/2502.07590, sections 2-3b) says neighbouring
tokens attend to the same things and that the pattern is data dependent; the
DiTango page (gist.science/de/paper/2607.15650) says attention is strongest for
nearby parts.  Q, K and V therefore carry a shared smooth random-Fourier-feature
term over the integer latent coordinates (t, y, x):

    F_h(t,y,x) = sqrt(2/32) * cos(Omega_h @ (t,y,x) + beta_h) @ P_h

with Omega_h in R^{32x3} ~ N(0, 0.3) (variance), beta_h ~ U[0, 2 pi)^32 and
P_h in R^{32xd} ~ N(0, 1).  Then Q = Z_Q + a F_h, K = Z_K + a F_h,
V = Z_V + a F_h with independent standard-normal Z, predictor weights
Wq, Wk ~ N(0, 1/d) per head, and dO ~ N(0, 1).  Every tensor is rounded once
(round-to-nearest-even) to its storage dtype; both sides of every comparison
read those same bytes.

All integer work is exact on any device.  The float part (log, cos, sin) is
evaluated in float64 on whichever device is asked; bytes can differ by a
rounding step between devices, so a test always generates once and hands the
same tensors to both sides.
"""
from __future__ import annotations

import hashlib
import math
from typing import Dict, Optional

import torch

from .configs import Workload, keep_to_k

_MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
CHUNK = 1 << 22          # elements per generation chunk (bounds temporary memory)


def _s64(u: int) -> int:
    """Unsigned 64-bit constant -> the int64 with the same bits."""
    u &= _MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _srl(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def mix64_tensor(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _s64(MIX1)
    z = (z ^ _srl(z, 27)) * _s64(MIX2)
    return z ^ _srl(z, 31)


def mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * MIX1) & _MASK64
    z = ((z ^ (z >> 27)) * MIX2) & _MASK64
    return z ^ (z >> 31)


def tag_of(name: str) -> int:
    """Fixed 64-bit stream tag for a tensor name."""
    return int.from_bytes(hashlib.sha256(name.encode()).digest()[:8], "little")


def stream_start(seed: int, tag: int) -> int:
    return mix64_int((seed & _MASK64) ^ mix64_int(tag))


def raw_u64(seed: int, tag: int, start: int, count: int, device) -> torch.Tensor:
    """Elements start..start+count-1 of stream (seed, tag), as int64 bit patterns."""
    s0 = _s64(stream_start(seed, tag))
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return mix64_tensor(s0 + i * _s64(GAMMA))


def uniform(seed: int, tag: int, start: int, count: int, device) -> torch.Tensor:
    x = raw_u64(seed, tag, start, count, device)
    return _srl(x, 11).to(torch.float64) * (2.0 ** -53)


def normal(seed: int, tag: int, count: int, device) -> torch.Tensor:
    """The first ``count`` standard normals (float64) of stream (seed, tag)."""
    return _normal_slice(seed, tag, 0, count + (count & 1), device)[:count]


def shuffled(seed: int, tag: int, items):
    """Fisher-Yates shuffle driven by the same counter stream."""
    items = list(items)
    n = len(items)
    s0 = stream_start(seed, tag)
    for i in range(n - 1, 0, -1):
        x = mix64_int(s0 + (n - 1 - i + 1) * GAMMA)
        j = x % (i + 1)
        items[i], items[j] = items[j], items[i]
    return items


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def fourier_features(wl: Workload, device) -> torch.Tensor:
    """F [H, N, d] float64 -- the shared locality term (see module docstring)."""
    H, d, nf = wl.H, wl.d, 32
    omega = normal(wl.seed, tag_of("rff.omega"), H * nf * 3, device).view(H, nf, 3) * math.sqrt(0.3)
    beta = uniform(wl.seed, tag_of("rff.beta"), 0, H * nf, device).view(H, nf) * (2.0 * math.pi)
    proj = normal(wl.seed, tag_of("rff.proj"), H * nf * d, device).view(H, nf, d)
    Lt, Lh, Lw = wl.latent
    # integer latent coordinates of every token, row-major (t, y, x); written column
    # by column (no tensor concatenation: a float64 concatenation kernel crashed
    # under a hardware-counter profiler)
    n = torch.arange(wl.N, device=device, dtype=torch.int64)
    coords = torch.empty(wl.N, 3, device=device, dtype=torch.float64)                   # [N, 3]
    coords[:, 0] = (n // (Lh * Lw)).to(torch.float64)
    coords[:, 1] = ((n // Lw) % Lh).to(torch.float64)
    coords[:, 2] = (n % Lw).to(torch.float64)
    F = torch.empty(H, wl.N, d, dtype=torch.float64, device=device)
    for h in range(H):
        phase = coords @ omega[h].T + beta[h]                                                # [N, 32]
        F[h] = math.sqrt(2.0 / nf) * (torch.cos(phase) @ proj[h])
    return F


def head_k(wl: Workload) -> torch.Tensor:
    """k per (b, h), int32 [B*H] (CPU)."""
    NB = wl.NB
    if wl.shuffle_keep:
        reps = -(-wl.H // len(wl.keep_percent))
        pool = list(wl.keep_percent) * reps
        perc = shuffled(wl.seed, tag_of("keep.shuffle"), pool)[: wl.H]
    else:
        perc = [wl.keep_percent[0]] * wl.H
    ks = [keep_to_k(p, NB) for p in perc]
    return torch.tensor([ks[h] for _ in range(wl.B) for h in range(wl.H)], dtype=torch.int32)


def generate(wl: Workload, device="cpu", with_grad: Optional[bool] = None,
             keep_override: Optional[int] = None, zero_q: bool = False) -> Dict[str, torch.Tensor]:
    """All inputs of one workload on ``device``.

    Returns Q, K, V [B,H,N,d], Wq, Wk [H,d,r], optionally dO [B,H,N,d] (storage
    dtype), and k [B*H] int32 on the CPU.  ``keep_override`` sets every k to one
    value (e.g. NB for keep = 1.0); ``zero_q`` replaces Q by zeros (a special
    case with a closed form).
    """
    dt = torch_dtype(wl.dtype)
    B, H, N, d, r = wl.B, wl.H, wl.N, wl.d, wl.r
    F = fourier_features(wl, device)
    amp = list(wl.amplitude) if len(wl.amplitude) == B else [wl.amplitude[0]] * B
    out: Dict[str, torch.Tensor] = {}
    for name in ("Q", "K", "V"):
        t = torch.empty(B, H, N, d, dtype=dt, device=device)
        for b in range(B):
            for h in range(H):
                # one stream per tensor; element index = flat position in [B,H,N,d]
                z = _normal_slice(wl.seed, tag_of("z." + name), (b * H + h) * N * d, N * d, device)
                t[b, h] = (z.view(N, d) + amp[b] * F[h]).to(dt)
        out[name] = t
    if zero_q:
        out["Q"].zero_()
    for name in ("Wq", "Wk"):
        w = normal(wl.seed, tag_of("w." + name), H * d * r, device).view(H, d, r) / math.sqrt(d)
        out[name] = w.to(dt)
    if with_grad is None:
        with_grad = wl.backward
    if with_grad:
        g = torch.empty(B, H, N, d, dtype=dt, device=device)
        for b in range(B):
            for h in range(H):
                z = _normal_slice(wl.seed, tag_of("z.dO"), (b * H + h) * N * d, N * d, device)
                g[b, h] = z.view(N, d).to(dt)
        out["dO"] = g
    k = head_k(wl)
    if keep_override is not None:
        k = torch.full_like(k, keep_override)
    out["k"] = k
    return out


def _normal_slice(seed: int, tag: int, start: int, count: int, device) -> torch.Tensor:
    """Normals start..start+count-1 of the stream (start and count even)."""
    assert start % 2 == 0 and count % 2 == 0
    out = torch.empty(count, dtype=torch.float64, device=device)
    npair = count // 2
    p0 = 0
    while p0 < npair:
        pc = min(CHUNK, npair - p0)
        u = uniform(seed, tag, start + 2 * p0, 2 * pc, device).view(pc, 2)
        rad = torch.sqrt(-2.0 * torch.log1p(-u[:, 0]))
        ang = (2.0 * math.pi) * u[:, 1]
        pair = out[2 * p0: 2 * (p0 + pc)].view(pc, 2)
        pair[:, 0] = rad * torch.cos(ang)
        pair[:, 1] = rad * torch.sin(ang)
        p0 += pc
    return out

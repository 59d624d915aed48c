"""Reference (oracle) for DSV-style dynamic block-sparse attention -- TEST INFRASTRUCTURE.

This module is the plain, slow, fp64 CPU statement of what the GPU library
computes.  It exists only to check the library: nothing in the product path
imports it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may use it.  It shares no code with the HIP kernels.

Method (DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video DiT
Training, gist.science/ar/paper/2502.07590):

* section 3a, low-rank predictor: before the expensive attention, a small cheap
  predictor estimates which part (about a tenth) of the attention matters;
* section 3b, query grouping: neighbouring tokens attend alike, so nearby tokens
  are grouped and share one selection;
* section 4 (stage two): the exact computation runs only on what the predictor
  selected.

The page gives no equations.  The readings used here (each one is listed with
its reason in the design notes of this repository):

* tokens are row-major over the (t, y, x) latent grid; a query tile and a key
  block are the same 3-D sub-box, so tile tau and block tau hold the same tokens;
* predictor: per head, rank-r projections Qh = Q Wq[h], Kh = K Wk[h], averaged
  over each tile (project, then pool), scored by the unscaled dot product
  S[tau, j] = Qbar[tau] . Kbar[j];
* selection: a query tile keeps its own block plus the k-1 best other blocks by
  score; equal scores go to the lower block index; the kept list is ascending,
  padded with -1;
* attention: exact softmax of (q . k) * scale over all keys of the kept blocks,
  scale = 1/sqrt(d), non-causal; LSE is a natural log;
* backward: the block mask is held fixed (no gradient reaches the predictor);
* predictor training (stage one, section 4): squared error of the scores against
  the pooled attention logits, gradient for Wq and Wk only;
* 3-D rotary positions (second page): per-axis rotary encoding of Q and K with a
  global time offset (see ``rope3d``).

Every array here is float64 (inputs are upcast exactly from their storage
dtype).  Library primitives used as steps: matrix products, argsort/lexsort,
exp/log.  No blocking, fusion or reordering beyond the definitions below.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# Geometry (query grouping, DSV page section 3b)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    Lt: int
    Lh: int
    Lw: int
    tt: int
    th: int
    tw: int

    @property
    def N(self) -> int:
        return self.Lt * self.Lh * self.Lw

    @property
    def T(self) -> int:
        """Tokens per tile (= per block)."""
        return self.tt * self.th * self.tw

    @property
    def grid(self) -> Tuple[int, int, int]:
        return (self.Lt // self.tt, self.Lh // self.th, self.Lw // self.tw)

    @property
    def NB(self) -> int:
        gt, gh, gw = self.grid
        return gt * gh * gw

    def check(self) -> None:
        if self.Lt % self.tt or self.Lh % self.th or self.Lw % self.tw:
            raise ValueError("tile extents must divide the latent extents")

    def token(self, t: int, y: int, x: int) -> int:
        """Row-major token index of latent coordinate (t, y, x)."""
        return (t * self.Lh + y) * self.Lw + x

    def tile_of(self, t: int, y: int, x: int) -> int:
        """Tile (= block) holding the token at (t, y, x); tiles are row-major too."""
        gt, gh, gw = self.grid
        return ((t // self.tt) * gh + (y // self.th)) * gw + (x // self.tw)

    def members(self) -> np.ndarray:
        """[NB, T] token indices of every tile, ascending within each tile."""
        self.check()
        out: List[List[int]] = [[] for _ in range(self.NB)]
        for t in range(self.Lt):
            for y in range(self.Lh):
                for x in range(self.Lw):
                    out[self.tile_of(t, y, x)].append(self.token(t, y, x))
        return np.asarray(out, dtype=np.int64)


# ----------------------------------------------------------------------------
# Predictor (DSV page section 3a): low-rank projection, tile-mean pooling, scores
# ----------------------------------------------------------------------------
def pooled_features(X: np.ndarray, W: np.ndarray, members: np.ndarray) -> np.ndarray:
    """Xbar[tau] = mean over the tokens n of tile tau of (X[n] @ W).

    X: [N, d] one head's Q or K; W: [d, r] that head's predictor weights.
    Project first, then pool.  Returns [NB, r].
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    projected = X @ W                                  # [N, r]
    return projected[members].mean(axis=1)             # [NB, r]


def block_scores(Qbar: np.ndarray, Kbar: np.ndarray) -> np.ndarray:
    """S[tau, j] = Qbar[tau] . Kbar[j] (unscaled).  Returns [NB, NB]."""
    return np.asarray(Qbar, np.float64) @ np.asarray(Kbar, np.float64).T


def predict_head(Q: np.ndarray, K: np.ndarray, Wq: np.ndarray, Wk: np.ndarray,
                 members: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    Qbar = pooled_features(Q, Wq, members)
    Kbar = pooled_features(K, Wk, members)
    return Qbar, Kbar, block_scores(Qbar, Kbar)


# ----------------------------------------------------------------------------
# Predictor training (DSV page section 4, stage one: the predictor is trained
# alongside the model so that it names the blocks that matter).  The page gives
# no loss.  Reading: the predictor's scores estimate the pooled attention logits,
# T[tau, j] = mean over query tokens i of tile tau and key tokens n of block j of
# q_i . k_n (the quantity a full-rank predictor would give), and stage one
# minimises the mean squared difference per (b, h):
#     loss = (1 / NB^2) * sum over tau, j of (S[tau, j] - T[tau, j])^2.
# Only the predictor weights receive a gradient.
# ----------------------------------------------------------------------------
def tile_means(X: np.ndarray, members: np.ndarray) -> np.ndarray:
    """P[tau] = mean over the tokens of tile tau of X[n].  Returns [NB, d]."""
    return np.asarray(X, dtype=np.float64)[members].mean(axis=1)


def pooled_logits(Q: np.ndarray, K: np.ndarray, members: np.ndarray) -> np.ndarray:
    """T[tau, j] = mean of q_i . k_n over i in tile tau, n in block j.

    The mean of the pairwise dot products equals the dot product of the two
    means (bilinearity), which is how it is evaluated here.  Returns [NB, NB].
    """
    return tile_means(Q, members) @ tile_means(K, members).T


def predictor_loss_head(Q, K, Wq, Wk, members: np.ndarray) -> float:
    """Stage-one loss of one (b, h): mean over all (tau, j) of (S - T)^2."""
    _, _, S = predict_head(Q, K, Wq, Wk, members)
    E = S - pooled_logits(Q, K, members)
    return float((E * E).sum() / E.size)


def predictor_grad_head(Q, K, Wq, Wk, members: np.ndarray):
    """(loss, dloss/dWq, dloss/dWk) of one (b, h); gradients [d, r].

    Chain rule through S = Qbar Kbar^T and Qbar = (tile mean of Q) Wq (the mean
    of the projections is the projection of the mean, so dQbar/dWq involves
    the tile means), likewise for Kbar.
    """
    Qbar, Kbar, S = predict_head(Q, K, Wq, Wk, members)
    E = S - pooled_logits(Q, K, members)
    loss = float((E * E).sum() / E.size)
    dS = 2.0 * E / E.size                              # d loss / d S
    dQbar = dS @ Kbar                                  # [NB, r]
    dKbar = dS.T @ Qbar
    dWq = tile_means(Q, members).T @ dQbar             # [d, r]
    dWk = tile_means(K, members).T @ dKbar
    return loss, dWq, dWk


def predictor_grad(Q, K, Wq, Wk, geom: "Geometry"):
    """loss [B,H] per (b, h); dWq, dWk [H,d,r] = gradients of the sum of all losses."""
    members = geom.members()
    B, H = Q.shape[:2]
    loss = np.zeros((B, H))
    dWq = np.zeros(np.shape(Wq))
    dWk = np.zeros(np.shape(Wk))
    for h in range(H):
        for b in range(B):
            loss[b, h], gq, gk = predictor_grad_head(Q[b, h], K[b, h], Wq[h], Wk[h], members)
            dWq[h] += gq
            dWk[h] += gk
    return loss, dWq, dWk


# ----------------------------------------------------------------------------
# 3-D rotary positions (second page, section 2: each frame's position in time is
# the start index of its chunk plus its index inside the chunk -- a global time
# index; with height and width this is a 3-D positional encoding).  The page
# gives no formula.  Reading: rotary encoding per axis -- the head dimension is
# cut into a time, a height and a width section of consecutive pairs (time takes
# what a three-way split leaves over: 22/21/21 pairs at d = 128); pair i of a
# section of 2m dimensions is rotated by the angle (position on that axis) *
# base^(-2i / 2m), base = 10000; positions are the latent coordinates plus an
# offset per axis (t0: the chunk's global start frame).  Applied to Q and K.
# ----------------------------------------------------------------------------
def rope_sections(d: int) -> Tuple[int, int, int]:
    """Pairs per axis (time, height, width)."""
    pairs = d // 2
    py = pairs // 3
    return pairs - 2 * py, py, py


def rope_angles(geom: "Geometry", d: int, base: float = 10000.0, offsets=(0, 0, 0)) -> np.ndarray:
    """Angle of every (token, pair): [N, d/2], fp64."""
    n = np.arange(geom.N)
    pos = (n // (geom.Lh * geom.Lw) + offsets[0], (n // geom.Lw) % geom.Lh + offsets[1], n % geom.Lw + offsets[2])
    cols = []
    for axis, m in enumerate(rope_sections(d)):
        for i in range(m):
            cols.append(pos[axis] * base ** (-2.0 * i / (2 * m)))
    return np.stack(cols, axis=1).astype(np.float64)


def rope3d(X: np.ndarray, geom: "Geometry", base: float = 10000.0, offsets=(0, 0, 0), inverse: bool = False):
    """Rotate every pair (X[n, 2p], X[n, 2p+1]) of one head's [N, d] rows by the
    token's angle for pair p (by minus that angle when ``inverse``)."""
    X = np.asarray(X, dtype=np.float64)
    a = rope_angles(geom, X.shape[1], base, offsets)
    if inverse:
        a = -a
    c, s = np.cos(a), np.sin(a)
    u, v = X[:, 0::2], X[:, 1::2]
    out = np.empty_like(X)
    out[:, 0::2] = u * c - v * s
    out[:, 1::2] = u * s + v * c
    return out


# ----------------------------------------------------------------------------
# Selection: top-k key blocks per query tile, own block forced in
# ----------------------------------------------------------------------------
def select_row(scores: np.ndarray, tau: int, k: int) -> np.ndarray:
    """Kept blocks of query tile ``tau``: itself plus the k-1 best others.

    Others are ranked by score descending, then block index ascending (so equal
    scores favour the lower index).  Returned ascending by block index.
    """
    scores = np.asarray(scores, dtype=np.float64)
    NB = scores.shape[0]
    if not 1 <= k <= NB:
        raise ValueError("k must be in [1, NB]")
    others = np.array([j for j in range(NB) if j != tau], dtype=np.int64)
    # np.lexsort sorts by the last key first: primary -score (descending score),
    # secondary block index (ascending).
    order = np.lexsort((others, -scores[others]))
    chosen = others[order[: k - 1]]
    return np.sort(np.concatenate(([tau], chosen)).astype(np.int64))


def select_head(S: np.ndarray, k: int, kmax: int) -> np.ndarray:
    """idx [NB, kmax] int32 for one head: ascending kept blocks, -1 padding."""
    NB = S.shape[0]
    if kmax < k:
        raise ValueError("kmax must be >= k")
    idx = np.full((NB, kmax), -1, dtype=np.int32)
    for tau in range(NB):
        idx[tau, :k] = select_row(S[tau], tau, k)
    return idx


# ----------------------------------------------------------------------------
# Block-sparse attention over the kept blocks (DSV page section 4, stage two)
# ----------------------------------------------------------------------------
def kept_keys(members: np.ndarray, blocks: Sequence[int]) -> np.ndarray:
    """Token indices of all keys in the kept blocks (block order, then token order)."""
    return np.concatenate([members[j] for j in blocks])


def attn_tile(Q: np.ndarray, K: np.ndarray, V: np.ndarray, members: np.ndarray,
              tau: int, blocks: Sequence[int], scale: float):
    """Forward for the queries of tile ``tau`` over the keys of ``blocks``.

    s_in = (q_i . k_n) * scale; P_in = exp(s_in - m_i) / l_i with
    m_i = max_n s_in and l_i = sum_n exp(s_in - m_i); O_i = sum_n P_in v_n;
    LSE_i = m_i + ln l_i.  Returns (O [T, d], LSE [T], P [T, nkeys], keys).
    """
    qi = members[tau]
    keys = kept_keys(members, blocks)
    s = (np.asarray(Q[qi], np.float64) @ np.asarray(K[keys], np.float64).T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    ell = e.sum(axis=1, keepdims=True)
    P = e / ell
    O = P @ np.asarray(V[keys], np.float64)
    LSE = (m + np.log(ell))[:, 0]
    return O, LSE, P, keys


def valid_blocks(idx_row: np.ndarray, k: int) -> List[int]:
    return [int(j) for j in idx_row[:k]]


def attn_fwd_head(Q, K, V, members: np.ndarray, idx: np.ndarray, k: int, scale: float,
                  tiles: Optional[Iterable[int]] = None):
    """O [N, d] and LSE [N] for one head (rows of tiles not in ``tiles`` stay NaN)."""
    N, d = np.asarray(Q).shape
    O = np.full((N, d), np.nan)
    LSE = np.full(N, np.nan)
    for tau in (range(members.shape[0]) if tiles is None else tiles):
        o, lse, _, _ = attn_tile(Q, K, V, members, tau, valid_blocks(idx[tau], k), scale)
        O[members[tau]] = o
        LSE[members[tau]] = lse
    return O, LSE


def attn_bwd_tile(Q, K, V, dO, members: np.ndarray, tau: int, blocks: Sequence[int], scale: float):
    """Gradients contributed by the queries of tile ``tau`` (mask held fixed).

    With the oracle's own O: D_i = dO_i . O_i, dP_in = dO_i . v_n,
    dS_in = P_in (dP_in - D_i); dQ_i = scale sum_n dS_in k_n;
    contributions dK_n += scale dS_in q_i and dV_n += P_in dO_i.
    Returns (dQ_tile [T, d], keys, dK_part [nkeys, d], dV_part [nkeys, d], dS).
    """
    O, _, P, keys = attn_tile(Q, K, V, members, tau, blocks, scale)
    qi = members[tau]
    g = np.asarray(dO[qi], np.float64)
    Dvec = (g * O).sum(axis=1, keepdims=True)
    dP = g @ np.asarray(V[keys], np.float64).T
    dS = P * (dP - Dvec)
    dQ = scale * (dS @ np.asarray(K[keys], np.float64))
    dK_part = scale * (dS.T @ np.asarray(Q[qi], np.float64))
    dV_part = P.T @ g
    return dQ, keys, dK_part, dV_part, dS


def attn_bwd_head(Q, K, V, dO, members: np.ndarray, idx: np.ndarray, k: int, scale: float):
    """dQ, dK, dV [N, d] for one head over every query tile."""
    N, d = np.asarray(Q).shape
    dQ = np.zeros((N, d))
    dK = np.zeros((N, d))
    dV = np.zeros((N, d))
    for tau in range(members.shape[0]):
        dq, keys, dk, dv, _ = attn_bwd_tile(Q, K, V, dO, members, tau, valid_blocks(idx[tau], k), scale)
        dQ[members[tau]] = dq
        np.add.at(dK, keys, dk)
        np.add.at(dV, keys, dv)
    return dQ, dK, dV


def attn_bwd_key_block(Q, K, V, dO, members: np.ndarray, idx: np.ndarray, k: int, scale: float, j: int):
    """dK, dV rows [T, d] of key block ``j`` only: sums over the query tiles that kept j."""
    T = members.shape[1]
    d = np.asarray(Q).shape[1]
    dK = np.zeros((T, d))
    dV = np.zeros((T, d))
    for tau in range(members.shape[0]):
        blocks = valid_blocks(idx[tau], k)
        if j not in blocks:
            continue
        _, keys, dk, dv, _ = attn_bwd_tile(Q, K, V, dO, members, tau, blocks, scale)
        pos = blocks.index(j) * T
        dK += dk[pos:pos + T]
        dV += dv[pos:pos + T]
    return dK, dV


# ----------------------------------------------------------------------------
# Whole-tensor helpers ([B, H, N, d] inputs, one k per (b, h))
# ----------------------------------------------------------------------------
def predict(Q, K, Wq, Wk, geom: Geometry):
    """Qbar, Kbar [B,H,NB,r] and S [B,H,NB,NB]."""
    members = geom.members()
    B, H = Q.shape[:2]
    r = Wq.shape[-1]
    Qbar = np.zeros((B, H, geom.NB, r))
    Kbar = np.zeros((B, H, geom.NB, r))
    S = np.zeros((B, H, geom.NB, geom.NB))
    for b in range(B):
        for h in range(H):
            Qbar[b, h], Kbar[b, h], S[b, h] = predict_head(Q[b, h], K[b, h], Wq[h], Wk[h], members)
    return Qbar, Kbar, S


def select(S: np.ndarray, k: Sequence[int], kmax: int) -> np.ndarray:
    """idx [B,H,NB,kmax] int32; k has one entry per (b, h), b-major."""
    B, H, NB, _ = S.shape
    idx = np.full((B, H, NB, kmax), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            idx[b, h] = select_head(S[b, h], int(k[b * H + h]), kmax)
    return idx


def attn_fwd(Q, K, V, idx, k, geom: Geometry, scale: float):
    members = geom.members()
    B, H, N, d = Q.shape
    O = np.zeros((B, H, N, d))
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = attn_fwd_head(Q[b, h], K[b, h], V[b, h], members, idx[b, h],
                                               int(k[b * H + h]), scale)
    return O, LSE


def attn_bwd(Q, K, V, dO, idx, k, geom: Geometry, scale: float):
    members = geom.members()
    B, H, N, d = Q.shape
    dQ = np.zeros((B, H, N, d))
    dK = np.zeros((B, H, N, d))
    dV = np.zeros((B, H, N, d))
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = attn_bwd_head(Q[b, h], K[b, h], V[b, h], dO[b, h], members,
                                                         idx[b, h], int(k[b * H + h]), scale)
    return dQ, dK, dV

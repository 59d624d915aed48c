"""Pins for the fp64 oracle: checks against facts that do not come from the oracle itself.

Each test names the fact it uses (a hand-written fixture, a closed form, brute
force on a tiny input, an independent textbook routine, an invariant, or a
finite-difference derivative).  No GPU needed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from dsa_inputs import WORKLOADS, generate
from dsa_inputs.configs import keep_to_k
import oracle
from oracle import Geometry

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def geom_of(wl):
    return Geometry(*wl.latent, *wl.tile)


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


@pytest.fixture(scope="module")
def tiny():
    wl = WORKLOADS["tiny_fp32"]
    x = generate(wl)
    return wl, {k: (f64(v) if v.is_floating_point() else v.numpy()) for k, v in x.items()}


# ---------------------------------------------------------------- geometry
def test_geometry_hand_fixture():
    """Hand-written members (tests/golden/tiny_geometry.json)."""
    g = json.load(open(os.path.join(GOLDEN, "tiny_geometry.json")))
    geom = Geometry(*g["latent"], *g["tile"])
    assert geom.NB == g["NB"]
    mem = geom.members()
    for tau, toks in g["members"].items():
        assert mem[int(tau)].tolist() == toks
    dyn = g["dynamic_55k_tile0"]
    geom2 = Geometry(*dyn["latent"], *dyn["tile"])
    assert geom2.NB == dyn["NB"]
    m0 = geom2.members()[0]
    runs = [m0[i * dyn["run_length"]:(i + 1) * dyn["run_length"]] for i in range(len(m0) // dyn["run_length"])]
    assert [int(r[0]) for r in runs] == [x[2] for x in dyn["first_run_per_frame_and_row"]]
    assert all((np.diff(r) == 1).all() for r in runs)


@pytest.mark.parametrize("name", ["tiny_fp32", "layer_32k", "dynamic_55k"])
def test_geometry_partition(name):
    """Every token lies in exactly one tile; each tile is a tt x th x tw box."""
    wl = WORKLOADS[name]
    geom = geom_of(wl)
    mem = geom.members()
    assert mem.shape == (wl.NB, wl.T)
    flat = np.sort(mem.reshape(-1))
    assert (flat == np.arange(wl.N)).all()
    Lt, Lh, Lw = wl.latent
    t, rem = np.divmod(mem, Lh * Lw)
    y, x = np.divmod(rem, Lw)
    for arr, ext in ((t, wl.tile[0]), (y, wl.tile[1]), (x, wl.tile[2])):
        assert ((arr.max(1) - arr.min(1)) == ext - 1).all()
        assert (arr.min(1) % ext == 0).all()
    assert (np.diff(mem, axis=1) > 0).all()


def test_block_counts():
    assert [WORKLOADS[n].NB for n in ("tiny_fp32", "layer_32k", "long_524k", "train_32k", "dynamic_55k")] == \
        [16, 512, 8192, 512, 864]
    assert keep_to_k(10, 512) == 52 and keep_to_k(5, 8192) == 410
    assert [keep_to_k(p, 864) for p in (2, 5, 10, 25)] == [18, 44, 87, 216]


# ---------------------------------------------------------------- generator
def test_splitmix64_known_answers():
    from dsa_inputs.generator import mix64_int, GAMMA, raw_u64
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))
    want = [int(h, 16) for h in g["outputs_hex"]]
    state, got = 0, []
    for _ in range(3):
        state = (state + GAMMA) & ((1 << 64) - 1)
        got.append(mix64_int(state))
    assert got == want
    # the vectorised torch version gives the same bits (stream started at state 0 <=> s0 = 0)
    from dsa_inputs import generator as G
    s0_zero = G._s64(0)
    i = torch.arange(1, 4, dtype=torch.int64)
    vec = G.mix64_tensor(s0_zero + i * G._s64(GAMMA))
    assert [int(v) & ((1 << 64) - 1) for v in vec] == want


def test_generator_moments(tiny):
    wl, x = tiny
    assert abs(x["Wq"].std() * math.sqrt(wl.d) - 1) < 0.05
    z = x["dO"].reshape(-1)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 1) < 0.02


# ---------------------------------------------------------------- predictor
def test_predictor_bruteforce_pairs(tiny):
    """P-1: S[tau, j] is the mean over all (query-token, key-token) pairs of the
    rank-r logits (q_i Wq) . (k_n Wk) -- computed pair by pair."""
    wl, x = tiny
    geom = geom_of(wl)
    mem = geom.members()
    for h in range(wl.H):
        Q, K, Wq, Wk = x["Q"][0, h], x["K"][0, h], x["Wq"][h], x["Wk"][h]
        _, _, S = oracle.predict_head(Q, K, Wq, Wk, mem)
        for tau in (0, 3, 7, 15):
            for j in (0, 5, 15):
                acc = 0.0
                for i in mem[tau]:
                    qi = Q[i] @ Wq
                    for n in mem[j]:
                        acc += float(qi @ (K[n] @ Wk))
                assert abs(S[tau, j] - acc / (len(mem[tau]) * len(mem[j]))) < 1e-12 * max(1.0, abs(acc))


def test_predictor_pool_then_project(tiny):
    """P-2: by linearity, pooling before projecting gives the same Qbar."""
    wl, x = tiny
    mem = geom_of(wl).members()
    Q, Wq = x["Q"][0, 1], x["Wq"][1]
    a = oracle.pooled_features(Q, Wq, mem)
    b = Q[mem].mean(axis=1) @ Wq
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_predictor_homogeneity(tiny):
    """P-3: scaling Wq by c scales S by c; swapping Q/K roles transposes S."""
    wl, x = tiny
    mem = geom_of(wl).members()
    Q, K, Wq, Wk = x["Q"][0, 0], x["K"][0, 0], x["Wq"][0], x["Wk"][0]
    _, _, S = oracle.predict_head(Q, K, Wq, Wk, mem)
    _, _, S3 = oracle.predict_head(Q, K, 3.0 * Wq, Wk, mem)
    assert np.abs(S3 - 3.0 * S).max() <= 1e-12 * np.abs(S).max()
    _, _, St = oracle.predict_head(K, Q, Wk, Wq, mem)
    assert np.abs(St - S.T).max() <= 1e-12 * np.abs(S).max()


# ---------------------------------------------------------------- predictor training
def _small_train_case(seed=5, d=6, r=3):
    """Tiny geometry (NB = 16 tiles of 4 tokens) with random fp64 Q, K, Wq, Wk."""
    geom = Geometry(2, 4, 8, 1, 2, 2)
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((geom.N, d))
    K = rng.standard_normal((geom.N, d)) + 0.5 * Q          # correlated, as attention inputs are
    Wq = rng.standard_normal((d, r)) / math.sqrt(d)
    Wk = rng.standard_normal((d, r)) / math.sqrt(d)
    return geom, geom.members(), Q, K, Wq, Wk


def test_pooled_logits_bruteforce_pairs():
    """T-1: T[tau, j] is the mean over all (query token, key token) pairs of q_i . k_n,
    computed pair by pair."""
    geom, mem, Q, K, _, _ = _small_train_case()
    T = oracle.pooled_logits(Q, K, mem)
    for tau in range(geom.NB):
        for j in (0, 3, 9, 15):
            acc = sum(float(Q[i] @ K[n]) for i in mem[tau] for n in mem[j])
            assert abs(T[tau, j] - acc / (len(mem[tau]) * len(mem[j]))) < 1e-12 * max(1.0, abs(acc))


def test_predictor_loss_special_cases():
    """T-2: Wq = 0 gives S = 0, so the loss is the mean of T^2; a full-rank
    predictor with Wq Wk^T = I reproduces T exactly (loss 0, gradients 0)."""
    geom, mem, Q, K, Wq, Wk = _small_train_case(d=6, r=6)
    T = oracle.pooled_logits(Q, K, mem)
    loss0 = oracle.predictor_loss_head(Q, K, np.zeros_like(Wq), Wk, mem)
    assert abs(loss0 - (T ** 2).mean()) <= 1e-12 * (T ** 2).mean()
    A = np.random.default_rng(1).standard_normal((6, 6)) + 3 * np.eye(6)
    loss, gq, gk = oracle.predictor_grad_head(Q, K, A, np.linalg.inv(A).T, mem)
    assert loss < 1e-24 and np.abs(gq).max() < 1e-12 and np.abs(gk).max() < 1e-12


def test_predictor_loss_quadratic_in_scale():
    """T-3: S is linear in Wq, so loss(c Wq) = a c^2 - 2 b c + loss(0) with
    a = mean(S^2), b = mean(S T) at c = 1."""
    geom, mem, Q, K, Wq, Wk = _small_train_case()
    _, _, S = oracle.predict_head(Q, K, Wq, Wk, mem)
    T = oracle.pooled_logits(Q, K, mem)
    a, b, t = (S * S).mean(), (S * T).mean(), (T * T).mean()
    for c in (-1.5, 0.3, 2.0):
        got = oracle.predictor_loss_head(Q, K, c * Wq, Wk, mem)
        assert abs(got - (a * c * c - 2 * b * c + t)) <= 1e-12 * max(1.0, t)


def test_predictor_grad_finite_differences():
    """T-4: the analytic gradient of the oracle equals central differences of
    its loss, entry by entry, for Wq and Wk."""
    geom, mem, Q, K, Wq, Wk = _small_train_case()
    _, gq, gk = oracle.predictor_grad_head(Q, K, Wq, Wk, mem)
    h = 1e-6
    for W, G, which in ((Wq, gq, 0), (Wk, gk, 1)):
        for e in range(W.shape[0]):
            for c in range(W.shape[1]):
                Wp, Wm = W.copy(), W.copy()
                Wp[e, c] += h
                Wm[e, c] -= h
                args_p = (Wp, Wk) if which == 0 else (Wq, Wp)
                args_m = (Wm, Wk) if which == 0 else (Wq, Wm)
                fd = (oracle.predictor_loss_head(Q, K, *args_p, mem) -
                      oracle.predictor_loss_head(Q, K, *args_m, mem)) / (2 * h)
                assert abs(fd - G[e, c]) <= 1e-7 * max(1.0, np.abs(G).max()), (which, e, c)


def test_predictor_grad_vanishes_at_least_squares_optimum():
    """T-5: for a fixed Wk the loss is a least-squares problem in Wq.  Its
    minimiser, Wq* = lstsq(Kbar-basis B = Pk Wk, Pk)^T (so that Wq* B^T is the
    projection of Pk^T onto the span of B), is computed by numpy's least squares;
    the oracle's dWq vanishes there and the loss does not drop nearby."""
    geom, mem, Q, K, Wq, Wk = _small_train_case(seed=9)
    Pk = K[mem].mean(axis=1)
    Bm = Pk @ Wk
    Wq_opt = np.linalg.lstsq(Bm, Pk, rcond=None)[0].T
    loss_opt, gq, _ = oracle.predictor_grad_head(Q, K, Wq_opt, Wk, mem)
    _, gq_rand, _ = oracle.predictor_grad_head(Q, K, Wq, Wk, mem)
    assert np.abs(gq).max() <= 1e-10 * np.abs(gq_rand).max()
    rng = np.random.default_rng(3)
    for _ in range(5):
        pert = Wq_opt + 1e-3 * rng.standard_normal(Wq_opt.shape)
        assert oracle.predictor_loss_head(Q, K, pert, Wk, mem) >= loss_opt


def test_predictor_grad_sums_over_batch(tiny):
    """T-6: the whole-tensor helper sums the per-(b, h) gradients over b."""
    wl, x = tiny
    geom = geom_of(wl)
    mem = geom.members()
    Q = np.concatenate([x["Q"], 0.5 * x["K"]], axis=0)     # B = 2
    K = np.concatenate([x["K"], x["Q"]], axis=0)
    loss, gq, gk = oracle.predictor_grad(Q, K, x["Wq"], x["Wk"], geom)
    for h in range(wl.H):
        parts = [oracle.predictor_grad_head(Q[b, h], K[b, h], x["Wq"][h], x["Wk"][h], mem) for b in range(2)]
        assert np.allclose(loss[:, h], [p[0] for p in parts], rtol=0, atol=0)
        assert np.abs(gq[h] - parts[0][1] - parts[1][1]).max() <= 1e-15 * np.abs(gq[h]).max()
        assert np.abs(gk[h] - parts[0][2] - parts[1][2]).max() <= 1e-15 * np.abs(gk[h]).max()


# ---------------------------------------------------------------- 3-D rotary positions
def test_rope_sections():
    """R-1: time, height and width sections of pairs; time takes the remainder."""
    assert oracle.rope_sections(128) == (22, 21, 21)
    assert oracle.rope_sections(64) == (12, 10, 10)
    assert oracle.rope_sections(6) == (1, 1, 1)


def test_rope_hand_cases():
    """R-2: with one pair per axis every frequency is 1, so token (t, y, x) turns
    (1, 0) into (cos p, sin p) and (0, 1) into (-sin p, cos p) for p = t, y, x; with
    two pairs per axis the second pair of a section turns by p * base^(-1/2)."""
    geom = Geometry(2, 3, 4, 1, 1, 1)
    n = (1 * 3 + 2) * 4 + 3                                       # (t, y, x) = (1, 2, 3)
    X = np.zeros((geom.N, 6))
    X[n] = [1, 0, 1, 0, 0, 1]
    Y = oracle.rope3d(X, geom)
    want = [math.cos(1), math.sin(1), math.cos(2), math.sin(2), -math.sin(3), math.cos(3)]
    assert np.abs(Y[n] - want).max() < 1e-15
    X2 = np.zeros((geom.N, 12))
    X2[n, 2] = 1.0                                                 # second time pair, x-component
    Y2 = oracle.rope3d(X2, geom, base=10000.0)
    assert abs(Y2[n, 2] - math.cos(0.01)) < 1e-15 and abs(Y2[n, 3] - math.sin(0.01)) < 1e-15
    Y3 = oracle.rope3d(X, geom, offsets=(4, 0, -3))                # offsets move the positions
    want3 = [math.cos(5), math.sin(5), math.cos(2), math.sin(2), -math.sin(0), math.cos(0)]
    assert np.abs(Y3[n] - want3).max() < 1e-15


def test_rope_relative_position_and_inverse():
    """R-3: rotations keep each pair's length, undo with the inverse, and q.k after
    rotation depends only on the difference of positions: shifting every position
    by the same offset leaves all dot products unchanged."""
    geom = Geometry(3, 4, 4, 1, 2, 2)
    rng = np.random.default_rng(2)
    Q = rng.standard_normal((geom.N, 16))
    K = rng.standard_normal((geom.N, 16))
    Qr, Kr = oracle.rope3d(Q, geom), oracle.rope3d(K, geom)
    assert np.abs((Qr[:, 0::2] ** 2 + Qr[:, 1::2] ** 2) - (Q[:, 0::2] ** 2 + Q[:, 1::2] ** 2)).max() < 1e-12
    assert np.abs(oracle.rope3d(Qr, geom, inverse=True) - Q).max() < 1e-12
    off = (7, -2, 5)
    G0 = Qr @ Kr.T
    G1 = oracle.rope3d(Q, geom, offsets=off) @ oracle.rope3d(K, geom, offsets=off).T
    assert np.abs(G0 - G1).max() < 1e-11 * np.abs(G0).max()
    # and it does change with a position difference (a shift of K alone)
    G2 = Qr @ oracle.rope3d(K, geom, offsets=(1, 0, 0)).T
    assert np.abs(G0 - G2).max() > 1e-3


def test_rope_global_time_index():
    """R-4: a chunk of frames s..s+c-1 rotated with time offset s equals those
    frames' rows of the whole clip rotated from 0 (position = chunk start + index)."""
    whole = Geometry(6, 4, 8, 1, 2, 2)
    chunk = Geometry(2, 4, 8, 1, 2, 2)
    rng = np.random.default_rng(4)
    X = rng.standard_normal((whole.N, 12))
    per_frame = whole.Lh * whole.Lw
    Yw = oracle.rope3d(X, whole)
    for s0 in (0, 2, 4):
        rows = slice(s0 * per_frame, (s0 + 2) * per_frame)
        Yc = oracle.rope3d(X[rows], chunk, offsets=(s0, 0, 0))
        assert np.abs(Yc - Yw[rows]).max() < 1e-13


# ---------------------------------------------------------------- selection
def brute_force_select(scores, tau, k):
    """Max-sum subset of k-1 other blocks; equal sums -> lexicographically smallest."""
    NB = len(scores)
    others = [j for j in range(NB) if j != tau]
    best, best_key = None, None
    for sub in itertools.combinations(others, k - 1):       # ascending tuples
        s = sum(scores[j] for j in sub)
        key = (-s, sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return sorted((tau,) + tuple(best))


@pytest.mark.parametrize("kind", ["gaussian", "integer_ties"])
def test_selection_bruteforce(kind):
    """Brute force over all C(15, 3) = 455 candidate subsets (NB = 16, k = 4)."""
    rng = np.random.default_rng(7)
    for trial in range(12):
        if kind == "gaussian":
            row = rng.standard_normal(16)
        else:
            row = rng.integers(-2, 3, size=16).astype(np.float64)   # many exact ties
        tau = int(rng.integers(0, 16))
        assert oracle.select_row(row, tau, 4).tolist() == brute_force_select(row, tau, 4)


def test_selection_invariants():
    """I-1 size k, I-2 ascending distinct, I-3 own block, I-4 threshold property."""
    rng = np.random.default_rng(3)
    NB = 40
    S = np.round(rng.standard_normal((NB, NB)), 1)    # rounding creates ties
    for k in (1, 2, 7, 39, 40):
        idx = oracle.select_head(S, k, kmax=k + 3)
        for tau in range(NB):
            row = idx[tau]
            sel = row[:k]
            assert (row[k:] == -1).all()
            assert len(sel) == k and (np.diff(sel) > 0).all()
            assert tau in sel and sel.min() >= 0 and sel.max() < NB
            chosen = [j for j in sel if j != tau]
            rest = [j for j in range(NB) if j != tau and j not in sel]
            if chosen and rest:
                worst_in = min(chosen, key=lambda j: (S[tau, j], -j))
                for j in rest:
                    assert S[tau, worst_in] > S[tau, j] or (S[tau, worst_in] == S[tau, j] and worst_in < j)


def test_selection_zero_scores_fixture():
    """Q = 0 gives S = 0; the hand-written fixture lists the lowest-index picks."""
    g = json.load(open(os.path.join(GOLDEN, "tiny_zero_q_selection.json")))
    S = np.zeros((g["NB"], g["NB"]))
    for tau, want in g["rows"].items():
        assert oracle.select_row(S[int(tau)], int(tau), g["k"]).tolist() == want


def test_selection_extremes():
    rng = np.random.default_rng(11)
    S = rng.standard_normal((16, 16))
    for tau in range(16):
        assert oracle.select_row(S[tau], tau, 16).tolist() == list(range(16))
        assert oracle.select_row(S[tau], tau, 1).tolist() == [tau]


# ---------------------------------------------------------------- forward
def dense_attention_torch(Q, K, V, scale):
    """Textbook dense softmax attention, written independently (torch fp64, CPU)."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)) for a in (Q, K, V))
    logits = (q @ k.transpose(0, 1)) * scale
    return (torch.softmax(logits, dim=-1) @ v).numpy(), torch.logsumexp(logits, dim=-1).numpy()


def test_keep_all_equals_dense(tiny):
    """k = NB (keep fraction 1.0) must equal dense attention (tiny workload)."""
    wl, x = tiny
    geom = geom_of(wl)
    mem = geom.members()
    scale = 1 / math.sqrt(wl.d)
    NB = geom.NB
    for h in range(wl.H):
        Q, K, V = x["Q"][0, h], x["K"][0, h], x["V"][0, h]
        idx = np.tile(np.arange(NB, dtype=np.int32), (NB, 1))
        O, LSE = oracle.attn_fwd_head(Q, K, V, mem, idx, NB, scale)
        Od, Ld = dense_attention_torch(Q, K, V, scale)
        assert np.abs(O - Od).max() < 1e-12
        assert np.abs(LSE - Ld).max() < 1e-12


def test_zero_query_closed_form(tiny):
    """Q = 0: uniform weights, so O is the mean of the kept V rows and LSE = ln(k T)."""
    wl, x = tiny
    geom = geom_of(wl)
    mem = geom.members()
    rng = np.random.default_rng(5)
    k = 4
    idx = np.full((geom.NB, k), -1, np.int32)
    for tau in range(geom.NB):
        others = rng.choice([j for j in range(geom.NB) if j != tau], k - 1, replace=False)
        idx[tau] = np.sort(np.concatenate(([tau], others)))
    Q = np.zeros_like(x["Q"][0, 0])
    O, LSE = oracle.attn_fwd_head(Q, x["K"][0, 0], x["V"][0, 0], mem, idx, k, 0.125)
    assert np.abs(LSE - 4.158883083359672).max() < 1e-12     # ln 64, 64 = 4 blocks x 16 tokens
    for tau in range(geom.NB):
        keys = np.concatenate([mem[j] for j in idx[tau]])
        want = x["V"][0, 0][keys].mean(axis=0)
        assert np.abs(O[mem[tau]] - want).max() < 1e-12


def test_constant_values_and_shift_invariance(tiny):
    """V = c gives O = c; adding one vector u to every key shifts each row's
    logits by a constant, leaving O unchanged and shifting LSE by scale q.u."""
    wl, x = tiny
    mem = geom_of(wl).members()
    Q, K, V = x["Q"][0, 1], x["K"][0, 1], x["V"][0, 1]
    S = oracle.predict_head(Q, K, x["Wq"][1], x["Wk"][1], mem)[2]
    idx = oracle.select_head(S, 5, 5)
    scale = 1 / math.sqrt(wl.d)
    O, LSE = oracle.attn_fwd_head(Q, K, np.full_like(V, 2.5), mem, idx, 5, scale)
    assert np.abs(O - 2.5).max() < 1e-12
    O1, L1 = oracle.attn_fwd_head(Q, K, V, mem, idx, 5, scale)
    u = np.random.default_rng(1).standard_normal(wl.d)
    O2, L2 = oracle.attn_fwd_head(Q, K + u, V, mem, idx, 5, scale)
    assert np.abs(O1 - O2).max() < 1e-11
    assert np.abs((L2 - L1) - scale * (Q @ u)).max() < 1e-11


def test_softmax_rows_sum_to_one(tiny):
    """I-5 rows of P sum to 1; I-6 the unnormalised sum is at least 1."""
    wl, x = tiny
    mem = geom_of(wl).members()
    scale = 1 / math.sqrt(wl.d)
    for tau in range(16):
        blocks = sorted({tau, (tau + 3) % 16, (tau + 7) % 16})
        _, LSE, P, keys = oracle.attn_tile(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], mem, tau, blocks, scale)
        assert np.abs(P.sum(1) - 1).max() < 1e-12
        s = x["Q"][0, 0][mem[tau]] @ x["K"][0, 0][keys].T * scale
        ell = np.exp(s - s.max(1, keepdims=True)).sum(1)
        assert (ell >= 1).all()


# ---------------------------------------------------------------- backward
def test_backward_finite_differences(tiny):
    """Central differences of L = sum(O * dO) in fp64 (step 1e-5)."""
    wl, x = tiny
    geom = geom_of(wl)
    mem = geom.members()
    h = 0
    Q, K, V, dO = (x[n][0, h].copy() for n in ("Q", "K", "V", "dO"))
    S = oracle.predict_head(Q, K, x["Wq"][h], x["Wk"][h], mem)[2]
    k = 4
    idx = oracle.select_head(S, k, k)
    scale = 1 / math.sqrt(wl.d)
    dQ, dK, dV = oracle.attn_bwd_head(Q, K, V, dO, mem, idx, k, scale)

    def loss(Qx, Kx, Vx):
        O, _ = oracle.attn_fwd_head(Qx, Kx, Vx, mem, idx, k, scale)
        return float((O * dO).sum())

    rng = np.random.default_rng(2)
    eps = 1e-5
    for name, grad in (("Q", dQ), ("K", dK), ("V", dV)):
        for _ in range(6):
            n, e = int(rng.integers(0, wl.N)), int(rng.integers(0, wl.d))
            args = {"Q": Q, "K": K, "V": V}
            plus = {kk: vv.copy() for kk, vv in args.items()}
            minus = {kk: vv.copy() for kk, vv in args.items()}
            plus[name][n, e] += eps
            minus[name][n, e] -= eps
            fd = (loss(plus["Q"], plus["K"], plus["V"]) - loss(minus["Q"], minus["K"], minus["V"])) / (2 * eps)
            assert abs(fd - grad[n, e]) < 1e-7 * max(1.0, abs(fd)), (name, n, e, fd, grad[n, e])


def test_backward_invariants(tiny):
    """I-7 sum_n dS_in = 0; I-8 sum dV = sum dO; I-9 sum dK = 0; I-10 in-degree >= 1."""
    wl, x = tiny
    mem = geom_of(wl).members()
    scale = 1 / math.sqrt(wl.d)
    for h in range(wl.H):
        Q, K, V, dO = (x[n][0, h] for n in ("Q", "K", "V", "dO"))
        S = oracle.predict_head(Q, K, x["Wq"][h], x["Wk"][h], mem)[2]
        idx = oracle.select_head(S, 4, 4)
        indeg = np.bincount(idx.reshape(-1), minlength=16)
        assert (indeg >= 1).all()
        for tau in range(16):
            *_, dS = oracle.attn_bwd_tile(Q, K, V, dO, mem, tau, list(idx[tau]), scale)
            assert np.abs(dS.sum(1)).max() < 1e-12
        dQ, dK, dV = oracle.attn_bwd_head(Q, K, V, dO, mem, idx, 4, scale)
        assert np.abs(dV.sum(0) - dO.sum(0)).max() < 1e-10
        assert np.abs(dK.sum(0)).max() < 1e-10
        # the per-key-block helper agrees with the full backward
        for j in (0, 9):
            dKj, dVj = oracle.attn_bwd_key_block(Q, K, V, dO, mem, idx, 4, scale, j)
            assert np.abs(dKj - dK[mem[j]]).max() < 1e-12 and np.abs(dVj - dV[mem[j]]).max() < 1e-12


def test_keep_all_gradients_equal_dense_autograd(tiny):
    """k = NB: gradients equal torch autograd of dense attention (fp64, CPU)."""
    wl, x = tiny
    mem = geom_of(wl).members()
    scale = 1 / math.sqrt(wl.d)
    h = 1
    Q, K, V, dO = (x[n][0, h] for n in ("Q", "K", "V", "dO"))
    idx = np.tile(np.arange(16, dtype=np.int32), (16, 1))
    dQ, dK, dV = oracle.attn_bwd_head(Q, K, V, dO, mem, idx, 16, scale)
    q, k, v = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    out = torch.softmax((q @ k.T) * scale, dim=-1) @ v
    (out * torch.from_numpy(dO)).sum().backward()
    for mine, ref in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-11


def test_whole_tensor_helpers_follow_batch_major_heads():
    """The [B, H, ...] helpers must hand head (b, h) its own tensors, its own
    weights Wq[h], Wk[h] and its own k = k[b*H + h] (b-major).  Every (b, h)
    below has different data and a different k, so a swapped b/h index, a k taken
    h-major, or weights taken per b would change some head's result; each head
    is compared with the pinned per-head functions called on hand-picked slices."""
    geom = Geometry(2, 4, 4, 1, 2, 2)                  # 32 tokens, 8 blocks of 4
    mem = geom.members()
    B, H, d, r = 2, 3, 8, 4
    rng = np.random.default_rng(11)
    Q, K, V, dO = (rng.standard_normal((B, H, geom.N, d)) for _ in range(4))
    Wq, Wk = rng.standard_normal((H, d, r)), rng.standard_normal((H, d, r))
    k = np.array([1, 3, 5, 8, 2, 6], dtype=np.int32)   # k[b*H + h]: all different
    kmax = int(k.max())
    scale = 1 / math.sqrt(d)
    Qb, Kb, S = oracle.predict(Q, K, Wq, Wk, geom)
    idx = oracle.select(S, k, kmax)
    O, LSE = oracle.attn_fwd(Q, K, V, idx, k, geom, scale)
    dQ, dK, dV = oracle.attn_bwd(Q, K, V, dO, idx, k, geom, scale)
    for b in range(B):
        for h in range(H):
            kk = int(k[b * H + h])
            qb, kb, s = oracle.predict_head(Q[b, h], K[b, h], Wq[h], Wk[h], mem)
            assert np.array_equal(Qb[b, h], qb) and np.array_equal(Kb[b, h], kb) and np.array_equal(S[b, h], s)
            ih = oracle.select_head(s, kk, kmax)
            assert np.array_equal(idx[b, h], ih)
            assert (idx[b, h, :, kk:] == -1).all() and (idx[b, h, :, :kk] >= 0).all()
            o, lse = oracle.attn_fwd_head(Q[b, h], K[b, h], V[b, h], mem, ih, kk, scale)
            assert np.array_equal(O[b, h], o) and np.array_equal(LSE[b, h], lse)
            g = oracle.attn_bwd_head(Q[b, h], K[b, h], V[b, h], dO[b, h], mem, ih, kk, scale)
            for got, want in zip((dQ[b, h], dK[b, h], dV[b, h]), g):
                assert np.array_equal(got, want)
    # k = NB for head (1, 0): every block kept, so that head is plain dense attention
    b, h = 1, 0
    s = Q[b, h] @ K[b, h].T * scale
    p = np.exp(s - s.max(1, keepdims=True))
    assert np.allclose(O[b, h], (p / p.sum(1, keepdims=True)) @ V[b, h], rtol=1e-12, atol=1e-12)

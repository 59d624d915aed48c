"""Both bf16 forward kernels (one-tile and tile-pair) against the fp64 oracle.

By default the library runs the tile-pair kernel only when one head's gathered
blocks reach 48 MiB, so at sizes the oracle finishes in seconds it would always
run the one-tile kernel.  These cases pick each kernel explicitly
(dsa_set_fwd_kernel) on geometries that exercise the pairing: an odd number of
tiles along the pairing axis (the last tile has no partner), pairing along the
height or the width axis when there is one time step, a single tile, tiles of
32 and fewer queries (a key half with no valid key), T = 64 at d = 64, a head
that keeps every block, unsorted index rows (the union walk then shares fewer
blocks but must stay exact) and the no-allocation entry point.  Attention runs
on the oracle's own block selection.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import WORKLOADS, generate
from parity import assert_close, f64, geom_of, layout_of, rne_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dynamic_sparse_attention_lowrank_amd as m
    yield m
    m.set_fwd_kernel(m.FWD_AUTO)


def case(name, **kw):
    base = dict(B=1, H=2, d=128, tile=(1, 8, 8), keep_percent=(25,), dtype="bf16", amplitude=(0.5,))
    base.update(kw)
    return dataclasses.replace(WORKLOADS["tiny_fp32"], name=name, **base)


CASES = [
    case("odd_time_tiles", seed=31, latent=(5, 16, 16)),                       # pairs (0,1) (2,3) (4,-)
    case("pairs_along_height", seed=32, latent=(1, 24, 16)),                   # one time step, 3 x 2 tiles
    case("pairs_along_width", seed=33, latent=(1, 8, 40)),                     # one tile row of 5
    case("single_tile", seed=34, latent=(1, 8, 8)),
    case("d64_t32", seed=35, d=64, latent=(4, 8, 16), tile=(1, 4, 8)),         # upper key half empty
    case("d64_t64", seed=36, d=64, latent=(3, 16, 16), tile=(1, 8, 8), keep_percent=(30,)),
    case("t12_ragged", seed=37, latent=(4, 9, 8), tile=(1, 3, 4), keep_percent=(40,)),
    case("vark_keep_all", seed=38, B=2, H=3, latent=(6, 12, 8), tile=(2, 3, 8), keep_percent=(5, 50, 100),
         shuffle_keep=True, amplitude=(0.2, 1.5)),
]


def _say(msg):
    print(msg, flush=True)


def oracle_selection(x, wl):
    """The oracle's predictor scores and top-k selection per head, as idx [B,H,NB,kmax]."""
    geom = geom_of(wl)
    mem = geom.members()
    ks = x["k"].tolist()
    kmax = max(ks)
    idx = np.full((wl.B, wl.H, geom.NB, kmax), -1, np.int32)
    for b in range(wl.B):
        for h in range(wl.H):
            _, _, S = oracle.predict_head(f64(x["Q"][b, h]), f64(x["K"][b, h]), f64(x["Wq"][h]), f64(x["Wk"][h]), mem)
            idx[b, h] = oracle.select_head(S, ks[b * wl.H + h], kmax)
    return mem, ks, idx


def run_fwd(dsa, kind, x, idx_d, kdev, lay, out_dtype):
    dsa.set_fwd_kernel(kind)
    try:
        return dsa.attn_fwd(x["Q"], x["K"], x["V"], idx_d, kdev, lay, out_dtype=out_dtype)
    finally:
        dsa.set_fwd_kernel(dsa.FWD_AUTO)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_forward_kernels_match_oracle(dsa, wl):
    _say(f"case {wl.name}: B={wl.B} H={wl.H} d={wl.d} latent={wl.latent} tile={wl.tile}")
    x = generate(wl, device="cuda", with_grad=False)
    lay = layout_of(wl)
    kdev = x["k"].cuda()
    mem, ks, idx_o = oracle_selection(x, wl)
    idx_d = torch.from_numpy(idx_o).cuda()
    res = {}
    for kind in (dsa.FWD_ONE_TILE, dsa.FWD_TILE_PAIR):
        O32, LSE = run_fwd(dsa, kind, x, idx_d, kdev, lay, torch.float32)
        Obf, LSE2 = run_fwd(dsa, kind, x, idx_d, kdev, lay, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(rne_bf16(O32), Obf.view(torch.int16)), f"kernel {kind}: bf16 store != RNE(fp32 store)"
        assert torch.equal(LSE, LSE2)
        res[kind] = (O32, LSE)
    scale = 1.0 / math.sqrt(wl.d)
    for b in range(wl.B):
        for h in range(wl.H):
            Q, K, V = (f64(x[n][b, h]) for n in ("Q", "K", "V"))
            Oo, Lo = oracle.attn_fwd_head(Q, K, V, mem, idx_o[b, h], ks[b * wl.H + h], scale)
            for kind, (O32, LSE) in res.items():
                assert_close(f64(O32[b, h]), Oo, "bf16", f"kernel {kind} O[{b},{h}]")
                assert_close(f64(LSE[b, h]), Lo, "bf16", f"kernel {kind} LSE[{b},{h}]")


def test_tile_pair_unsorted_rows(dsa):
    """Index rows in a shuffled order: the tile-pair kernel still attends to exactly
    the kept blocks (a block kept by both tiles may then be gathered twice)."""
    wl = CASES[0]
    x = generate(wl, device="cuda", with_grad=False)
    lay = layout_of(wl)
    kdev = x["k"].cuda()
    mem, ks, idx_o = oracle_selection(x, wl)
    rng = np.random.default_rng(7)
    idx_s = idx_o.copy()
    for b in range(wl.B):
        for h in range(wl.H):
            k = ks[b * wl.H + h]
            for tau in range(idx_s.shape[2]):
                idx_s[b, h, tau, :k] = rng.permutation(idx_s[b, h, tau, :k])
    assert not np.array_equal(idx_s, idx_o)
    O, LSE = run_fwd(dsa, dsa.FWD_TILE_PAIR, x, torch.from_numpy(idx_s).cuda(), kdev, lay, torch.float32)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(wl.d)
    for h in range(wl.H):
        Q, K, V = (f64(x[n][0, h]) for n in ("Q", "K", "V"))
        Oo, Lo = oracle.attn_fwd_head(Q, K, V, mem, idx_o[0, h], ks[h], scale)
        assert_close(f64(O[0, h]), Oo, "bf16", f"O[0,{h}]")
        assert_close(f64(LSE[0, h]), Lo, "bf16", f"LSE[0,{h}]")


def test_tile_pair_noalloc_matches(dsa):
    """dsa_attn_fwd_noalloc runs the chosen kernel too: bit-identical to dsa_attn_fwd."""
    wl = CASES[-1]
    x = generate(wl, device="cuda", with_grad=False)
    lay = layout_of(wl)
    kdev = x["k"].cuda()
    _, _, idx_o = oracle_selection(x, wl)
    idx_d = torch.from_numpy(idx_o).cuda()
    dsa.set_fwd_kernel(dsa.FWD_TILE_PAIR)
    try:
        O1, L1 = dsa.attn_fwd(x["Q"], x["K"], x["V"], idx_d, kdev, lay, out_dtype=torch.float32)
        O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
        dsa.attn_fwd_noalloc(x["Q"], x["K"], x["V"], idx_d, kdev, lay, out=(O2, L2))
        torch.cuda.synchronize()
    finally:
        dsa.set_fwd_kernel(dsa.FWD_AUTO)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)

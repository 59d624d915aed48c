"""The Python binding checks every tensor's shape, dtype and device before it
calls the library, so a short or mis-typed buffer never reaches a kernel.  All
cases here fail on the host (CPU tensors; no GPU and no kernel launch needed)."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dsa():
    if not os.path.exists(os.path.join(ROOT, "dynamic_sparse_attention_lowrank_amd", "libdsa.so")):
        from dynamic_sparse_attention_lowrank_amd import build as b
        b.build()
    import dynamic_sparse_attention_lowrank_amd as m
    return m


B, H, d, r, kmax = 1, 2, 64, 16, 4
LAT, TILE = (4, 8, 8), (1, 4, 4)          # 256 tokens, 16 blocks
N, NB = 256, 16


def base(dtype=torch.bfloat16):
    t = lambda *s, dt=dtype: torch.zeros(*s, dtype=dt)
    return dict(Q=t(B, H, N, d), K=t(B, H, N, d), V=t(B, H, N, d), dO=t(B, H, N, d),
                Wq=t(H, d, r), Wk=t(H, d, r), idx=t(B, H, NB, kmax, dt=torch.int32), k=t(B * H, dt=torch.int32),
                O=t(B, H, N, d, dt=torch.float32), LSE=t(B, H, N, dt=torch.float32))


def fwd(dsa, x, **over):
    x = dict(x, **over)
    lay = dsa.Layout(LAT, TILE)
    out = over.get("out")
    return dsa.attn_fwd(x["Q"], x["K"], x["V"], x["idx"], x["k"], lay, out=out, workspace=over.get("workspace"))


@pytest.mark.parametrize("what,bad,msg", [
    ("K", torch.zeros(B, H, N, d + 64, dtype=torch.bfloat16), "K: shape"),
    ("V", torch.zeros(B, H, N, d, dtype=torch.float32), "V: dtype"),
    ("idx", torch.zeros(B, H, NB, kmax, dtype=torch.int64), "idx: dtype"),
    ("idx", torch.zeros(B, H, NB - 1, kmax, dtype=torch.int32), "idx: shape"),
    ("k", torch.zeros(B * H, dtype=torch.int64), "k: dtype"),
    ("k", torch.zeros(B * H + 1, dtype=torch.int32), "k: shape"),
    ("Q", torch.zeros(B, H, N - 16, d, dtype=torch.bfloat16), "tokens"),
    ("Q", torch.zeros(B, H, N, d, dtype=torch.float16), "Q: dtype"),
])
def test_forward_rejects_bad_tensors(dsa, what, bad, msg):
    with pytest.raises(ValueError, match=msg):
        fwd(dsa, base(), **{what: bad})


def test_forward_rejects_bad_outputs_and_workspace(dsa):
    x = base()
    with pytest.raises(ValueError, match="O: shape"):
        fwd(dsa, x, out=(torch.zeros(B, H, N, d // 2), torch.zeros(B, H, N)))
    with pytest.raises(ValueError, match="LSE: dtype"):
        fwd(dsa, x, out=(torch.zeros(B, H, N, d), torch.zeros(B, H, N, dtype=torch.float64)))
    with pytest.raises(ValueError, match="bytes"):
        fwd(dsa, x, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="uint8"):
        fwd(dsa, x, workspace=torch.zeros(1 << 20, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):                       # everything else valid: the device
        fwd(dsa, x)


def test_predictor_and_selection_reject_bad_tensors(dsa):
    x = base()
    lay = dsa.Layout(LAT, TILE)
    with pytest.raises(ValueError, match="Wk: shape"):
        dsa.predict(x["Q"], x["K"], x["Wq"], torch.zeros(H, d, r + 1, dtype=torch.bfloat16), lay)
    with pytest.raises(ValueError, match="Wq: dtype"):
        dsa.predict(x["Q"], x["K"], x["Wq"].float(), x["Wk"], lay)
    with pytest.raises(ValueError, match="S: shape"):
        dsa.predict(x["Q"], x["K"], x["Wq"], x["Wk"], lay,
                    out=(torch.zeros(B, H, NB, r), torch.zeros(B, H, NB, r), torch.zeros(B, H, NB, NB - 1)))
    with pytest.raises(ValueError, match="S: shape"):
        dsa.select(torch.zeros(B, H, NB, NB - 1), x["k"], kmax, lay, d=d)
    with pytest.raises(ValueError, match="idx: shape"):
        dsa.select(torch.zeros(B, H, NB, NB), x["k"], kmax, lay, d=d,
                   out=torch.zeros(B, H, NB, kmax + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="k: dtype"):
        dsa.predict_select(x["Q"], x["K"], x["Wq"], x["Wk"], x["k"].long(), kmax, lay)
    with pytest.raises(ValueError, match="dWq: dtype"):
        dsa.predictor_grad(x["Q"], x["K"], x["Wq"], x["Wk"], lay,
                           out=(torch.zeros(B, H), torch.zeros(H, d, r, dtype=torch.bfloat16), torch.zeros(H, d, r)))
    with pytest.raises(ValueError, match="out: dtype"):
        dsa.rope3d(x["Q"], lay, out=torch.zeros(B, H, N, d))


def test_backward_rejects_bad_tensors(dsa):
    x = base()
    lay = dsa.Layout(LAT, TILE)
    args = lambda **o: [dict(x, **o)[n] for n in ("Q", "K", "V", "O", "dO", "LSE", "idx", "k")]
    with pytest.raises(ValueError, match="O: dtype"):                  # the bf16 forward output is refused
        dsa.attn_bwd(*args(O=torch.zeros(B, H, N, d, dtype=torch.bfloat16)), lay)
    with pytest.raises(ValueError, match="dO: dtype"):
        dsa.attn_bwd(*args(dO=torch.zeros(B, H, N, d)), lay)
    with pytest.raises(ValueError, match="LSE: shape"):
        dsa.attn_bwd(*args(LSE=torch.zeros(B, H, N + 1)), lay)
    with pytest.raises(ValueError, match="dK: dtype"):
        dsa.attn_bwd(*args(), lay, out=(torch.zeros(B, H, N, d), torch.zeros(B, H, N, d, dtype=torch.bfloat16),
                                         torch.zeros(B, H, N, d)))
    ws = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="bytes"):
        dsa.attn_bwd_prepare(x["O"], x["dO"], x["idx"], x["k"], lay, ws)
    with pytest.raises(ValueError, match="dV: shape"):
        dsa.attn_bwd_dkdv(x["Q"], x["K"], x["V"], x["dO"], x["LSE"], kmax, lay, ws, torch.zeros(B, H, N, d),
                          torch.zeros(B, H, N, d // 2))
    with pytest.raises(ValueError, match="idx: dtype"):
        dsa.attn_bwd_dq(x["Q"], x["K"], x["V"], x["dO"], x["LSE"], x["idx"].long(), x["k"], lay, ws,
                        torch.zeros(B, H, N, d))
    with pytest.raises(ValueError, match="GPU"):
        dsa.attn_bwd(*args(), lay)

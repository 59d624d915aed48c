"""dsa_attn_fwd_noalloc -- the forward for callers that cannot allocate (its
workspace is the library's fixed per-GPU scratch array) -- against dsa_attn_fwd,
through the C ABI: O and LSE must be bit-identical.  Two calls in a row on one
GPU, the second with a smaller input: first the 32,768-token layer (24 heads, bf16,
d = 128: the heads run in two groups through the 144 MiB array), then the tiny
fp32 case (2 heads, d = 64) and a bf16 d = 64 case, with bf16 and fp32 outputs;
the array keeps the previous call's contents, which must not matter."""
import dataclasses
import math

import pytest
import torch

import dynamic_sparse_attention_lowrank_amd as dsa
from dsa_inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu


# a bf16 case with 16-token tiles (T < 64), d = 64 and an odd head count
EXTRA = {"bf16_d64_t16": dataclasses.replace(WORKLOADS["tiny_fp32"], name="bf16_d64_t16", seed=12, B=1, H=3, d=64,
                                             latent=(5, 8, 12), tile=(1, 4, 4), keep_percent=(20,), dtype="bf16")}


def _inputs(name):
    wl = EXTRA.get(name) or WORKLOADS[name]
    dev = torch.device("cuda:0")
    x = generate(wl, device=dev, with_grad=False)
    lay = dsa.Layout(tuple(wl.latent), tuple(wl.tile))
    kdev = x["k"].to(dev)
    kmax = int(x["k"].max())
    _, _, idx = dsa.predict_select(x["Q"], x["K"], x["Wq"], x["Wk"], kdev, kmax, lay)
    return x, lay, kdev, idx


def _compare(name, out_dtype):
    x, lay, kdev, idx = _inputs(name)
    Q, K, V = x["Q"], x["K"], x["V"]
    print(f"case {name}: shape {tuple(Q.shape)} {Q.dtype} -> O {out_dtype}", flush=True)
    O1, L1 = dsa.attn_fwd(Q, K, V, idx, kdev, lay, out_dtype=out_dtype)
    O2 = torch.full(Q.shape, math.nan, device=Q.device, dtype=out_dtype)
    L2 = torch.full(Q.shape[:3], math.nan, device=Q.device, dtype=torch.float32)
    dsa.attn_fwd_noalloc(Q, K, V, idx, kdev, lay, out=(O2, L2))
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16) if out_dtype == torch.bfloat16 else O1.view(torch.int32),
                       O2.view(torch.int16) if out_dtype == torch.bfloat16 else O2.view(torch.int32)), \
        f"{name}: O differs from dsa_attn_fwd"
    assert torch.equal(L1.view(torch.int32), L2.view(torch.int32)), f"{name}: LSE differs from dsa_attn_fwd"
    return Q.shape


def test_noalloc_forward_matches_forward_on_consecutive_calls():
    big = _compare("layer_32k", torch.bfloat16)                # 24 heads: groups of 17 and 7
    small = _compare("tiny_fp32", torch.float32)               # then a smaller input on the same scratch
    assert small.numel() < big.numel()
    _compare("bf16_d64_t16", torch.float32)
    print("noalloc forward: bit-identical to dsa_attn_fwd on three consecutive calls", flush=True)


def test_noalloc_forward_rejects_heads_beyond_the_scratch():
    # one bf16 head of 9,216 key blocks at d = 128 needs 144 MiB + 512 B: rejected
    # on the host before any device work
    Q = torch.empty((1, 1, 96 * 96 * 64, 128), device="cuda:0", dtype=torch.bfloat16)
    lay = dsa.Layout((1, 768, 768), (1, 8, 8))
    idx = torch.zeros((1, 1, 9216, 1), device="cuda:0", dtype=torch.int32)
    kdev = torch.ones(1, device="cuda:0", dtype=torch.int32)
    O = torch.empty_like(Q)
    LSE = torch.empty(Q.shape[:3], device="cuda:0", dtype=torch.float32)
    with pytest.raises(dsa.DsaError) as e:
        dsa.attn_fwd_noalloc(Q, Q, Q, idx, kdev, lay, out=(O, LSE))
    assert e.value.status == 10

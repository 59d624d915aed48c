#!/usr/bin/env python3
"""Benchmark: one training step of DSV-style dynamic block-sparse attention on one MI355X.

A step is one pass of the whole path over one batch of synthetic video tokens:
pooled low-rank predictor -> top-k block selection (scores formed per row, no
score matrix; --score-matrix times the two-step path) -> block-sparse attention
forward -> backward (D + reverse index, dK/dV, dQ).  Workload: B=1, H=24, d=128, latent
16x32x64 = 32,768 tokens, 1x8x8 tiles (512 blocks), rank 16, 10 % of the blocks
kept (k = 52), bf16 inputs.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is attended TFLOP/s of the whole step with the
attended work counted as 4*d FLOP per (query, key) pair forward and 10*d
backward (workloads without a backward: forward only).  `headline` is the
layer's forward alone, the median of 20 repetitions each after a 512 MiB
cache-evicting write (L2 and memory-attached cache cold); `fwd` gives the same
call warm, inside the steps.  `roofline` describes the dominant kernel (its
algorithmic FLOP: forward 4*d, dK/dV 8*d, dQ 2*d per pair -- the dQ pass's
recomputation of S and dP is not counted), timed with HIP events on the stream
it runs on, beside the average duration of the same kernel in the committed
rocprofv3 trace when that trace was taken on the current sources;
`bwd_roofline` is the whole backward at 10*d.  `cpu_baseline` times the fp64
oracle per phase on a bounded sample of this workload and of the other
configurations (one GPU only).  `phase_stats_ms` gives the median / min / max
of every phase over the timed steps, `clocks` the engine / memory clock levels
read from sysfs before and after.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-sparse attn ms/layer + attended TFLOP/s (% bf16 MFMA peak), 32,768 tok"
BF16_PEAK_TFLOPS = 2500.0          # MI355X dense bf16 matrix peak (published)
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train_32k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--cpu-configs", default="tiny_fp32,layer_32k,long_524k,dynamic_55k",
                    help="other configurations the oracle baseline also samples (comma list; empty: none)")
    ap.add_argument("--cpu-config-seconds", type=float, default=3.0,
                    help="oracle budget per configuration of --cpu-configs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="repetitions of the forward alone after a 512 MiB cache-evicting write (the headline)")
    ap.add_argument("--score-matrix", action="store_true",
                    help="predict (writes the NB x NB scores) then select, instead of the fused entry point")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one int32 bitwise-not of this many MiB (a plain streaming "
                         "kernel of known traffic, the HBM counter calibration)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 output under DIR and exit "
                         "(DIR/trace, DIR/fetch, DIR/write, each with the bench JSON line in out.json "
                         "and the command in cmd.txt)")
    return ap.parse_args()


def stats(v):
    """median / min / max of a list of times in ms"""
    import numpy as np
    return {"median": round(float(np.median(v)), 4), "min": round(float(min(v)), 4), "max": round(float(max(v)), 4)}


def read_clocks():
    """Current engine and memory clock levels (MHz) of each GPU from sysfs, or None
    where the files are not readable."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        card = {}
        for name in ("sclk", "mclk"):
            try:
                for line in open(os.path.join(dev, f"pp_dpm_{name}")):
                    if "*" in line:
                        card[name] = int("".join(ch for ch in line.split(":")[1] if ch.isdigit()))
            except (OSError, ValueError, IndexError):
                pass
        if card:
            out[os.path.basename(os.path.dirname(dev))] = card
    return out or None


def pct_at_clock(tflops, c0, c1):
    """Percentage of the bf16 matrix peak scaled to the mean engine clock read before
    and after the timed region (the published peak assumes 2.4 GHz), or None."""
    vals = [c["sclk"] for c in (c0 or {}).values() if "sclk" in c] + \
           [c["sclk"] for c in (c1 or {}).values() if "sclk" in c]
    if not vals:
        return None
    mhz = sum(vals) / len(vals)
    return round(100 * tflops / (BF16_PEAK_TFLOPS * mhz / 2400.0), 2)


def source_hash() -> str:
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_lowrank_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, prof_dir: Optional[str] = None):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(prof_dir or os.path.join(ROOT, "profiles"), f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def load_trace_avg_us(kernel: str, workload: str, prof_dir: Optional[str] = None):
    """Average duration (us) of the kernel's bf16 d = 128 variant in the committed
    rocprofv3 kernel-trace summary, if that summary was taken on the current kernel
    sources (else None)."""
    path = os.path.join(prof_dir or os.path.join(ROOT, "profiles"), f"{workload}_kernel_trace.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"source_hash {source_hash()}" not in text:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and cells[0].startswith(kernel + "<bf16,128"):
            try:
                return float(cells[2])
            except ValueError:
                return None
    return None


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Threads the oracle's BLAS uses (its only multi-threaded part)."""
    try:
        from threadpoolctl import threadpool_info
        return max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_sample(x, wl, seconds: float, with_bwd: bool):
    """The fp64 oracle, as it stands, on a bounded sample of one workload: heads in
    order, each head's pooled predictor, then its query tiles in a fixed shuffled
    order (score row, top-k selection, forward and, for training workloads,
    backward of the tile) until the time budget is spent (whole tiles only).  Wall
    time per phase, and each phase extrapolated to the whole workload (pooling by
    heads, score rows and selection by tiles, forward and backward by attended
    pairs)."""
    import oracle
    f = lambda t: t.detach().cpu().double().numpy()
    geom = oracle.Geometry(*wl.latent, *wl.tile)
    mem = geom.members()
    scale = 1.0 / math.sqrt(wl.d)
    T = geom.T
    order = np.random.default_rng(0).permutation(geom.NB)
    ph = {"predict": 0.0, "select": 0.0, "fwd": 0.0, "bwd": 0.0}
    pool_s, tiles, heads, pairs = 0.0, 0, 0, 0
    names = ("Q", "K", "V", "dO") if with_bwd else ("Q", "K", "V")
    ks = [int(v) for v in x["k"].tolist()]
    for bh in range(wl.B * wl.H):
        b, h = divmod(bh, wl.H)
        arr = {n: f(x[n][b, h]) for n in names}                 # staging, not timed
        Wq, Wk = f(x["Wq"][h]), f(x["Wk"][h])
        k = ks[bh]
        c0 = time.perf_counter()
        Qb = oracle.pooled_features(arr["Q"], Wq, mem)
        Kb = oracle.pooled_features(arr["K"], Wk, mem)
        dt = time.perf_counter() - c0
        ph["predict"] += dt
        pool_s += dt
        heads += 1
        for tau in order:
            t0 = time.perf_counter()
            srow = oracle.block_scores(Qb[tau:tau + 1], Kb)[0]
            t1 = time.perf_counter()
            blocks = list(oracle.select_row(srow, int(tau), k))
            t2 = time.perf_counter()
            oracle.attn_tile(arr["Q"], arr["K"], arr["V"], mem, int(tau), blocks, scale)
            t3 = time.perf_counter()
            if with_bwd:
                oracle.attn_bwd_tile(arr["Q"], arr["K"], arr["V"], arr["dO"], mem, int(tau), blocks, scale)
            t4 = time.perf_counter()
            ph["predict"] += t1 - t0
            ph["select"] += t2 - t1
            ph["fwd"] += t3 - t2
            ph["bwd"] += t4 - t3
            tiles += 1
            pairs += k * T * T
            if sum(ph.values()) >= seconds:
                break
        if sum(ph.values()) >= seconds:
            break
    total_tiles = wl.B * wl.H * geom.NB
    total_pairs = sum(geom.NB * kk * T * T for kk in ks)
    full = {"predict": pool_s * (wl.B * wl.H) / heads + (ph["predict"] - pool_s) * total_tiles / tiles,
            "select": ph["select"] * total_tiles / tiles,
            "fwd": ph["fwd"] * total_pairs / pairs,
            "bwd": ph["bwd"] * total_pairs / pairs if with_bwd else 0.0}
    fl_per_pair = (14.0 if with_bwd else 4.0) * wl.d
    busy = sum(ph.values())
    return {"value": fl_per_pair * pairs / busy / 1e12, "unit": "TFLOP/s",
            "phases_s": {p: round(v, 4) for p, v in ph.items() if with_bwd or p != "bwd"},
            "extrapolated_full_s": {p: round(v, 2) for p, v in full.items() if with_bwd or p != "bwd"},
            "sample": f"{wl.name}: {tiles} of {total_tiles} query tiles over {heads} head(s) of {wl.B * wl.H}: "
                      f"per head the pooled predictor, per tile its score row, top-k selection and fp64 forward"
                      f"{' + backward' if with_bwd else ''}; {busy:.1f} s of oracle time; value = counted "
                      f"attended FLOP ({int(fl_per_pair / wl.d)}*d per pair) of the sample / that time; the "
                      f"full-workload times are extrapolated from the sample"}


def cpu_baseline(x, wl, seconds: float, others, per_config: float, dev):
    """cpu_sample on this workload (x) and on each configuration in `others`
    (inputs generated on the device like the bench's, then staged to the host)."""
    from dsa_inputs import WORKLOADS, generate
    out = cpu_sample(x, wl, seconds, with_bwd=wl.backward)
    out.update({"cores": oracle_threads(), "cpu_model": cpu_model(), "kind": "oracle"})
    cfgs = {}
    for name in others:
        if name == wl.name or name not in WORKLOADS:
            continue
        w2 = WORKLOADS[name]
        x2 = generate(w2, device=dev, with_grad=w2.backward)
        cfgs[name] = cpu_sample(x2, w2, per_config, with_bwd=w2.backward)
        del x2
    out["configs"] = cfgs
    return out


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    lib_path = os.path.join(ROOT, "dynamic_sparse_attention_lowrank_amd", "libdsa.so")
    if not os.path.exists(lib_path):
        from dynamic_sparse_attention_lowrank_amd import build as b
        b.build()
    import dynamic_sparse_attention_lowrank_amd as dsa
    from dsa_inputs import WORKLOADS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = generate(wl, device=dev, with_grad=wl.backward)
    lay = dsa.Layout(tuple(wl.latent), tuple(wl.tile))
    B, H, N, d, NB, T = wl.B, wl.H, wl.N, wl.d, wl.NB, wl.T
    kdev = x["k"].to(dev)
    ks = x["k"].tolist()
    kmax = int(max(ks))
    r = wl.r
    f32 = torch.float32
    Qbar = torch.empty(B, H, NB, r, device=dev, dtype=f32)
    Kbar = torch.empty_like(Qbar)
    S = torch.empty(B, H, NB, NB, device=dev, dtype=f32) if args.score_matrix else None
    idx = torch.empty(B, H, NB, kmax, device=dev, dtype=torch.int32)
    O = torch.empty(B, H, N, d, device=dev, dtype=f32)
    LSE = torch.empty(B, H, N, device=dev, dtype=f32)
    dQ = torch.empty(B, H, N, d, device=dev, dtype=torch.bfloat16)
    dK = torch.empty_like(dQ)
    dV = torch.empty_like(dQ)
    ws = (torch.empty(dsa.bwd_workspace_bytes(x["Q"], lay, kmax), device=dev, dtype=torch.uint8)
          if wl.backward else None)
    fws = torch.empty(dsa.fwd_workspace_bytes(x["Q"], lay), device=dev, dtype=torch.uint8)
    Q, K, V, Wq, Wk = (x[n] for n in ("Q", "K", "V", "Wq", "Wk"))
    dO = x.get("dO")

    train = wl.backward                       # forward-only workloads skip the backward phases
    phases = ["predict", "select", "fwd", "bwd_prepare", "bwd_dkdv", "bwd_dq"]
    if not args.score_matrix:
        phases[0:2] = ["predict_select", "-"]
    if not train:
        phases = phases[:3]

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        if args.score_matrix:
            dsa.predict(Q, K, Wq, Wk, lay, out=(Qbar, Kbar, S))
            rec(1)
            dsa.select(S, kdev, kmax, lay, d=d, out=idx)
        else:
            # pooled predictor, then per-row scores + top-k without the score matrix
            dsa.predict_select(Q, K, Wq, Wk, kdev, kmax, lay, out=(Qbar, Kbar, idx))
            rec(1)
        rec(2)
        dsa.attn_fwd(Q, K, V, idx, kdev, lay, out=(O, LSE), workspace=fws)
        rec(3)
        if not train:
            return
        dsa.attn_bwd_prepare(O, dO, idx, kdev, lay, ws)
        rec(4)
        dsa.attn_bwd_dkdv(Q, K, V, dO, LSE, kmax, lay, ws, dK, dV)
        rec(5)
        dsa.attn_bwd_dq(Q, K, V, dO, LSE, idx, kdev, lay, ws, dQ)
        rec(6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides; HIP events on the
    # launch stream (torch's current stream) bracket every phase of every step
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    clocks_start = read_clocks()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per_step = {p: [ev[j].elapsed_time(ev[j + 1]) for ev in events] for j, p in enumerate(phases)}
    phase_ms = {p: sum(v) / args.steps for p, v in per_step.items()}
    span_ms = events[0][0].elapsed_time(events[-1][-1]) / args.steps

    # stage-one predictor training signal on the same inputs, timed on its own (not
    # part of the step above): loss and dWq/dWk, HBM-bound on reading Q and K once
    pws = torch.empty(dsa.predictor_grad_workspace_bytes(Q, lay), device=dev, dtype=torch.uint8)
    pout = (torch.empty(B, H, device=dev, dtype=f32), torch.empty(Wq.shape, device=dev, dtype=f32),
            torch.empty(Wk.shape, device=dev, dtype=f32))
    for _ in range(2):
        dsa.predictor_grad(Q, K, Wq, Wk, lay, out=pout, workspace=pws)
    torch.cuda.synchronize()
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    pe[0].record()
    for _ in range(10):
        dsa.predictor_grad(Q, K, Wq, Wk, lay, out=pout, workspace=pws)
    pe[1].record()
    torch.cuda.synchronize()
    pg_ms = pe[0].elapsed_time(pe[1]) / 10
    pg_bytes = 2.0 * Q.numel() * Q.element_size()

    # 3-D rotary positions of Q and K (forward) and of dQ and dK (inverse), timed on
    # their own: four HBM passes of read + write
    rq, rk = torch.empty_like(Q), torch.empty_like(K)
    for _ in range(2):
        dsa.rope3d(Q, lay, out=rq)
    torch.cuda.synchronize()
    re_ = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    re_[0].record()
    for _ in range(10):
        dsa.rope3d(Q, lay, out=rq)
        dsa.rope3d(K, lay, out=rk)
        dsa.rope3d(dQ, lay, inverse=True, out=dQ)
        dsa.rope3d(dK, lay, inverse=True, out=dK)
    re_[1].record()
    torch.cuda.synchronize()
    rope_ms = re_[0].elapsed_time(re_[1]) / 10
    rope_bytes = 2.0 * (Q.numel() * Q.element_size() + K.numel() * K.element_size() +
                        dQ.numel() * dQ.element_size() + dK.numel() * dK.element_size())
    del rq, rk

    # the forward alone with cold caches: before each repetition a 512 MiB write
    # (twice the 256 MB memory-attached cache, and far above the L2s) evicts what
    # the previous repetition left; the in-step phase times above are the warm ones
    flush = torch.empty(512 << 20, device=dev, dtype=torch.uint8)
    cold = []
    for i in range(args.cold_reps + 1 if args.cold_reps > 0 else 0):
        flush.fill_(i & 0xFF)
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ce[0].record()
        dsa.attn_fwd(Q, K, V, idx, kdev, lay, out=(O, LSE), workspace=fws)
        ce[1].record()
        torch.cuda.synchronize()
        if i:                                           # the first one only sets the pattern up
            cold.append(ce[0].elapsed_time(ce[1]))
    del flush
    clocks_end = read_clocks()

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        a_ = torch.zeros(n, device=dev, dtype=torch.int32)
        b_ = torch.empty_like(a_)
        torch.bitwise_not(a_, out=b_)                   # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()

    pairs = sum(NB * kk * T * T for kk in ks)          # attended (query, key) pairs
    flop_fwd = 4.0 * d * pairs
    flop_bwd = 10.0 * d * pairs if train else 0.0
    flop_step = flop_fwd + flop_bwd
    value = flop_step / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = flop_fwd / (phase_ms["fwd"] * 1e-3) / 1e12

    # dominant single-kernel phase and its algorithmic work per launch: forward 4*d
    # per pair; dK/dV 8*d (S, dP, dV, dK); dQ 2*d (dQ only: its recomputation of S
    # and dP is extra work, not algorithmic)
    fwd_kernel = "attn_fwd_pair_kernel" if dsa.fwd_kernel_for(Q, lay) == dsa.FWD_TILE_PAIR else "attn_fwd_kernel"
    algo = {"fwd": (4.0 * d * pairs, fwd_kernel)}
    if train:
        algo.update({"bwd_dkdv": (8.0 * d * pairs, "bwd_dkdv_kernel"), "bwd_dq": (2.0 * d * pairs, "bwd_dq_kernel")})
    dom = max(algo, key=lambda p: phase_ms[p])
    achieved = algo[dom][0] / (phase_ms[dom] * 1e-3) / 1e12
    traffic = load_traffic(algo[dom][1], wl.name)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": algo[dom][1], "ms": round(phase_ms[dom], 4),
                "algorithmic_flop_per_launch": algo[dom][0]}
    # the same kernel's average duration in the committed rocprofv3 trace (when it
    # was taken on the current sources) and the fraction it gives
    tr = load_trace_avg_us(algo[dom][1], wl.name)
    if tr is not None:
        roofline["rocprof_avg_ms"] = round(tr / 1e3, 4)
        roofline["frac_at_rocprof_avg"] = round(algo[dom][0] / (tr * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
    bwd_roofline = None
    if train:
        bwd_ms = phase_ms["bwd_prepare"] + phase_ms["bwd_dkdv"] + phase_ms["bwd_dq"]
        bwd_tf = flop_bwd / (bwd_ms * 1e-3) / 1e12
        bwd_roofline = {"bound": "mfma", "what": "prepare + dK/dV + dQ, 10*d FLOP per pair", "ms": round(bwd_ms, 4),
                        "achieved": round(bwd_tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(bwd_tf / BF16_PEAK_TFLOPS, 4)}
    cold_med = float(np.median(cold)) if cold else None
    cold_tf = flop_fwd / (cold_med * 1e-3) / 1e12 if cold else None

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: one attention layer, " + ("training step (predict+select+fwd+bwd)"
                                                                       if train else "forward (predict+select+fwd)"),
                   "predictor": "two-step (score matrix)" if args.score_matrix else "fused predict+select",
                   "B": B, "H": H, "d": d, "latent": list(wl.latent), "tokens": N, "tile": list(wl.tile),
                   "blocks": NB, "rank": r, "k": kmax, "keep_percent": list(wl.keep_percent)},
        "pct_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "headline": {"what": f"dsa_attn_fwd alone, median of {len(cold)} repetitions each after a 512 MiB "
                             "cache-evicting write (L2 and memory-attached cache cold)",
                     "ms_per_layer": round(cold_med, 4), "tflops": round(cold_tf, 2),
                     "pct_bf16_peak": round(100 * cold_tf / BF16_PEAK_TFLOPS, 2),
                     "pct_bf16_peak_at_measured_sclk": pct_at_clock(cold_tf, clocks_start, clocks_end)}
                    if cold else None,
        "fwd": {"what": "warm, inside the timed steps", "ms": round(phase_ms["fwd"], 4), "tflops": round(fwd_tflops, 2),
                "pct_bf16_peak": round(100 * fwd_tflops / BF16_PEAK_TFLOPS, 2),
                "pct_bf16_peak_at_measured_sclk": pct_at_clock(fwd_tflops, clocks_start, clocks_end)},
        "phase_ms": {p: round(v, 4) for p, v in phase_ms.items() if p != "-"},
        "phase_stats_ms": {p: stats(v) for p, v in per_step.items() if p != "-"},
        "fwd_cold": dict(stats(cold), reps=len(cold), flush_mib=512,
                         tflops_at_median=round(flop_fwd / (float(np.median(cold)) * 1e-3) / 1e12, 2))
                    if cold else None,
        "clocks": {"start": clocks_start, "end": clocks_end},
        "event_ms_per_step": round(span_ms, 4),
        "counted_flop": {"fwd": flop_fwd, "bwd": flop_bwd, "pairs": pairs},
        "roofline": roofline,
        "bwd_roofline": bwd_roofline,
        "rope3d": {"ms": round(rope_ms, 4), "what": "Q, K rotated + dQ, dK rotated back", "bound": "hbm",
                   "algorithmic_bytes": rope_bytes, "GBps": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
                   "peak_GBps": 8000.0},
        "predictor_grad": {"ms": round(pg_ms, 4), "bound": "hbm", "algorithmic_bytes": pg_bytes,
                           "GBps": round(pg_bytes / (pg_ms * 1e-3) / 1e9, 1), "peak_GBps": 8000.0},
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        others = [c for c in args.cpu_configs.split(",") if c]
        out["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_seconds, others, args.cpu_config_seconds, dev)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# rocprofv3 output -> profiles/ summaries

def _kernel_label(raw: str) -> str:
    """Short name of a library kernel from its (mangled or demangled) symbol."""
    import re
    m = re.search(r"([a-z][a-z0-9_]*_kernel)", raw)
    if not m:
        return raw[:60]
    name = m.group(1)
    tail = raw[m.end():]
    args = []
    if name in ("fused_select_kernel", "select_kernel"):     # <slots per lane[, rank, exact rank]>
        ints = re.findall(r"Li(\d+)E", tail[:40]) or re.findall(r"(\d+)", tail[:tail.find(">") + 1])
        exact = "Lb1E" in tail[:40] or "true>" in tail[:40]
        return f"{name}<{','.join(ints + (['exact'] if exact else []))}>"
    if tail.startswith("I") or tail.startswith("<"):
        if "DF16b" in tail[:8] or "__bf16" in tail[:12]:
            args.append("bf16")
        elif tail.startswith("If") or tail.startswith("<float"):
            args.append("fp32")
        d = re.match(r"I(?:DF16b|f)?(?:Li(\d+)E)+", tail) or re.match(r"<[^,>]*, (\d+)", tail)
        if d:
            args.append(d.group(1))
        s = re.match(r"ILi(\d+)EE", tail) or re.match(r"<(\d+)>", tail)
        if s and not args:
            args.append(s.group(1))
        if name == "attn_fwd_pair_kernel":           # bf16 only, template <d, full>
            dd = re.match(r"ILi(\d+)E", tail) or re.match(r"<(\d+),", tail)
            args = ["bf16"] + ([dd.group(1)] if dd else [])
        if "Lb1E" in tail[:30] or "true>" in tail[:30]:
            args.append("full")
    return f"{name}<{','.join(args)}>" if args else name


def _is_library_kernel(raw: str) -> bool:
    return "dsa" in raw and "_kernel" in raw


def _read_run(sub: str):
    cmd = open(os.path.join(sub, "cmd.txt")).read().strip()
    out = None
    for line in open(os.path.join(sub, "out.json")):
        line = line.strip()
        if line.startswith("{"):
            out = json.loads(line)
    return cmd, out


def _counter_rows(sub: str, counter: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(sub, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize(root: str, prof_dir: Optional[str] = None):
    """Write profiles/<workload>_kernel_trace.md from a `--kernel-trace --stats` run
    and profiles/traffic_<kernel>_<workload>.txt from one FETCH_SIZE and one
    WRITE_SIZE `--pmc` run, each counter scaled by what it reads for the
    calibration kernel (an int32 bitwise-not over --copy-probe-mib MiB: exactly
    that many bytes read and written)."""
    import csv
    import glob
    prof = prof_dir or os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)

    cmd, out = _read_run(os.path.join(root, "trace"))
    wl_name = out["config"]["workload"].split(":")[0]
    stats = glob.glob(os.path.join(root, "trace", "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = [r for r in csv.DictReader(open(stats)) if _is_library_kernel(r["Name"])]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    # launch resources as the profiler reports them (first dispatch of each kernel)
    res = {}
    for f in glob.glob(os.path.join(root, "trace", "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if _is_library_kernel(r["Kernel_Name"]):
                res.setdefault(_kernel_label(r["Kernel_Name"]), r)
    c = out["config"]
    lines = [f"# Kernel trace: {wl_name} training step (B={c['B']} H={c['H']} d={c['d']}, {c['tokens']:,} tokens, "
             f"tile {'x'.join(map(str, c['tile']))}, k={c['k']}, bf16)", "",
             "Command (from the repository root, on one MI355X):", "", "    " + cmd, "",
             f"Library sources: source_hash {out['source_hash']} (bench.py prints the same hash).", "",
             f"Library kernels only ({out['warmup']} warm-up + {out['steps']} timed steps per kernel); "
             "the other rows of the raw summary are torch's input generator.", "",
             "Launch resources as the kernel trace reports them: VGPR / AGPR (VGPR_Count, "
             "Accum_VGPR_Count), LDS bytes per work-group (LDS_Block_Size), scratch bytes per lane "
             "(Scratch_Size), work-group size.", "",
             "| kernel | calls | avg us | min us | max us | VGPR | AGPR | LDS B | scratch B | WG |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lab = _kernel_label(r["Name"])
        rr = res.get(lab, {})
        g = lambda k: rr.get(k, "-")
        lines.append(f"| {lab} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {g('VGPR_Count')} | "
                     f"{g('Accum_VGPR_Count')} | {g('LDS_Block_Size')} | {g('Scratch_Size')} | "
                     f"{g('Workgroup_Size_X')} |")
    lines += ["", "In-bench HIP-event phase times of the same run, ms:", "",
              "    " + json.dumps(out["phase_ms"]), "",
              f"Step {out['ms_per_step']} ms, {out['value']} attended TFLOP/s; forward {out['fwd']['ms']} ms = "
              f"{out['fwd']['tflops']} TFLOP/s warm (the profiler's serialisation inflates the step slightly)."]
    with open(os.path.join(prof, f"{wl_name}_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    per = {}
    cmds = {}
    probe = {}
    hashes = set()
    for counter, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        cmds[counter], o = _read_run(os.path.join(root, sub))
        hashes.add(o["source_hash"])
        mib = None
        import re
        m = re.search(r"--copy-probe-mib (\d+)", cmds[counter])
        if m:
            mib = int(m.group(1))
        rows = _counter_rows(os.path.join(root, sub), counter)
        cal = [v for n, v in rows if "bitwise_not" in n]
        probe[counter] = (mib, max(cal) if cal else None)
        for n, v in rows:
            if _is_library_kernel(n):
                per.setdefault(_kernel_label(n), {}).setdefault(counter, []).append(v)
    if len(hashes) != 1:
        raise SystemExit(f"counter runs come from different sources: {hashes}")
    src_hash = hashes.pop()
    for label, cs in per.items():
        if "FETCH_SIZE" not in cs or "WRITE_SIZE" not in cs:
            continue
        kname = label.split("<")[0]
        body = [f"# HBM traffic per launch of {label} on {wl_name}, from rocprofv3 counters", "#",
                f"# fetch command: {cmds['FETCH_SIZE']}", f"# write command: {cmds['WRITE_SIZE']}", "#",
                "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by bytes / counter reading of the",
                "# calibration kernel (int32 bitwise-not over the probe size: reads and writes exactly that many bytes).",
                f"kernel: {label}", f"workload: {wl_name}"]
        tot = 0.0
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            v = cs[counter]
            avg = sum(v) / len(v)
            mib, cal = probe[counter]
            scale = (mib * (1 << 20)) / (cal * 1024.0) if (mib and cal) else 1.0
            key = counter.split("_")[0].lower()
            body += [f"{key}_dispatches: {len(v)}", f"{key}_kib_per_dispatch: {avg:.1f}",
                     f"{key}_probe_kib: {cal if cal is not None else 'none'}", f"{key}_scale: {scale:.4f}",
                     f"{key}_bytes_per_launch: {avg * 1024.0 * scale:.0f}"]
            tot += avg * 1024.0 * scale
        body += [f"hbm_bytes_per_launch: {tot:.0f}", f"source_hash: {src_hash}"]
        with open(os.path.join(prof, f"traffic_{kname}_{wl_name}.txt"), "w") as fh:
            fh.write("\n".join(body) + "\n")
    print(f"wrote profiles for {wl_name} (source_hash {src_hash}); current sources {source_hash()}")
    summarize_counters(root, wl_name, src_hash, prof)


# per attention kernel: counts of SQ / TA / TCP events per dispatch, and the same
# per (wave, block) unit -- one wave's 32 queries x 32 keys of one kept block
# (forward), one wave's 16 keys against one query tile (dK/dV) or its 16 queries
# against one kept block (dQ): four waves share each (query tile, kept block) pair
# in every kernel -- so that instruction mixes and unit busy times compare
_UNITS = {"attn_fwd_kernel": 4, "attn_fwd_pair_kernel": 4, "bwd_dkdv_kernel": 4, "bwd_dq_kernel": 4}


def summarize_counters(root: str, wl_name: str, src_hash: str, prof: str):
    """profiles/counters_<workload>.md from the --pmc runs under DIR/counters_* (each
    with cmd.txt and out.json like the traffic runs), for the attention kernels."""
    import glob
    subs = sorted(glob.glob(os.path.join(root, "counters_*")))
    if not subs:
        return
    vals, cmds, pairs = {}, [], None
    for sub in subs:
        cmd, o = _read_run(sub)
        if o["source_hash"] != src_hash:
            raise SystemExit(f"{sub} comes from sources {o['source_hash']}, the other runs from {src_hash}")
        cmds.append(cmd)
        pairs = o["counted_flop"]["pairs"]
        import csv
        for f in sorted(glob.glob(os.path.join(sub, "**", "*counter_collection.csv"), recursive=True)):
            for r in csv.DictReader(open(f)):
                label = _kernel_label(r["Kernel_Name"])
                kname = label.split("<")[0]
                if kname not in _UNITS:
                    continue
                d = vals.setdefault(label, {}).setdefault(r["Counter_Name"], {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    blocks = pairs / (64 * 64)            # (query tile, kept block) pairs of the workload
    lines = [f"# Hardware counters of the attention kernels on {wl_name}", "",
             "Commands (from the repository root, on one MI355X; one rocprofv3 pass each):", ""]
    lines += ["    " + c for c in cmds]
    lines += ["", f"Library sources: source_hash {src_hash}.", "",
              "Per dispatch: the counter summed over all its instances, averaged over the dispatches of "
              "the run. Per unit: divided by the number of (wave, block) units of one launch -- "
              f"{blocks:.0f} (query tile, kept block) pairs times the waves that share one pair "
              "(4 in each kernel).", ""]
    names = sorted({c for k in vals.values() for c in k})
    raw = ("SQ_", "TA_", "TD_", "TCC_", "TCP_", "GRBM_")
    for label in sorted(vals):
        units = blocks * _UNITS[label.split("<")[0]]
        lines += [f"## {label}", "", "| counter | per dispatch | per unit |", "|---|---|---|"]
        avg = {}
        for c in names:
            if c not in vals[label]:
                continue
            v = list(vals[label][c].values())
            avg[c] = sum(v) / len(v)
            # derived metrics (percentages, mean occupancy) are per dispatch only
            per_unit = f"{avg[c] / units:.1f}" if c.startswith(raw) else "-"
            lines.append(f"| {c} | {avg[c]:.4g} | {per_unit} |")
        extra = []
        if avg.get("TCC_HIT_sum") is not None and avg.get("TCC_MISS_sum") is not None:
            tot = avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"]
            if tot > 0:
                extra.append(f"L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS): {100 * avg['TCC_HIT_sum'] / tot:.1f} %")
        if avg.get("SQ_LDS_BANK_CONFLICT") is not None and avg.get("SQ_LDS_IDX_ACTIVE"):
            extra.append("LDS bank-conflict cycles per LDS-active cycle, SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE: "
                         f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.3f}")
        if extra:
            lines += [""] + ["- " + e for e in extra]
        lines.append("")
    with open(os.path.join(prof, f"counters_{wl_name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote profiles/counters_{wl_name}.md")


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the DeMo / FlexDeMo optimizer step on one GPU's shard.

A step is one pass of the whole path over the shard: demo_encode (momentum,
32-element chunks, DCT-II, top-k, ternary sign packing, inverse transform,
error feedback) followed by demo_decode_apply over R replica payloads
(aggregate, inverse transform, parameter update).  Inputs are synthetic and
resident in HBM before the timed region: the OLMo2-1B-shaped half shard
(639,697,920 fp32 parameters), gradients s_layer * N(0, 1e-3) with per-layer
scales U(0.5, 2), theta ~ N(0, 0.02), momentum from 0; the second replica's
payload is the encode of a state drawn from seed 1.

Prints one JSON line.  Timing: W untimed warm-up steps, then K steps between
two device synchronisations; per-kernel durations come from HIP events
recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
METRIC = "params/s and HBM GB/s (% of peak) of DeMo encode+decode, OLMo2-1B half shard"

WORKLOADS = {
    # name: (scheme, k, value_fmt, R)
    "olmo2-1b-half-shard-demo-k1": ("dct", 1, "ternary", 2),
    "olmo2-1b-half-shard-demo-k2": ("dct", 2, "ternary", 2),
    "olmo2-1b-half-shard-random-n8": ("random", 8, "ternary", 2),
    "olmo2-1b-half-shard-random-n16": ("random", 16, "ternary", 2),
    "olmo2-1b-half-shard-random-n8-f16": ("random", 8, "f16", 2),
    "olmo2-1b-half-shard-random-n8-f32": ("random", 8, "f32", 2),
    "olmo2-1b-half-shard-stride-n8": ("stride", 8, "ternary", 2),
    "vit-b-set-demo-k1": ("dct", 1, "ternary", 2),
}


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "communication_compressed_optimizer_elt_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".inc")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="olmo2-1b-half-shard-demo-k1", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU work budget of the oracle baseline")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU's shard only; run it with --gpus 1 "
              "(the step has no cross-GPU part in this build)", file=sys.stderr)
        return 2

    import torch

    from communication_compressed_optimizer_elt_amd import binding as L
    from communication_compressed_optimizer_elt_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    L.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    scheme_name, k, fmt_name, R = WORKLOADS[args.workload]
    scheme = {"dct": L.SCHEME_DCT, "random": L.SCHEME_RANDOM, "stride": L.SCHEME_STRIDE}[scheme_name]
    fmt = {"ternary": L.VAL_TERNARY, "f16": L.VAL_F16, "f32": L.VAL_F32}[fmt_name]
    segs = synth.vit_b_set() if args.workload.startswith("vit") else synth.olmo2_half_shard()
    n = synth.shard_numel(segs)
    scales = synth.layer_scales(0, max(s.group for s in segs) + 1)
    g_std = 1e-2 if args.workload.startswith("vit") else 1e-3

    cfg = L.Config(scheme=scheme, k=k, value_fmt=fmt, beta=0.9, lr=1e-3, seed=0, step=0)
    lay = L.demo_payload_layout(cfg, n)
    stride = lay["total_bytes"]
    payload_bytes = lay["idx_bytes"] + 2 * lay["plane_bytes"] + lay["val_bytes"]

    # ---- inputs, resident in HBM -------------------------------------------
    g = synth.scaled_grad_torch(segs, scales, g_std, 0, 0)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    theta = synth.normal_torch(n, 0.02, 0, synth.TAG_THETA)
    pay = torch.zeros(R * stride, dtype=torch.uint8, device=dev)
    # replicas 1..R-1: payloads encoded from states drawn from seeds 1..R-1
    pg = torch.empty_like(g)
    pm = torch.empty_like(m)
    for r in range(1, R):
        synth.scaled_grad_torch(segs, scales, g_std, r, 0, out=pg)
        pm.zero_()
        L.demo_encode(cfg, n, pg, pm, pay[r * stride:])
    torch.cuda.synchronize()
    del pg, pm
    torch.cuda.empty_cache()

    # ---- achievable copy bandwidth on this device (context) -----------------
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * n * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    stream = torch.cuda.current_stream()

    def step(t, ev=None):
        cfg.step = t
        if ev is not None:
            ev[0].record(stream)
        L.demo_encode(cfg, n, g, m, pay, None, stream)
        if ev is not None:
            ev[1].record(stream)
        L.demo_decode_apply(cfg, n, theta, pay, stride, R, stream)
        if ev is not None:
            ev[2].record(stream)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    step_ms = wall * 1e3 / args.steps
    enc_bytes = 12 * n + payload_bytes
    dec_bytes = 8 * n + R * payload_bytes
    enc_gbps = enc_bytes / (enc_ms.mean() / 1e3) / 1e9
    dec_gbps = dec_bytes / (dec_ms.mean() / 1e3) / 1e9
    step_gbps = (enc_bytes + dec_bytes) / (step_ms / 1e3) / 1e9

    kern = {
        "encode": {"avg_ms": float(enc_ms.mean()), "min_ms": float(enc_ms.min()), "bytes": enc_bytes,
                   "gbps": enc_gbps},
        "decode": {"avg_ms": float(dec_ms.mean()), "min_ms": float(dec_ms.min()), "bytes": dec_bytes,
                   "gbps": dec_gbps},
    }
    dom = "encode" if enc_ms.mean() >= dec_ms.mean() else "decode"
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{dom}_{args.workload}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            rec = json.load(f)
        if rec.get("source_hash") == source_hash():
            traffic = rec.get("hbm_bytes_per_launch")

    out = {
        "metric": METRIC,
        "value": n / (step_ms / 1e3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n_elems": n, "scheme": scheme_name, "k": k,
                   "value_fmt": fmt_name, "replicas": R, "chunk": 32},
        "hbm_gbps": step_gbps,
        "pct_hbm_peak": 100.0 * step_gbps / HBM_PEAK_GBPS,
        "copy_gbps": copy_gbps,
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["gbps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": kern[dom]["gbps"] / HBM_PEAK_GBPS, "traffic": traffic},
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        def peer_grad(r):
            return synth.scaled_grad_torch(segs, scales, g_std, r, 0)

        out["cpu_baseline"] = cpu_baseline(cfg, n, g, m, theta, peer_grad, R, args.cpu_seconds)

    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(cfg, n, g, m, theta, peer_grad, R, budget_s):
    """The fp64 oracle, timed on this host's cores, on a bounded sample of the
    same shard: the first S chunks (the same input bytes as the GPU state; the
    other replicas' slots come from the oracle's own encode of their seeded
    states), stepped until the CPU budget is used."""
    import oracle

    C = n // 32
    S = min(C, 1 << 21)
    ids = np.arange(S, dtype=np.uint64)
    nv = np.full(S, 32, np.int32)
    zeros = np.zeros((S, 32), np.float32)
    g_rows = g[: S * 32].view(S, 32).cpu().numpy()
    own = oracle.Shard(ids, nv, m[: S * 32].view(S, 32).cpu().numpy(), theta[: S * 32].view(S, 32).cpu().numpy())
    p = oracle.Params(scheme=cfg.scheme, k=cfg.k, value_fmt=cfg.value_fmt, beta=cfg.beta, lr=cfg.lr, seed=cfg.seed)
    peers_idx, peers_val = [], []
    for r in range(1, R):
        peer = oracle.Shard(ids, nv, zeros, zeros)
        gi, gv, _, _ = peer.encode(p, peer_grad(r)[: S * 32].view(S, 32).cpu().numpy())
        peers_idx.append(gi)
        peers_val.append(gv)
    steps = 0
    t0 = time.perf_counter()
    while True:
        idx, val, _, _ = own.encode(p, g_rows)
        own.decode(p, [idx] + peers_idx, [val] + peers_val)
        steps += 1
        if time.perf_counter() - t0 >= budget_s or steps >= 50:
            break
    dt = time.perf_counter() - t0
    return {"value": S * 32 * steps / dt, "unit": "params/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {S} chunks ({S * 32} params) of the shard, {steps} encode+decode steps "
                      f"in {dt:.1f} s, fp64 state"}


if __name__ == "__main__":
    sys.exit(main())

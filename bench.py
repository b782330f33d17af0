#!/usr/bin/env python3
"""Benchmark of the DeMo / FlexDeMo optimizer step on one GPU's shard.

A step is one pass of the whole path over the shard: demo_encode (momentum,
32-element chunks, DCT-II, top-k, ternary sign packing, inverse transform,
error feedback) followed by demo_decode_apply over R replica payloads
(aggregate, inverse transform, parameter update).  Inputs are synthetic and
resident in HBM before the timed region: the default workload is the
OLMo2-1B-shaped half shard (639,697,920 fp32 parameters), gradients
s_layer * N(0, 1e-3) with per-layer scales U(0.5, 2), theta ~ N(0, 0.02),
momentum from 0; the second replica's payload is the encode of a state drawn
from seed 1.

Prints one JSON line.  Timing: W untimed warm-up steps, then K steps between
two device synchronisations; per-kernel durations come from HIP events
recorded between the launches on the stream the kernels run on.  The fp64 CPU oracle is timed
afterwards on the same input bytes (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from dataclasses import dataclass

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
METRIC = "params/s and HBM GB/s (% of peak) of DeMo encode+decode, OLMo2-1B half shard"
DILOCO_PERIOD = 16


@dataclass(frozen=True)
class Workload:
    shard: str           # "olmo2" (half shard), "olmo2-full", "vit", "tensor4096"
    scheme: str          # "dct", "random", "stride", "diloco"
    k: int
    fmt: str             # "ternary", "f16", "f32"
    R: int
    mode: str = "step"   # "step": encode + decode per step; "decode": decode only
    sign: int = 1        # 0: the slots carry the selected values themselves
    adamw: bool = False  # Decoupled AdamW (second moment read and written by the encode)


WORKLOADS = {
    "olmo2-1b-half-shard-demo-k1": Workload("olmo2", "dct", 1, "ternary", 2),
    "olmo2-1b-half-shard-demo-k2": Workload("olmo2", "dct", 2, "ternary", 2),
    "olmo2-1b-half-shard-random-n8": Workload("olmo2", "random", 8, "ternary", 2),
    "olmo2-1b-half-shard-random-n16": Workload("olmo2", "random", 16, "ternary", 2),
    "olmo2-1b-half-shard-random-n8-f16": Workload("olmo2", "random", 8, "f16", 2),
    "olmo2-1b-half-shard-random-n8-f32": Workload("olmo2", "random", 8, "f32", 2),
    "olmo2-1b-half-shard-random-n16-f16": Workload("olmo2", "random", 16, "f16", 2),
    "olmo2-1b-half-shard-random-n16-f32": Workload("olmo2", "random", 16, "f32", 2),
    "olmo2-1b-half-shard-stride-n8": Workload("olmo2", "stride", 8, "ternary", 2),
    "olmo2-1b-half-shard-stride-n16": Workload("olmo2", "stride", 16, "ternary", 2),
    "olmo2-1b-half-shard-diloco-p16": Workload("olmo2", "diloco", 32, "ternary", 2),
    "olmo2-1b-half-shard-decode-r64-demo-k1": Workload("olmo2", "dct", 1, "ternary", 64, "decode"),
    "olmo2-1b-half-shard-decode-r64-random-n8": Workload("olmo2", "random", 8, "ternary", 64, "decode"),
    "vit-b-set-demo-k1": Workload("vit", "dct", 1, "ternary", 2),
    "tensor-4096-demo-k4": Workload("tensor4096", "dct", 4, "ternary", 2),
    "olmo2-1b-full-demo-k1": Workload("olmo2-full", "dct", 1, "ternary", 2),
    "olmo2-1b-half-shard-adamw-demo-k1-f32": Workload("olmo2", "dct", 1, "f32", 2, sign=0, adamw=True),
    "olmo2-1b-half-shard-adamw-random-n8-f32": Workload("olmo2", "random", 8, "f32", 2, sign=0, adamw=True),
    "olmo2-1b-half-shard-demo-k1-f32-sign-off": Workload("olmo2", "dct", 1, "f32", 2, sign=0),
    "olmo2-1b-half-shard-demo-k1-f16-sign-off": Workload("olmo2", "dct", 1, "f16", 2, sign=0),
    "olmo2-1b-half-shard-random-n8-f16-sign-off": Workload("olmo2", "random", 8, "f16", 2, sign=0),
    "olmo2-1b-half-shard-random-n8-f32-sign-off": Workload("olmo2", "random", 8, "f32", 2, sign=0),
}
# the 4096-element tensor is L2-resident and launch-bound: no roofline point
LAUNCH_BOUND = {"tensor-4096-demo-k4"}


def _elf_section(path: str, wanted: str) -> bytes:
    """Bytes of one section of a 64-bit little-endian ELF file (our own build)."""
    import struct

    with open(path, "rb") as f:
        data = f.read()
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    def header(i):
        name, _, _, _, off, size = struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize)
        return name, off, size
    _, str_off, _ = header(shstrndx)
    for i in range(shnum):
        name, off, size = header(i)
        end = data.index(b"\0", str_off + name)
        if data[str_off + name:end].decode() == wanted:
            return data[off:off + size]
    raise KeyError(wanted)


def library_hash() -> str:
    """SHA-256 prefix of the device code in the built libdemo.so (its .hip_fatbin
    section): a traffic record taken with rocprofv3 applies only to the exact
    kernels it measured; host-side and comment-only changes keep the hash."""
    from communication_compressed_optimizer_elt_amd import binding

    return hashlib.sha256(_elf_section(binding.LIB_PATH, ".hip_fatbin")).hexdigest()[:16]


class Inputs:
    """The workload's seeded inputs, drawn on the device (the 4096-element
    tensor on the host: g, m ~ N(0, 1), theta ~ N(0, 0.02))."""

    def __init__(self, w: Workload, torch, synth):
        self.w = w
        self.torch = torch
        self.synth = synth
        if w.shard == "tensor4096":
            self.segs = None
            self.n = 4096
        else:
            self.segs = {"vit": synth.vit_b_set, "olmo2": synth.olmo2_half_shard,
                         "olmo2-full": synth.olmo2_full}[w.shard]()
            self.n = synth.shard_numel(self.segs)
            self.scales = synth.layer_scales(0, max(s.group for s in self.segs) + 1)
            self.g_std = 1e-2 if w.shard == "vit" else 1e-3

    def grad(self, seed, out=None):
        if self.segs is None:
            t = self.torch.from_numpy(self.synth.normal_np(self.n, 1.0, seed, self.synth.TAG_GRAD, 0)).cuda()
            return t if out is None else out.copy_(t)
        return self.synth.scaled_grad_torch(self.segs, self.scales, self.g_std, seed, 0, out=out)

    def momentum(self, seed):
        if self.segs is None:
            return self.torch.from_numpy(self.synth.normal_np(self.n, 1.0, seed, self.synth.TAG_MOM)).cuda()
        return self.torch.zeros(self.n, dtype=self.torch.float32, device="cuda")

    def theta(self):
        if self.segs is None:
            return self.torch.from_numpy(self.synth.normal_np(self.n, 0.02, 0, self.synth.TAG_THETA)).cuda()
        return self.synth.normal_torch(self.n, 0.02, 0, self.synth.TAG_THETA)


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
        print("bench.py measures the optimizer step on one GPU's shard only; run it with --gpus 1 "
              "(libdemo has no cross-GPU part: the exchange between replicas is simulated)", file=sys.stderr)
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

    w = WORKLOADS[args.workload]
    R, mode = w.R, w.mode
    scheme = {"dct": L.SCHEME_DCT, "random": L.SCHEME_RANDOM, "stride": L.SCHEME_STRIDE,
              "diloco": L.SCHEME_DILOCO}[w.scheme]
    fmt = {"ternary": L.VAL_TERNARY, "f16": L.VAL_F16, "f32": L.VAL_F32}[w.fmt]
    inp = Inputs(w, torch, synth)
    n = inp.n

    cfg = L.Config(scheme=scheme, k=w.k, value_fmt=fmt, beta=0.9, lr=1e-3, seed=0, step=0,
                   period=DILOCO_PERIOD, sign=w.sign)
    lay = L.demo_payload_layout(cfg, n)
    stride = lay["total_bytes"]
    payload_bytes = lay["idx_bytes"] + 2 * lay["plane_bytes"] + lay["val_bytes"]

    def sends(t):
        return scheme != L.SCHEME_DILOCO or t % DILOCO_PERIOD == DILOCO_PERIOD - 1

    adamw = L.AdamW() if w.adamw else None

    # ---- inputs, resident in HBM -------------------------------------------
    g = inp.grad(0)
    m = inp.momentum(0)
    v = torch.zeros(n, dtype=torch.float32, device=dev) if adamw else None
    theta = inp.theta()
    pay = torch.zeros(R * stride, dtype=torch.uint8, device=dev)
    # the other replicas' payloads: the step-0 encode of states drawn from their
    # own seeds (decode-only workloads: all R replicas, seeds 0..R-1).  DiLoCo
    # sends only on sync steps, so its peers encode at the first sync step.
    pg = torch.empty_like(g)
    peer_cfg = L.Config(**{**cfg.__dict__, "step": DILOCO_PERIOD - 1 if scheme == L.SCHEME_DILOCO else 0})
    for r in range(1 if mode == "step" else 0, R):
        inp.grad(r, out=pg)
        pm = inp.momentum(r)
        if adamw:
            L.demo_encode_adamw(peer_cfg, adamw, n, pg, pm, torch.zeros_like(pm), pay[r * stride:])
        else:
            L.demo_encode(peer_cfg, n, pg, pm, pay[r * stride:])
    torch.cuda.synchronize()
    del pg
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
    # per timed call: (kind, start event, end event, algorithmic bytes).  The
    # events are chained: one event between consecutive launches marks the end
    # of one call and the start of the next (a pair of events around every
    # call measured 10-20 us more per step), so a call's interval also holds
    # the dispatch gap after the previous kernel.
    calls = []
    boundary = [None]

    def timed(kind, nbytes, fn, record):
        if not record:
            fn()
            return
        if boundary[0] is None:
            boundary[0] = torch.cuda.Event(enable_timing=True)
            boundary[0].record(stream)
        fn()
        eb = torch.cuda.Event(enable_timing=True)
        eb.record(stream)
        calls.append((kind, boundary[0], eb, nbytes))
        boundary[0] = eb

    enc_state = (20 if adamw else 12) * n   # g, m (and v) read, m (and v) written
    dec_state = (12 if adamw else 8) * n    # theta read and written (and v read)

    def step(t, record):
        cfg.step = t
        # decode-only workloads decode the step-0 payloads (Random positions of step 0)
        dcfg = cfg if mode == "step" else L.Config(**{**cfg.__dict__, "step": 0})
        if mode == "step":
            enc_bytes = enc_state + (payload_bytes if sends(t) else 0)
            if adamw:
                timed("encode", enc_bytes, lambda: L.demo_encode_adamw(cfg, adamw, n, g, m, v, pay, None, stream),
                      record)
            else:
                timed("encode", enc_bytes, lambda: L.demo_encode(cfg, n, g, m, pay, None, stream), record)
        if sends(t):
            if adamw:
                timed("decode", dec_state + R * payload_bytes,
                      lambda: L.demo_decode_apply_adamw(dcfg, adamw, n, theta, v, pay, stride, R, stream), record)
            else:
                timed("decode", dec_state + R * payload_bytes,
                      lambda: L.demo_decode_apply(dcfg, n, theta, pay, stride, R, stream), record)

    for t in range(args.warmup):
        step(t, False)
    torch.cuda.synchronize()
    total_bytes = 0
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps

    kern = {}
    for kind in ("encode", "decode"):
        ms = np.array([ea.elapsed_time(eb) for kd, ea, eb, _ in calls if kd == kind])
        nb = [b for kd, _, _, b in calls if kd == kind]
        if len(ms) == 0:
            continue
        total_bytes += sum(nb)
        kern[kind] = {"calls": len(ms), "avg_ms": float(ms.mean()), "min_ms": float(ms.min()),
                      "bytes": float(np.mean(nb)), "gbps": float(sum(nb) / (ms.sum() / 1e3) / 1e9)}
    step_bytes = total_bytes / args.steps
    step_gbps = step_bytes / (step_ms / 1e3) / 1e9
    dom = max(kern, key=lambda kd: kern[kd]["avg_ms"] * kern[kd]["calls"])
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{dom}_{args.workload}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            rec = json.load(f)
        if rec.get("library_hash") == library_hash():
            traffic = rec.get("hbm_bytes_per_launch")

    if args.workload in LAUNCH_BOUND:
        roofline = None
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["gbps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": kern[dom]["gbps"] / HBM_PEAK_GBPS, "traffic": traffic}
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
        "config": {"workload": args.workload, "n_elems": n,
                   "optimizer": "decoupled-adamw" if adamw else "demo-sgd",
                   "scheme": w.scheme, "k": w.k, "value_fmt": w.fmt, "sign": cfg.sign,
                   "replicas": R, "chunk": 32, "mode": mode},
        "hbm_gbps": step_gbps,
        "pct_hbm_peak": 100.0 * step_gbps / HBM_PEAK_GBPS,
        "copy_gbps": copy_gbps,
        "kernels": kern,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if args.workload in LAUNCH_BOUND:
        out["launch_bound"] = (f"{n} parameters, {int(step_bytes)} algorithmic bytes per step: L2-resident, "
                               f"the time is launch and pipeline fill; not a roofline point")

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, cfg, adamw, n, g, m, v, theta, pay, stride, payload_bytes,
                                           enc_state, dec_state, args.cpu_seconds)

    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(w, cfg, adamw, n, g, m, v, theta, pay, stride, payload_bytes, enc_state, dec_state, budget_s):
    """The fp64 oracle as it stands, timed on this host's cores on the same
    input bytes as the GPU (gradients, state and the other replicas' payloads
    copied from the device).  A step is what the GPU step does: encode of the
    own replica and decode of all R payloads (decode-only workloads: the
    decode; DiLoCo: the average over one period of 16 steps).  The chunks
    timed are the whole shard when three steps fit the budget on all cores,
    else its first S chunks; one core runs a smaller sample for a third of the
    budget.  GB/s uses the GPU's accounting of algorithmic fp32 bytes for the
    chunks timed (the oracle itself moves fp64 state)."""
    import oracle

    from communication_compressed_optimizer_elt_amd import binding as L

    C = (n + 31) // 32
    p = oracle.Params(scheme=cfg.scheme, k=cfg.k, period=cfg.period, sign=cfg.sign, value_fmt=cfg.value_fmt,
                      beta=cfg.beta, lr=cfg.lr, seed=cfg.seed, step=0)
    ow = None if adamw is None else oracle.AdamW(beta2=adamw.beta2, eps=adamw.eps,
                                                 weight_decay=adamw.weight_decay)
    decode_only = w.mode == "decode"
    diloco = cfg.scheme == L.SCHEME_DILOCO
    period = cfg.period if diloco else 1
    payload_p = oracle.Params(**{**p.__dict__, "step": cfg.period - 1 if diloco else 0})

    def rows(t, S):
        return oracle.pad_chunks(t[: min(n, S * 32)].cpu().numpy(), min(n, S * 32))

    def setup(S):
        """host copies of the first S chunks: own state and the R payloads' slots"""
        ids = np.arange(S, dtype=np.uint64)
        nv = np.full(S, 32, np.int32)
        nv[-1] = min(n, S * 32) - (S - 1) * 32
        g_rows = rows(g, S)
        peers = []
        for r in range(1 if not decode_only else 0, w.R):
            gi, gv, _ = oracle.unpack(payload_p, n, pay[r * stride:(r + 1) * stride].cpu().numpy(),
                                      chunks=np.arange(S, dtype=np.uint64))
            peers.append((gi, gv))
        own = oracle.Shard(ids, nv, rows(m, S), rows(theta, S), None if v is None else rows(v, S))
        return own, g_rows, peers

    def run_steps(own, g_rows, peers, nsteps, t0=0):
        """nsteps oracle steps (DiLoCo: whole periods); returns seconds."""
        t_start = time.perf_counter()
        for t in range(t0, t0 + nsteps * period):
            # decode-only: the step-0 payloads, decoded with step-0 positions as on the GPU
            pt = oracle.Params(**{**p.__dict__, "step": 0 if decode_only else t})
            if decode_only:
                own.decode(pt, [x[0] for x in peers], [x[1] for x in peers], ow)
                continue
            idx, val, _, _ = own.encode(pt, g_rows, ow)
            if oracle.slots(pt):
                own.decode(pt, [idx] + [x[0] for x in peers], [val] + [x[1] for x in peers], ow)
        return time.perf_counter() - t_start

    # GPU accounting of one step's algorithmic bytes over the whole shard
    if decode_only:
        shard_bytes = dec_state + w.R * payload_bytes
    else:
        sync = enc_state + payload_bytes + dec_state + w.R * payload_bytes
        shard_bytes = (sync + (period - 1) * enc_state) / period

    def measure(budget, steps_wanted):
        # calibrate on a small sample, then size S to the budget
        S0 = min(C, 1 << 14)
        own, g_rows, peers = setup(S0)
        per_chunk = run_steps(own, g_rows, peers, 1) / S0
        S = int(min(C, max(S0, budget / max(steps_wanted * per_chunk, 1e-12))))
        own, g_rows, peers = setup(S)
        done, dt = 0, 0.0
        # at least steps_wanted steps and a quarter of the budget (small shards repeat)
        while (done < steps_wanted or dt < budget / 4) and done < 100000 and not (done and dt >= budget):
            dt += run_steps(own, g_rows, peers, 1, t0=done * period)
            done += 1
        params = min(n, S * 32)
        steps = done * period
        what = f"{done} period{'s' if done > 1 else ''} of {period} steps" if period > 1 else \
            f"{done} step{'s' if done > 1 else ''}"
        return {"value": params * steps / dt, "unit": "params/s",
                "gbps": shard_bytes * (params / n) * steps / dt / 1e9,
                "sample": (f"{'the whole shard' if S == C else f'the first {S} of {C} chunks'} "
                           f"({params} parameters), {what} in {dt:.2f} s, fp64 state")}

    cores = oracle.threads()
    allc = measure(budget_s, 3)
    oracle.set_threads(1)
    one = measure(budget_s / 3, 1)
    oracle.set_threads(cores)
    return {"value": allc["value"], "unit": "params/s", "gbps": allc["gbps"], "cores": cores, "kind": "oracle",
            "sample": allc["sample"], "single_core": {**one, "cores": 1},
            "host": {"cpu": _cpu_model(), "nproc": os.cpu_count()}}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())

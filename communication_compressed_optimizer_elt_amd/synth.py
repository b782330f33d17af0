"""Seeded synthetic workloads for the optimizer step (inputs only).

This module holds no arithmetic of the method.  It defines the parameter
layouts the benchmarks run on and draws the seeded inputs (gradients, initial
momentum, initial parameters, per-layer gradient scales).  The GPU tests, the
oracle tests and the benchmark take their inputs from here, so both sides of a
parity check see the same bytes.

Layouts (stand-ins for the models the method was evaluated on; no weights or
data are used):

* OLMo2-1B-shaped decoder: 16 layers, d_model 2048, MLP 8192, vocabulary
  100352 with a tied embedding.  Per layer: q, k, v, o (2048x2048), q-norm and
  k-norm (2048), post-attention norm (2048), gate and up (2048x8192), down
  (8192x2048), post-MLP norm (2048); then a final norm.  1,279,395,840
  parameters; one GPU's FSDP shard is the contiguous first half, 639,697,920.
* ViT-B-shaped set: 12 blocks of qkv 768x2304, proj 768x768, fc1 768x3072,
  fc2 3072x768 and four vectors of 768, 768, 2304, 3072 elements.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TAG_GRAD = 1
TAG_MOM = 2
TAG_THETA = 3
TAG_SCALE = 4

_MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_seed(seed: int, tag: int, step: int = 0) -> int:
    """A 63-bit seed for the input stream (seed, tag, step)."""
    h = _splitmix64(seed & _MASK64)
    h = _splitmix64(h ^ (tag & _MASK64))
    h = _splitmix64(h ^ (step & _MASK64))
    return h & ((1 << 63) - 1)


# --------------------------------------------------------------------------- #
# parameter layouts                                                           #
# --------------------------------------------------------------------------- #

@dataclass(frozen=True)
class Segment:
    name: str
    start: int   # element offset in the flat shard
    numel: int
    group: int   # gradient-scale group


def olmo2_1b_tensors():
    """(name, numel, group) of the whole OLMo2-1B-shaped model, in flat order."""
    d, f, vocab, layers = 2048, 8192, 100352, 16
    out = [("embed", vocab * d, 0)]
    for layer in range(layers):
        g = layer + 1
        p = f"layer{layer}."
        out += [(p + "q", d * d, g), (p + "k", d * d, g), (p + "v", d * d, g), (p + "o", d * d, g),
                (p + "q_norm", d, g), (p + "k_norm", d, g), (p + "post_attn_norm", d, g),
                (p + "gate", d * f, g), (p + "up", d * f, g), (p + "down", f * d, g),
                (p + "post_mlp_norm", d, g)]
    out.append(("final_norm", d, layers + 1))
    return out


def _segments(tensors, limit=None):
    segs, off = [], 0
    for name, n, g in tensors:
        if limit is not None and off >= limit:
            break
        take = n if limit is None else min(n, limit - off)
        segs.append(Segment(name, off, take, g))
        off += take
    return segs


def olmo2_half_shard():
    """Segments of the first half of the flattened OLMo2-1B-shaped parameters."""
    tensors = olmo2_1b_tensors()
    total = sum(n for _, n, _ in tensors)
    assert total == 1_279_395_840
    return _segments(tensors, total // 2)


def olmo2_full():
    """Segments of the whole flattened OLMo2-1B-shaped model: the shard when
    one data-parallel replica holds every parameter (shard group of size 1)."""
    segs = _segments(olmo2_1b_tensors())
    assert sum(s.numel for s in segs) == 1_279_395_840
    return segs


def vit_b_tensors():
    out = []
    for b in range(12):
        p = f"block{b}."
        out += [(p + "qkv", 768 * 2304, b), (p + "proj", 768 * 768, b), (p + "fc1", 768 * 3072, b),
                (p + "fc2", 3072 * 768, b), (p + "ln1", 768, b), (p + "ln2", 768, b),
                (p + "qkv_bias", 2304, b), (p + "fc1_bias", 3072, b)]
    return out


def vit_b_set():
    segs = _segments(vit_b_tensors())
    assert sum(s.numel for s in segs) == 85_017_600
    return segs


def shard_numel(segs) -> int:
    return sum(s.numel for s in segs)


def layer_scales(seed: int, n_groups: int) -> np.ndarray:
    """Per-group gradient scale ~ U(0.5, 2)."""
    rng = np.random.default_rng(stream_seed(seed, TAG_SCALE))
    return rng.uniform(0.5, 2.0, size=n_groups).astype(np.float32)


# --------------------------------------------------------------------------- #
# draws on the host (numpy) -- small cases                                    #
# --------------------------------------------------------------------------- #

def normal_np(n: int, std: float, seed: int, tag: int, step: int = 0) -> np.ndarray:
    rng = np.random.default_rng(stream_seed(seed, tag, step))
    return (rng.standard_normal(n, dtype=np.float32) * np.float32(std)).astype(np.float32)


# --------------------------------------------------------------------------- #
# draws on the device (torch generator) -- full-size shards                    #
# --------------------------------------------------------------------------- #

def normal_torch(n: int, std: float, seed: int, tag: int, step: int = 0, device="cuda", out=None):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(stream_seed(seed, tag, step))
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    out.normal_(0.0, std, generator=gen)
    return out


def scaled_grad_torch(segs, scales, std: float, seed: int, step: int, device="cuda", out=None):
    """g = s_group * N(0, std) over a list of segments, drawn on the device."""
    import torch

    n = shard_numel(segs)
    out = normal_torch(n, std, seed, TAG_GRAD, step, device=device, out=out)
    # consecutive segments of one group are scaled as one slice
    start, group = segs[0].start, segs[0].group
    for s in segs[1:] + [Segment("", n, 0, -1)]:
        if s.group != group:
            out[start:s.start].mul_(float(scales[group]))
            start, group = s.start, s.group
    torch.cuda.synchronize() if str(device).startswith("cuda") else None
    return out

"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the storage dtype; it holds none
of the attention arithmetic, so both the fp64 oracle and the HIP path can take their inputs
from it without sharing any of the method.

Recipe (the pages print no workload of their own, so these synthetic inputs are the
workload): numpy ``Generator(PCG64(seed))``, draws in the order Q, K, V, dO, each
``standard_normal`` in float32 and laid out ``[B, H, S, D]`` (K and V with the kv-head
count), dO multiplied by ``do_std`` before rounding, then rounded to the storage dtype
with round-to-nearest-even by torch on the CPU.  The same rounded bits feed both sides.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "HEADLINE", "get", "make_inputs", "make_inputs_device", "scaled"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp32" | "fp16" | "bf16"
    B: int
    H: int
    H_kv: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    seed: int
    do_std: float = 1.0
    window: int = 0     # sliding window in keys (0 = none)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def group(self) -> int:
        return self.H // self.H_kv

    def allowed_pairs(self) -> float:
        """(b, h, query, key) pairs counted as work: B*H*Sq*Sk, halved when causal (the fixed
        half of the metric, not the exact (S+1)/2S); with a window, the exact number of
        pairs it keeps (query i keeps keys j with i - W < j <= i, or |i - j| < W without
        the causal mask, below Sk)."""
        if self.window <= 0:
            p = float(self.B) * self.H * self.Sq * self.Sk
            return p / 2 if self.causal else p
        i = np.arange(self.Sq, dtype=np.int64)
        lo = np.maximum(i - self.window + 1, 0)
        hi = np.minimum(i if self.causal else i + self.window - 1, self.Sk - 1)
        return float(self.B) * self.H * float(np.maximum(hi - lo + 1, 0).sum())

    def bwd_flops(self) -> float:
        """Counted backward FLOPs: 10*D per allowed pair (the five contractions over the
        pairs the method must visit)."""
        return 10.0 * self.D * self.allowed_pairs()

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["scale"] = self.scale
        return d


WORKLOADS = {w.name: w for w in [
    Workload("fp32_h2_s128_d64", "fp32", 1, 2, 2, 128, 128, 64, False, seed=1),
    Workload("bf16_causal_h8_s1024_d64", "bf16", 2, 8, 8, 1024, 1024, 64, True, seed=2),
    Workload("bf16_causal_h16_s2048_d128", "bf16", 4, 16, 16, 2048, 2048, 128, True, seed=3,
             do_std=0.1),
    Workload("bf16_gqa4_causal_h32_s4096_d128", "bf16", 2, 32, 8, 4096, 4096, 128, True, seed=4),
    Workload("fp16_causal_h16_s16384_d128", "fp16", 1, 16, 16, 16384, 16384, 128, True, seed=51),
    Workload("fp16_gqa4_h16_sq512_sk8192_d128", "fp16", 4, 16, 4, 512, 8192, 128, False, seed=52),
    # the headline shape at the other head dims
    Workload("bf16_gqa4_causal_h32_s4096_d32", "bf16", 2, 32, 8, 4096, 4096, 32, True, seed=7),
    Workload("bf16_gqa4_causal_h32_s4096_d64", "bf16", 2, 32, 8, 4096, 4096, 64, True, seed=10),
    Workload("bf16_gqa4_causal_h32_s4096_d96", "bf16", 2, 32, 8, 4096, 4096, 96, True, seed=8),
    Workload("bf16_gqa4_causal_h32_s4096_d256", "bf16", 2, 32, 8, 4096, 4096, 256, True, seed=9),
    # sliding window of 4096 keys over 16384 positions (a long-context local-attention shape)
    Workload("bf16_gqa4_causal_win4096_h16_s16384_d128", "bf16", 1, 16, 4, 16384, 16384, 128, True,
             seed=6, window=4096),
]}

# The grouped-query causal bf16 case at S=4096, D=128 is the throughput headline.
HEADLINE = "bf16_gqa4_causal_h32_s4096_d128"


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller shapes for fast tests)."""
    return dataclasses.replace(w, **changes)


def _torch_dtype(dtype: str):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def make_inputs(w: Workload):
    """Return (q, k, v, do) as contiguous CPU torch tensors in ``w.dtype``."""
    import torch
    rng = np.random.Generator(np.random.PCG64(w.seed))
    qs = (w.B, w.H, w.Sq, w.D)
    ks = (w.B, w.H_kv, w.Sk, w.D)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    do = rng.standard_normal(qs, dtype=np.float32)
    if w.do_std != 1.0:
        do *= np.float32(w.do_std)
    dt = _torch_dtype(w.dtype)
    return tuple(torch.from_numpy(x).to(dt).contiguous() for x in (q, k, v, do))


def make_inputs_device(w: Workload, device):
    """Return (q, k, v, do) drawn directly on ``device``, for shapes too large to draw on the
    host (a tensor of 2**31 elements).  Recipe: torch's seeded device generator (Philox),
    seeded with ``w.seed``, draws Q, K, V, dO in that order as standard normals in float32;
    dO is multiplied by ``do_std``; each is rounded to ``w.dtype`` (round-to-nearest-even).
    The oracle's inputs are slices of these very tensors copied to the host, so both sides
    still see the same bits."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = _torch_dtype(w.dtype)

    def draw(shape, mul=1.0):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if mul != 1.0:
            x.mul_(mul)
        return x if dt == torch.float32 else x.to(dt)

    qs = (w.B, w.H, w.Sq, w.D)
    ks = (w.B, w.H_kv, w.Sk, w.D)
    q = draw(qs)
    k = draw(ks)
    v = draw(ks)
    do = draw(qs, w.do_std)
    return q, k, v, do

"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: it only draws Q, K, V and dO.  The
recipe is fixed so that the HIP path and the CPU oracle always see the same
values: a CPU ``torch.Generator`` seeded with ``seed``, float32 standard-normal
draws in the order Q, K, V, dO, an optional multiplier, then one cast to the
storage dtype (round-to-nearest-even).  The oracle upcasts those rounded
values to float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}


@dataclass(frozen=True)
class Shape:
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: str = "bf16"
    causal: bool = False
    mult: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]


def make_inputs(shape: Shape, seed: int, with_grad: bool = True):
    """CPU tensors (q, k, v, do) in ``shape.dtype``; ``do`` is None if not with_grad."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    qs = (shape.B, shape.Hq, shape.N, shape.D)
    ks = (shape.B, shape.Hkv, shape.N, shape.D)
    out = []
    for s in (qs, ks, ks, qs) if with_grad else (qs, ks, ks):
        t = torch.randn(s, generator=g, dtype=torch.float32)
        if shape.mult != 1.0:
            t.mul_(shape.mult)
        out.append(t.to(shape.torch_dtype))
    if not with_grad:
        out.append(None)
    return tuple(out)


# The workloads the library is exercised on (bf16/fp16, D=128 or 64, causal or
# not, MHA and 4:1 grouped-query heads, a ragged N=4000 tail).  Seeds follow
# 1000 * workload_id + variant.
WORKLOADS = {
    "tiny_fp16": [Shape(1, 2, 2, 256, 64, "fp16", c) for c in (False, True)],
    "fwd_bf16_n4096": [Shape(4, 16, 16, 4096, 128, "bf16", False)],
    "fwd_bf16_long": [Shape(1, 16, 16, n, 128, "bf16", False) for n in (8192, 16384)],
    "gqa_causal_fp16": [Shape(1, 16, 4, n, d, "fp16", True)
                        for n in (2048, 4096, 4000) for d in (64, 128)],
    "causal_long_bf16": [Shape(1, 8, 8, 16384, 128, "bf16", True, 0.5)],
    # one GPU's share of the long causal workload sharded by heads over 8 GPUs
    "shard_causal_bf16": [Shape(1, 1, 1, 16384, 128, "bf16", True, 0.5)],
}
WORKLOAD_IDS = {name: i + 1 for i, name in enumerate(WORKLOADS)}


def workload_seed(name: str, variant: int) -> int:
    return 1000 * WORKLOAD_IDS[name] + variant

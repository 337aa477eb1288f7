"""PyTorch operator registration for the fused attention kernels.

Registers ``torch.ops.fa_mi355x.fwd`` and ``torch.ops.fa_mi355x.bwd`` as custom operators
with fake (meta) implementations and an autograd formula. Models can then call
:func:`attention` as a differentiable op, and ``torch.compile`` traces it as one node
without a graph break. The fake implementations let shape propagation run without a GPU.

Every computation still goes through the C ABI (``fa_fwd`` / ``fa_bwd``). Like the rest of
the binding, this module only marshals arguments.

    o = attention(q, k, v, causal=True)            # q: (B, Hq, N, D), k/v: (B, Hkv, N, D)
    o.backward(do)                                  # dq, dk, dv through fa_bwd
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import fa_bwd as _fa_bwd
from . import fa_fwd as _fa_fwd

__all__ = ["attention"]


@torch.library.custom_op("fa_mi355x::fwd", mutates_args=())
def _fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool,
         softmax_scale: float) -> Tuple[torch.Tensor, torch.Tensor]:
    return _fa_fwd(q, k, v, causal=causal, softmax_scale=softmax_scale)


@_fwd.register_fake
def _fwd_fake(q, k, v, causal, softmax_scale):
    B, Hq, N, _ = q.shape
    return torch.empty_like(q), q.new_empty((B, Hq, N), dtype=torch.float32)


@torch.library.custom_op("fa_mi355x::bwd", mutates_args=())
def _bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, do: torch.Tensor,
         lse: torch.Tensor, causal: bool, softmax_scale: float) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    return _fa_bwd(q, k, v, o, do.contiguous(), lse, causal=causal, softmax_scale=softmax_scale)


@_bwd.register_fake
def _bwd_fake(q, k, v, o, do, lse, causal, softmax_scale):
    return torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)


def _setup_context(ctx, inputs, output):
    q, k, v, causal, softmax_scale = inputs
    o, lse = output
    ctx.save_for_backward(q, k, v, o, lse)
    ctx.causal = causal
    ctx.softmax_scale = softmax_scale


def _backward(ctx, do, dlse):
    # The LSE output is an auxiliary result for the backward; gradients through it are not
    # part of the operation (it is returned only so the backward can recompute P).
    q, k, v, o, lse = ctx.saved_tensors
    dq, dk, dv = _bwd(q, k, v, o, do, lse, ctx.causal, ctx.softmax_scale)
    return dq, dk, dv, None, None


torch.library.register_autograd("fa_mi355x::fwd", _backward, setup_context=_setup_context)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              softmax_scale: Optional[float] = None) -> torch.Tensor:
    """Exact softmax attention O = softmax(scale * Q K^T [causal mask]) V, differentiable.

    q: (B, Hq, N, D), k, v: (B, Hkv, N, D), contiguous, float16 or bfloat16 (float32 runs the
    fp32 verification path), on the GPU;
    D in {64, 128}; Hq a multiple of Hkv; scale defaults to 1/sqrt(D).
    """
    scale = 1.0 / math.sqrt(q.shape[-1]) if softmax_scale is None else float(softmax_scale)
    o, _ = _fwd(q, k, v, bool(causal), scale)
    return o

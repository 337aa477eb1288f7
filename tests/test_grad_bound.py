"""The derived gradient bound (parity_util.grad_error_bound) that the GPU tests apply where the
fixed relative tolerance does not (nearly one-hot rows), checked without a GPU: an emulation of
the backward's arithmetic (fp32 products and sums, 16-bit operands and outputs, D from a
16-bit O, a perturbed LSE) stays within it, and a planted mistake in that emulation does not."""
import numpy as np
import pytest
import torch

from exact_attention_fa_amd.inputs import Shape, make_inputs
from parity_util import assert_within_bound, attention_forward, grad_error_bound


def emulate_backward(q, k, v, do, o16, lse, scale, causal, dt, d_bias=0.0):
    """fp32 emulation of the kernels' backward arithmetic on one (b, h) grid (MHA)."""
    f = lambda x: torch.as_tensor(x, dtype=torch.float32)
    q, k, v, do, o16, lse = (f(x) for x in (q, k, v, do, o16, lse))
    N = q.shape[2]
    c2 = torch.tensor(scale * 1.4426950408889634, dtype=torch.float32)
    s = q @ k.transpose(-1, -2)
    l2 = lse * torch.tensor(1.4426950408889634, dtype=torch.float32)
    p = torch.exp2(s * c2 - l2[..., None])
    if causal:
        vis = torch.ones(N, N, dtype=torch.bool).tril()
        p = torch.where(vis, p, torch.zeros((), dtype=torch.float32))
    dp = do @ v.transpose(-1, -2)
    dd = (do * o16).sum(-1) * (1.0 + d_bias)
    ds = p * (dp - dd[..., None])
    ds16, p16 = ds.to(dt).float(), p.to(dt).float()
    dq = (scale * (ds16 @ k)).to(dt)
    dk = (scale * (ds16.transpose(-1, -2) @ q)).to(dt)
    dv = (p16.transpose(-1, -2) @ do).to(dt)
    return [x.double().numpy() for x in (dq, dk, dv)]


@pytest.mark.parametrize("dtype,causal,ramp", [("bf16", False, 40.0), ("fp16", False, 30.0), ("bf16", True, 6.0)])
def test_emulated_backward_within_bound(dtype, causal, ramp):
    shape = Shape(1, 2, 2, 160, 64, dtype, causal)
    q, k, v, do = make_inputs(shape, seed=11)
    n = shape.N
    k = (k.float() * (1.0 + (ramp - 1.0) * torch.arange(n, dtype=torch.float32) / (n - 1))[None, None, :, None]).to(k.dtype)
    f = lambda x: x.double().numpy()
    o_ref, lse_ref = attention_forward(f(q), f(k), f(v), shape.scale, causal)
    # a forward result as the GPU returns it: O rounded to the 16-bit type, LSE within 2e-4
    o16 = torch.as_tensor(o_ref).to(shape.torch_dtype).double().numpy()
    lse_g = lse_ref + np.random.default_rng(1).uniform(-2e-4, 2e-4, lse_ref.shape)
    g = emulate_backward(f(q), f(k), f(v), f(do), o16, lse_g, shape.scale, causal, shape.torch_dtype)
    bounds, refs = grad_error_bound(f(q), f(k), f(v), f(do), o16, lse_g, shape.scale, causal, dtype)
    for name, gg, r, bd in zip(("dq", "dk", "dv"), g, refs, bounds):
        assert_within_bound(gg, r, bd, name, "emulation")
    # not vacuous: a 2% error in D (a plausible slip in the preprocess) breaks it
    bad = emulate_backward(f(q), f(k), f(v), f(do), o16, lse_g, shape.scale, causal, shape.torch_dtype,
                           d_bias=0.02)
    with pytest.raises(AssertionError, match="derived bound"):
        for name, gg, r, bd in zip(("dq", "dk"), bad, refs, bounds):
            assert_within_bound(gg, r, bd, name, "planted")
